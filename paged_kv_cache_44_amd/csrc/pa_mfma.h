// pa_mfma.h — pieces the matrix-core attention kernels share: operand
// packing, the 16x16 MFMA calls, output stores, and the whole-line K load
// layout with its lane exchange.
//
// CDNA 16x16xK MFMA layout (checked on gfx950): lane l holds A[row l%16][k in
// (l/16)*KL ..], B[k in (l/16)*KL ..][col l%16] and C[rows 4*(l/16) .. +3][col
// l%16]. The score product K[16 tokens][D] . X^T[D][16 columns] therefore
// wants lane l to hold token l%16 and 8 dims per step.
#pragma once

#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int DW>
__device__ __forceinline__ void ld(const uint32_t* __restrict__ p, uint32_t* w) {
  if constexpr (DW == 1) {
    w[0] = *p;
  } else if constexpr (DW == 2) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else {
    static_assert(DW == 4, "load width");
    uint4 x = *reinterpret_cast<const uint4*>(p);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  }
}

// The same loads with the non-temporal hint, for data a launch reads exactly
// once (a decode's K/V stream): L2 and the Infinity Cache keep such lines at
// the front of their eviction order instead of displacing the lines that are
// reused. On the GQA bf16 decode (256 sequences, ~1 GB of K/V per call) this
// took the attention kernel from 5.1 to 5.7 TB/s.
template <int DW>
__device__ __forceinline__ void ld_stream(const uint32_t* __restrict__ p, uint32_t* w) {
  if constexpr (DW == 1) {
    w[0] = __builtin_nontemporal_load(p);
  } else if constexpr (DW == 2) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    w[0] = x.x; w[1] = x.y;
  } else {
    static_assert(DW == 4, "load width");
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  }
}

// Operand type of a matrix product: bf16 or f16 (exact for the inputs that
// reach them: 16-bit codes as stored, E4M3 codes widened).
enum class Op { BF16, F16 };

template <Op O>
__device__ __forceinline__ uint32_t pack2(float a, float b) {   // RNE
  if constexpr (O == Op::BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, half2_t));
  }
}

template <Op O>
__device__ __forceinline__ void unpack2(uint32_t w, float& a, float& b) {
  if constexpr (O == Op::BF16) {
    a = u2f(w << 16);
    b = u2f(w & 0xffff0000u);
  } else {
    half2_t h = __builtin_bit_cast(half2_t, w);
    a = (float)h[0];
    b = (float)h[1];
  }
}

// 4 E4M3 codes -> two packed 16-bit pairs of operand type O (exact)
template <Op O>
__device__ __forceinline__ void fp8x4_to(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (O == Op::BF16) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  } else {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
}

template <Op O>
__device__ __forceinline__ f32x4_t mfma_k32(const uint32_t* a, const uint32_t* b, f32x4_t c) {
  u32x4_t av = {a[0], a[1], a[2], a[3]}, bv = {b[0], b[1], b[2], b[3]};
  if constexpr (O == Op::BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                    __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av),
                                                   __builtin_bit_cast(f16x8_t, bv), c, 0, 0, 0);
}

template <Op O>
__device__ __forceinline__ f32x4_t mfma_k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                            f32x4_t c) {
  u32x2_t av = {a0, a1}, bv = {b0, b1};
  if constexpr (O == Op::BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, av),
                                                      __builtin_bit_cast(bf16x4_t, bv), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, av),
                                                  __builtin_bit_cast(f16x4_t, bv), c, 0, 0, 0);
}

template <Ty QT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (QT == Ty::F32) {
    reinterpret_cast<float*>(out)[idx] = x;
  } else if constexpr (QT == Ty::BF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(x);
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16_rne(x);
  }
}

// First of the 8 dims that lane group a (= lane / 16) holds in MFMA step k
// of the score product, for K rows of D * EB bytes: whole-line loads put
// dims 16a + {0, 8, 64, 72} (16-bit, D = 128), 16a + {0, 8} (16-bit, D = 64)
// and 32a + 8k (FP8, D = 128) there; otherwise the operand layout puts dims
// 32k + 8a.
template <int D, int EB>
__device__ __forceinline__ int kdim_t(int k, int a) {
  if constexpr (D * EB == 256) return 16 * a + (k & 1) * 8 + (k >> 1) * 64;
  else if constexpr (D * EB == 128 && EB == 2) return 16 * a + 8 * k;
  else if constexpr (D * EB == 128) return 32 * a + 8 * k;
  else return 32 * k + 8 * a;
}

// K rows of D * EB bytes are read in whole 128-byte lines when a row has at
// least one: load u, lane l takes token row (l&7) + 8(u&1), 16-byte column
// (l>>3) + 8(u>>1) (8 rows per load); k_operand then exchanges halves with
// lane l^8 (DPP row rotation by 8) so that lane l holds token l%16. Reading
// the operand layout directly (64 bytes of 16 rows per load) streams
// markedly slower. Rows shorter than a line (FP8, D = 64) are loaded in the
// operand layout: lane l token l%16, dims 32k + 8(l/16) of step k.
template <int D, int EB>
struct KLayout {
  static constexpr int KS = D / 32;                        // score MFMA steps
  static constexpr int KDW = 8 * EB / 4;                   // raw dwords per lane per step
  static constexpr bool FULL = D * EB >= 128;
  static constexpr int KR = FULL ? D * EB / 64 : KS;       // K loads per 16 tokens
  static constexpr int KW = FULL ? 4 : KDW;                // dwords per lane per K load
};

// Element offset (from the token row's start of dim 0) and token row (0..15)
// of lane `lane`'s K load u.
template <int D, int EB>
__device__ __forceinline__ int k_load_row(int u, int lane) {
  if constexpr (KLayout<D, EB>::FULL) return (lane & 7) + 8 * (u & 1);
  else return lane & 15;
}
template <int D, int EB>
__device__ __forceinline__ int k_load_col(int u, int lane) {
  if constexpr (KLayout<D, EB>::FULL) return ((lane >> 3) + 8 * (u >> 1)) * (16 / EB);
  else return 32 * u + 8 * (lane >> 4);
}

// Raw K of MFMA step k for lane `lane`'s token (l % 16), from its loads.
template <int D, int EB>
__device__ __forceinline__ void k_operand(const uint32_t (&kr)[KLayout<D, EB>::KR][KLayout<D, EB>::KW],
                                          uint32_t (&kraw)[KLayout<D, EB>::KS][KLayout<D, EB>::KDW],
                                          int lane) {
  using L = KLayout<D, EB>;
  if constexpr (L::FULL) {
    const bool hs = (lane >> 3) & 1;                // lane l holds token l%16 half the time
    if constexpr (EB == 2) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
#pragma unroll
        for (int v = 0; v < L::KR / 2; ++v) {
          // loads 2v, 2v+1 are token rows p and p+8 of the same columns
          const uint32_t mine0 = kr[2 * v][x], mine1 = kr[2 * v + 1][x];
          const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(hs ? mine0 : mine1),
                                                                     0x128, 0xF, 0xF, false);
          kraw[2 * v][x] = hs ? got : mine0;
          kraw[2 * v + 1][x] = hs ? mine1 : got;
        }
      }
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t own = hs ? kr[1][x] : kr[0][x];
        const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(hs ? kr[0][x] : kr[1][x]),
                                                                   0x128, 0xF, 0xF, false);
        const uint32_t lo = hs ? got : own, hi = hs ? own : got;
        kraw[x >> 1][x & 1] = lo;
        kraw[2 + (x >> 1)][x & 1] = hi;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < L::KS; ++k)
#pragma unroll
      for (int x = 0; x < L::KDW; ++x) kraw[k][x] = kr[k][x];
  }
}

// Lazy rescale threshold of the online softmax (log2 units): the reference
// max moves only when a score exceeds it by more than 2^TAU, so weights stay
// <= 2^TAU and most chunks need no cross-lane traffic.
constexpr float SM_TAU = 8.0f;

// Operand types of the two products: scores in the query type, P.V in the
// pool's 16-bit type (FP8 values are widened exactly to f16).
template <Ty KV, Ty QT>
struct ChunkOps {
  static constexpr Op QK = (QT == Ty::F16) ? Op::F16 : Op::BF16;
  static constexpr Op PV = (KV == Ty::BF16) ? Op::BF16 : Op::F16;
};

// Score tile of a 16-token chunk against 16 columns: S[16 tokens][16 cols] =
// K[16][D] . X^T[D][16] (D/32 steps of v_mfma_f32_16x16x32). kraw is the
// lane's raw K operand (k_operand); xb(k) gives the lane's B operand of step
// k (its column's dims kdim_t(k, lane / 16) .. +8) as 16 bytes. Lane l gets
// tokens 4(l/16) .. +3 of column l%16.
template <Ty KV, Ty QT, int D, class XB>
__device__ __forceinline__ f32x4_t chunk_scores_raw(
    const uint32_t (&kraw)[KLayout<D, TyInfo<KV>::bytes>::KS][KLayout<D, TyInfo<KV>::bytes>::KDW],
    XB xb) {
  using L = KLayout<D, TyInfo<KV>::bytes>;
  constexpr Op OQK = ChunkOps<KV, QT>::QK;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < L::KS; ++k) {
    uint32_t ka[4];
    if constexpr (KV == Ty::FP8) {
      fp8x4_to<OQK>(kraw[k][0], ka[0], ka[1]);
      fp8x4_to<OQK>(kraw[k][1], ka[2], ka[3]);
    } else {
      ka[0] = kraw[k][0]; ka[1] = kraw[k][1]; ka[2] = kraw[k][2]; ka[3] = kraw[k][3];
    }
    const uint4 x4 = xb(k);
    const uint32_t xv[4] = {x4.x, x4.y, x4.z, x4.w};
    s = mfma_k32<OQK>(ka, xv, s);
  }
  return s;
}

// The same from the lane's K loads (rebuilds the operand first).
template <Ty KV, Ty QT, int D, class XB>
__device__ __forceinline__ f32x4_t chunk_scores(
    const uint32_t (&kr)[KLayout<D, TyInfo<KV>::bytes>::KR][KLayout<D, TyInfo<KV>::bytes>::KW],
    XB xb, int lane) {
  constexpr int EB = TyInfo<KV>::bytes;
  using L = KLayout<D, EB>;
  uint32_t kraw[L::KS][L::KDW];
  k_operand<D, EB>(kr, kraw, lane);
  return chunk_scores_raw<KV, QT, D>(kraw, xb);
}

// Value operands of a chunk for P.V: the lane's value loads (slice
// [VPL*(l%16), +VPL) of tokens 4(l/16)+r) as packed 16-bit pairs, element m
// of the four token vectors gathered with byte permutes later; live[r] false
// for value rows that must read as zero (past the context: they may hold NaN
// codes). FP8 codes are widened exactly to f16.
template <Ty KV, Ty QT, int D>
__device__ __forceinline__ void v_operand(const uint32_t (&vr)[4][D / 16 * TyInfo<KV>::bytes / 4],
                                          const bool (&live)[4], uint32_t (&vw)[4][D / 32]) {
  constexpr int VPL = D / 16;
  constexpr int VDW = VPL * TyInfo<KV>::bytes / 4;
  constexpr Op OPV = ChunkOps<KV, QT>::PV;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (KV == Ty::FP8) {
#pragma unroll
      for (int x = 0; x < VDW; ++x) fp8x4_to<OPV>(live[r] ? vr[r][x] : 0u, vw[r][2 * x], vw[r][2 * x + 1]);
    } else {
#pragma unroll
      for (int x = 0; x < VPL / 2; ++x) vw[r][x] = live[r] ? vr[r][x] : 0u;
    }
  }
}

// One chunk of online softmax and P.V for the lane's column (l % 16):
// z[r] = scaled score of token 4(l/16)+r (log2 units; -inf where masked), vw
// the chunk's value operands (v_operand). The score tile is exactly the
// A-operand layout of P[16 cols][16 tokens] . V[16 tokens][D]
// (v_mfma_f32_16x16x16), so the probabilities never leave their lane; acc[m]
// holds output rows 4(l/16)+r (columns), dim VPL*(l%16) + m. The row sum adds
// exactly the rounded 16-bit weights the matrix core multiplies.
template <Ty KV, Ty QT, int D>
__device__ __forceinline__ void softmax_pv(const float (&z)[4], const uint32_t (&vw)[4][D / 32],
                                           f32x4_t (&acc)[D / 16], float& m_ref, float& l_sum,
                                           int lane) {
  constexpr int VPL = D / 16;
  constexpr Op OPV = ChunkOps<KV, QT>::PV;
  const int g = lane >> 4;
  const float lmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  if (__any(lmax > m_ref + SM_TAU)) {
    float hm = fmaxf(lmax, __shfl_xor(lmax, 16));
    hm = fmaxf(hm, __shfl_xor(hm, 32));
    const float mn = fmaxf(m_ref, hm);
    const float al = (mn == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_ref - mn);
    m_ref = mn;
    l_sum *= al;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(al, 4 * g + r);      // factor of accumulator row 4g + r
#pragma unroll
      for (int m = 0; m < VPL; ++m) acc[m][r] *= ar;
    }
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    p[r] = (z[r] == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(z[r] - m_ref);
  const uint32_t pa0 = pack2<OPV>(p[0], p[1]);
  const uint32_t pa1 = pack2<OPV>(p[2], p[3]);
  {
    float q0, q1, q2, q3;
    unpack2<OPV>(pa0, q0, q1);
    unpack2<OPV>(pa1, q2, q3);
    l_sum += (q0 + q1) + (q2 + q3);
  }
#pragma unroll
  for (int m = 0; m < VPL; ++m) {
    const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t b0 = __builtin_amdgcn_perm(vw[1][m >> 1], vw[0][m >> 1], sel);
    const uint32_t b1 = __builtin_amdgcn_perm(vw[3][m >> 1], vw[2][m >> 1], sel);
    acc[m] = mfma_k16<OPV>(pa0, pa1, b0, b1, acc[m]);
  }
}

// The B operands of the P.V products of one chunk (element m of the four
// token vectors, two byte permutes per m), for kernels that apply the same
// chunk to several column tiles.
template <int D>
__device__ __forceinline__ void pv_operands(const uint32_t (&vw)[4][D / 32], uint32_t (&b)[D / 16][2]) {
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
    b[m][0] = __builtin_amdgcn_perm(vw[1][m >> 1], vw[0][m >> 1], sel);
    b[m][1] = __builtin_amdgcn_perm(vw[3][m >> 1], vw[2][m >> 1], sel);
  }
}

// The same B operands straight from FP8 value codes (f16 operands, exact):
// the raw codes of token rows 0 and 1 (and 2 and 3) are byte-interleaved,
// one permute per two dims, and each interleaved dword converts to two
// operand pairs, so a dim costs three instructions instead of four. vr is
// the lane's value loads (slice [VPL*(l%16), +VPL) of tokens 4(l/16)+r);
// live[r] false for rows that must read as zero (code 0 is +0).
template <int D>
__device__ __forceinline__ void pv_operands_fp8(const uint32_t (&vr)[4][D / 64], const bool (&live)[4],
                                                uint32_t (&b)[D / 16][2]) {
#pragma unroll
  for (int x = 0; x < D / 64; ++x) {
    uint32_t a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = live[r] ? vr[r][x] : 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // bytes {row 2p dim 2h, row 2p+1 dim 2h, row 2p dim 2h+1, row 2p+1 dim 2h+1}
      const uint32_t sel = h ? 0x07030602u : 0x05010400u;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t t = __builtin_amdgcn_perm(a[2 * p + 1], a[2 * p], sel);
        b[4 * x + 2 * h][p] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 1.0f, false));
        b[4 * x + 2 * h + 1][p] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 1.0f, true));
      }
    }
  }
}

// softmax_pv with the B operands already built (pv_operands).
template <Ty KV, Ty QT, int D>
__device__ __forceinline__ void softmax_pv_b(const float (&z)[4], const uint32_t (&b)[D / 16][2],
                                             f32x4_t (&acc)[D / 16], float& m_ref, float& l_sum,
                                             int lane) {
  constexpr int VPL = D / 16;
  constexpr Op OPV = ChunkOps<KV, QT>::PV;
  const int g = lane >> 4;
  const float lmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  if (__any(lmax > m_ref + SM_TAU)) {
    float hm = fmaxf(lmax, __shfl_xor(lmax, 16));
    hm = fmaxf(hm, __shfl_xor(hm, 32));
    const float mn = fmaxf(m_ref, hm);
    const float al = (mn == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m_ref - mn);
    m_ref = mn;
    l_sum *= al;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(al, 4 * g + r);
#pragma unroll
      for (int m = 0; m < VPL; ++m) acc[m][r] *= ar;
    }
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    p[r] = (z[r] == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(z[r] - m_ref);
  const uint32_t pa0 = pack2<OPV>(p[0], p[1]);
  const uint32_t pa1 = pack2<OPV>(p[2], p[3]);
  {
    float q0, q1, q2, q3;
    unpack2<OPV>(pa0, q0, q1);
    unpack2<OPV>(pa1, q2, q3);
    l_sum += (q0 + q1) + (q2 + q3);
  }
#pragma unroll
  for (int m = 0; m < VPL; ++m) acc[m] = mfma_k16<OPV>(pa0, pa1, b[m][0], b[m][1], acc[m]);
}

// v_operand followed by softmax_pv (one column tile per chunk).
template <Ty KV, Ty QT, int D>
__device__ __forceinline__ void chunk_softmax_pv(const float (&z)[4],
                                                 const uint32_t (&vr)[4][D / 16 * TyInfo<KV>::bytes / 4],
                                                 const bool (&live)[4], f32x4_t (&acc)[D / 16],
                                                 float& m_ref, float& l_sum, int lane) {
  if constexpr (KV == Ty::FP8) {
    static_assert(ChunkOps<KV, QT>::PV == Op::F16, "FP8 values are multiplied as f16");
    uint32_t b[D / 16][2];
    pv_operands_fp8<D>(vr, live, b);
    softmax_pv_b<KV, QT, D>(z, b, acc, m_ref, l_sum, lane);
  } else {
    uint32_t vw[4][D / 32];
    v_operand<KV, QT, D>(vr, live, vw);
    softmax_pv<KV, QT, D>(z, vw, acc, m_ref, l_sum, lane);
  }
}

}  // namespace pa
