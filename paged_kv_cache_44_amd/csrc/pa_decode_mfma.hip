// pa_decode_mfma.hip — paged decode attention with the grouped-query tile on
// the gfx950 matrix cores.
//
// Same result as the VALU kernel ("Efficient Memory Management for Large
// Language Model Serving with PagedAttention", kernel paragraph: fetch each
// block through the block table, score the query group against it, combine
// with its values; identical to ordinary attention). With G query heads per
// KV head both products of a 16-token chunk are small dense contractions:
//   S[16 tokens][G heads] = K[16][D] . Q^T[D][G]   (v_mfma_f32_16x16x32)
//   O[G heads][D]        += P[G][16] . V[16][D]    (v_mfma_f32_16x16x16)
// G <= 16 fills the 16 columns of the tile.
//
// Layout facts used (CDNA 16x16xK MFMA, checked on gfx950): lane l holds
// A[row l%16][k in (l/16)*KL ..], B[k in (l/16)*KL ..][col l%16] and
// C[rows 4*(l/16) .. +3][col l%16].
//  * K: lane l loads token l%16, dims 32c + 8(l/16) .. +8 of step c: the A
//    operand of the score MFMA straight from memory (16 tokens x 64 B per
//    load instruction).
//  * The score tile comes out as lane l = (tokens 4(l/16)..+3, head l%16),
//    which is exactly the A-operand layout of the P.V MFMA: probabilities never
//    leave their lane.
//  * V: lane (g, n) loads the full 16-byte slice [VPL*n, +VPL) of tokens
//    4g..4g+3 (four whole 256-byte rows per load instruction); P.V MFMA m then
//    uses output column n for dim VPL*n + m and takes element m of each of the
//    four vectors (two byte permutes).
//  * Online softmax with a lazily moved reference maximum per head: the
//    reference only moves (exact cross-lane max, rescale) when a score exceeds
//    it by more than 2^TAU, so probabilities stay <= 2^8 and most chunks need
//    no cross-lane traffic at all.
//  * One wave owns one (sequence, KV head, partition); a workgroup holds the
//    4 KV heads of one (sequence, partition) and shares their block-table
//    slice through LDS. No other LDS traffic and no atomics.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int NWM = 4;          // waves (KV heads) per workgroup
constexpr int CH = 16;          // tokens per chunk
constexpr float TAU = 8.0f;     // lazy rescale threshold (log2 units)

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

// Operand type of a matrix product: bf16 or f16 (both exact for the inputs
// that reach them: 16-bit codes as stored, E4M3 codes widened).
enum class Op { BF16, F16 };

// fp32 pair -> packed 16-bit pair, round to nearest even
template <Op O>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (O == Op::BF16) {
    bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
  } else {
    half2_t v = __builtin_convertvector((f32x2_t){a, b}, half2_t);
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Packed 16-bit pair -> fp32 pair
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
  auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  if constexpr (O == Op::BF16) {
    // the values fit bf16 exactly: keep the upper halves of the fp32 words
    lo = __builtin_amdgcn_perm(f2u(a[1]), f2u(a[0]), 0x07060302u);
    hi = __builtin_amdgcn_perm(f2u(b[1]), f2u(b[0]), 0x07060302u);
  } else {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a[0], a[1]));  // exact
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(b[0], b[1]));
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
__device__ __forceinline__ void store_row(void* out, int64_t idx, const float* x, int n) {
  // n consecutive outputs starting at element idx
  if constexpr (QT == Ty::F32) {
    float* o = reinterpret_cast<float*>(out) + idx;
    for (int i = 0; i < n; ++i) o[i] = x[i];
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + idx;
    for (int i = 0; i < n; ++i) o[i] = (QT == Ty::BF16) ? f32_to_bf16_rne(x[i]) : f32_to_f16_rne(x[i]);
  }
}

__device__ __forceinline__ int ctx_bad(const DecodeParams& a, int ctx) {
  if (ctx < 0 || ctx > a.max_context_len) return 1;
  int64_t nb = ((int64_t)ctx + a.block_size - 1) >> a.log2_block_size;
  return nb > a.max_blocks_per_seq ? 1 : 0;
}

}  // namespace

template <Ty KV, Ty QT, int D, int G>
__global__ void __launch_bounds__(NWM * 64)
attend_mfma_kernel(const DecodeParams a) {
  static_assert(QT == Ty::BF16 || QT == Ty::F16, "16-bit queries");
  static_assert(G >= 1 && G <= 16, "group fits the 16-column tile");
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr Op OQK = (QT == Ty::F16) ? Op::F16 : Op::BF16;          // score operands
  constexpr Op OPV = (KV == Ty::BF16) ? Op::BF16 : Op::F16;         // P.V operands
  constexpr int EB = TyInfo<KV>::bytes;
  constexpr int KS = D / 32;              // score MFMA steps
  constexpr int VPL = D / 16;             // value elements per lane per token = P.V MFMAs
  constexpr int KDW = 8 * EB / 4;         // raw K dwords per lane per step
  constexpr int VDW = VPL * EB / 4;       // raw V dwords per lane per token

  __shared__ int s_tbl[PA_MAX_PART_BLOCKS];
  __shared__ int s_bad;

  // Grid (sequence, KV-head group, partition). Workgroups are dealt to the
  // 8 XCDs round-robin by linear id, i.e. by blockIdx.x here; rotating the
  // sequence by the partition index spreads the partitions of one sequence
  // over all XCDs instead of tying partition p to one XCD.
  const int part = blockIdx.z;
  const int seq = (int)((blockIdx.x + (unsigned)part) % (unsigned)a.num_seqs);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;                // row group
  const int n = lane & 15;                // column: head (scores) / dim slice (values)
  const int kvh = blockIdx.y * NWM + wave;
  const bool kv_ok = kvh < a.num_kv_heads;

  const int ctx = a.context_lens[seq];
  const int P = a.part_tokens;
  const int bad_ctx = ctx_bad(a, ctx);
  const int nparts = (bad_ctx || ctx == 0) ? 1 : (ctx + P - 1) / P;
  if (part >= nparts) return;
  const int hq0 = kvh * G;
  const int64_t out_row0 = ((int64_t)seq * a.num_q_heads + hq0) * D;
  if (bad_ctx || ctx == 0) {
    if (kv_ok) {
      const float fill = bad_ctx ? __builtin_nanf("") : 0.f;
      for (int i = lane; i < G * D; i += 64) store_row<QT>(a.out, out_row0 + i, &fill, 1);
    }
    return;
  }

  const int p0 = part * P;
  const int pend = min(p0 + P, ctx);
  const int lg = a.log2_block_size;
  const int lb0 = p0 >> lg;
  const int nlb = ((pend - 1) >> lg) - lb0 + 1;

  // q as the B operand of the score MFMA: lane l holds head l%16, dims
  // 32c + 8(l/16) .. +8 for step c (zero columns beyond the group)
  uint32_t qb[KS][4];
  {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.q);
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      if (kv_ok && n < G) {
        ld<4>(qw + ((out_row0 + (int64_t)n * D + 32 * c + 8 * g) >> 1), qb[c]);
      } else {
        qb[c][0] = qb[c][1] = qb[c][2] = qb[c][3] = 0u;
      }
    }
  }

  if (tid == 0) s_bad = 0;
  __syncthreads();
  const int32_t* trow = a.block_tables + (int64_t)seq * a.max_blocks_per_seq + lb0;
  for (int i = tid; i < nlb; i += NWM * 64) {
    int id = trow[i];
    if (id < 0 || id >= a.num_blocks) { s_bad = 1; id = 0; }
    s_tbl[i] = id;
  }
  __syncthreads();
  if (!kv_ok) return;
  const bool bad_tbl = s_bad != 0;

  const uint32_t* kpool = reinterpret_cast<const uint32_t*>(a.k_pool);
  const uint32_t* vpool = reinterpret_cast<const uint32_t*>(a.v_pool);
  const int64_t head_off = a.layer_offset + (int64_t)kvh * a.block_size * D;
  const int bmask = a.block_size - 1;
  const float qk_scale = a.qk_scale_log2;

  f32x4_t acc[VPL];
#pragma unroll
  for (int m = 0; m < VPL; ++m) acc[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();        // reference max of head n (log2 units)
  float l_sum = 0.f;                      // sum of this lane's probabilities (head n)

  const int ntok = pend - p0;
  const int nchunks = (ntok + CH - 1) / CH;

  auto elem_of = [&](int t) -> int64_t {  // element index of token t, dim 0
    t = min(t, pend - 1);
    return (int64_t)s_tbl[(t >> lg) - lb0] * a.block_stride + head_off + (int64_t)(t & bmask) * D;
  };
  auto load_chunk = [&](int k, uint32_t (&kr)[KS][KDW], uint32_t (&vr)[4][VDW]) {
    const int cb = p0 + k * CH;
    const int64_t ek = elem_of(cb + n) + 8 * g;
    int64_t ev[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ev[r] = elem_of(cb + 4 * g + r) + VPL * n;
#pragma unroll
    for (int c = 0; c < KS; ++c) ld<KDW>(kpool + (ek + 32 * c) * EB / 4, kr[c]);
#pragma unroll
    for (int r = 0; r < 4; ++r) ld<VDW>(vpool + ev[r] * EB / 4, vr[r]);
  };

  auto process_chunk = [&](int k, uint32_t (&kr)[KS][KDW], uint32_t (&vr)[4][VDW]) {
    const int cb = p0 + k * CH;
    // ---- scores: S[token 4g + r][head n] --------------------------------
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      uint32_t ka[4];
      if constexpr (KV == Ty::FP8) {
        fp8x4_to<OQK>(kr[c][0], ka[0], ka[1]);
        fp8x4_to<OQK>(kr[c][1], ka[2], ka[3]);
      } else {
        ka[0] = kr[c][0]; ka[1] = kr[c][1]; ka[2] = kr[c][2]; ka[3] = kr[c][3];
      }
      s = mfma_k32<OQK>(ka, qb[c], s);
    }
    const bool tail = cb + CH > pend;
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = (n < G) && (cb + 4 * g + r < pend);
      z[r] = valid ? s[r] * qk_scale : -__builtin_inff();
    }
    const float lmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    if (__any(lmax > m_ref + TAU)) {
      // move the reference to the exact running max of each head
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
    for (int r = 0; r < 4; ++r) p[r] = (z[r] == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(z[r] - m_ref);
    const uint32_t pa0 = pack2<OPV>(p[0], p[1]);
    const uint32_t pa1 = pack2<OPV>(p[2], p[3]);
    {
      // the normaliser sums exactly the rounded weights the matrix core uses
      float q0, q1, q2, q3;
      unpack2<OPV>(pa0, q0, q1);
      unpack2<OPV>(pa1, q2, q3);
      l_sum += (q0 + q1) + (q2 + q3);
    }
    // ---- values: zero tokens past the context, widen FP8 -------------------
    if (tail) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (cb + 4 * g + r >= pend)
#pragma unroll
          for (int w = 0; w < VDW; ++w) vr[r][w] = 0u;
    }
    uint32_t vw[4][VPL / 2];                   // value words of operand type OPV
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (KV == Ty::FP8) {
#pragma unroll
        for (int w = 0; w < VDW; ++w) fp8x4_to<OPV>(vr[r][w], vw[r][2 * w], vw[r][2 * w + 1]);
      } else {
#pragma unroll
        for (int w = 0; w < VPL / 2; ++w) vw[r][w] = vr[r][w];
      }
    }
    // ---- P.V: MFMA m covers dims VPL*n + m -------------------------------
#pragma unroll
    for (int m = 0; m < VPL; ++m) {
      const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t b0 = __builtin_amdgcn_perm(vw[1][m >> 1], vw[0][m >> 1], sel);
      const uint32_t b1 = __builtin_amdgcn_perm(vw[3][m >> 1], vw[2][m >> 1], sel);
      acc[m] = mfma_k16<OPV>(pa0, pa1, b0, b1, acc[m]);
    }
  };

  if (!bad_tbl) {
    uint32_t ka[KS][KDW], va[4][VDW], kb[KS][KDW], vb[4][VDW];
    const int last = nchunks - 1;
    int k = 0;
    int left = nchunks;
    load_chunk(0, ka, va);
    for (; left >= 2; left -= 2) {
      load_chunk(min(k + 1, last), kb, vb);
      process_chunk(k, ka, va);
      ++k;
      load_chunk(min(k + 1, last), ka, va);
      process_chunk(k, kb, vb);
      ++k;
    }
    if (left == 1) process_chunk(k, ka, va);
  }

  // ---- finish: per-head sums over the 4 row groups, then write -------------
  float lt = l_sum + __shfl_xor(l_sum, 16);
  lt += __shfl_xor(lt, 32);
  const bool single = nparts == 1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;                        // accumulator row = head
    const float lh = __shfl(lt, h);
    const float mh = __shfl(m_ref, h);
    if (h < G) {
      float o[VPL];
#pragma unroll
      for (int m = 0; m < VPL; ++m) o[m] = acc[m][r];
      if (bad_tbl) {
#pragma unroll
        for (int m = 0; m < VPL; ++m) o[m] = __builtin_nanf("");
      }
      if (single) {
        const float norm = a.v_scale / lh;
#pragma unroll
        for (int m = 0; m < VPL; ++m) o[m] *= norm;
        store_row<QT>(a.out, out_row0 + (int64_t)h * D + VPL * n, o, VPL);
      } else {
        const int64_t pr = ((int64_t)seq * a.num_q_heads + hq0 + h) * a.num_parts + part;
        float* wo = a.ws_o + pr * D + VPL * n;
#pragma unroll
        for (int m = 0; m < VPL; ++m) wo[m] = o[m];
        if (n == 0) {
          a.ws_m[pr] = bad_tbl ? 0.f : mh;
          a.ws_l[pr] = bad_tbl ? __builtin_nanf("") : lh;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <Ty KV, Ty QT, int D, int G>
static hipError_t launch_t(const DecodeParams& a, hipStream_t st) {
  dim3 grid(a.num_seqs, (a.num_kv_heads + NWM - 1) / NWM, a.num_parts);
  hipLaunchKernelGGL((attend_mfma_kernel<KV, QT, D, G>), grid, dim3(NWM * 64), 0, st, a);
  return hipGetLastError();
}

template <Ty KV, Ty QT, int D>
static hipError_t launch_g(const DecodeParams& a, int g, hipStream_t st) {
  switch (g) {
    case 1: return launch_t<KV, QT, D, 1>(a, st);
    case 2: return launch_t<KV, QT, D, 2>(a, st);
    case 4: return launch_t<KV, QT, D, 4>(a, st);
    case 8: return launch_t<KV, QT, D, 8>(a, st);
    case 16: return launch_t<KV, QT, D, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <Ty KV, Ty QT>
static hipError_t launch_d(const DecodeParams& a, int g, hipStream_t st) {
  if (a.head_dim == 64) return launch_g<KV, QT, 64>(a, g, st);
  if (a.head_dim == 128) return launch_g<KV, QT, 128>(a, g, st);
  return hipErrorInvalidValue;
}

bool mfma_supported(int kv_ty, int q_ty, int head_dim, int g) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  const bool types = (kv == Ty::BF16 && q == Ty::BF16) || (kv == Ty::F16 && q == Ty::F16) ||
                     (kv == Ty::FP8 && (q == Ty::BF16 || q == Ty::F16));
  return types && (head_dim == 64 || head_dim == 128) &&
         (g == 1 || g == 2 || g == 4 || g == 8 || g == 16);
}

hipError_t launch_attend_mfma(const DecodeParams& a, int kv_ty, int q_ty, int g, hipStream_t st) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  if (kv == Ty::BF16 && q == Ty::BF16) return launch_d<Ty::BF16, Ty::BF16>(a, g, st);
  if (kv == Ty::F16 && q == Ty::F16) return launch_d<Ty::F16, Ty::F16>(a, g, st);
  if (kv == Ty::FP8 && q == Ty::BF16) return launch_d<Ty::FP8, Ty::BF16>(a, g, st);
  if (kv == Ty::FP8 && q == Ty::F16) return launch_d<Ty::FP8, Ty::F16>(a, g, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
