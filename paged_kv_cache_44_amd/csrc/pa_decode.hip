// pa_decode.hip — paged decode attention for gfx950.
//
// What is computed ("Efficient Memory Management for Large Language Model
// Serving with PagedAttention", kernel paragraph): for every sequence s and
// query head h, softmax(scale * q K^T) V over the sequence's context tokens,
// where token t is fetched from physical block block_tables[s][t / B], slot
// t % B. The result equals ordinary attention over the same tokens; only the
// addressing differs ("Continuous Batching and PagedAttention", section "The
// block table is a page table").
//
// Design (one GPU, HBM-bound):
//  * One workgroup per (context partition, KV head, sequence); it reads every
//    key/value byte of its partition exactly once and serves all G query
//    heads that share the KV head (grouped-query attention), so HBM traffic
//    does not grow with G.
//  * 4 waves per workgroup. A wave walks 16-token chunks of the partition. A
//    16-lane row of the wave owns one token per load and 1/16 of its head
//    vector (16 B per lane for bf16/fp16 at D = 128), so one wave load covers
//    4 consecutive tokens = 1 KiB of contiguous memory.
//  * q.k partial sums are completed by a reduce-scatter over the 16 lanes of
//    a row using DPP lane exchanges (no LDS traffic); each lane then owns one
//    (token, head) score, exponentiates it, and the probabilities are shared
//    inside the row through a few LDS words for the P.V accumulation.
//  * Each 16-lane row keeps its own online-softmax state (running max, sum,
//    accumulators); rows and waves are merged once at the end of the
//    partition. Partitions of one sequence are merged by a second small
//    kernel, in partition order, with no atomics: results do not depend on
//    where blocks sit in the pool.
//  * Probabilities are computed in the exp2 domain with fp32 accumulation.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int ROWS = 4;       // 16-lane rows per wave
constexpr int LPT = 16;       // lanes per token row
constexpr int NL = 4;         // loads per 16-token chunk
constexpr int CHUNK = NL * ROWS;

template <int DW>
__device__ __forceinline__ void gload(const uint32_t* __restrict__ p, uint32_t* w) {
  if constexpr (DW == 1) {
    w[0] = *p;
  } else if constexpr (DW == 2) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (DW == 4) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else {
    static_assert(DW % 4 == 0, "unsupported load width");
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
      uint4 x = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  }
}

// How a (KV storage, query) type pair forms q.k.
enum class DotMode { BF16x2, F16x2, F32 };
template <Ty KV, Ty QT> struct DotSel;
template <> struct DotSel<Ty::BF16, Ty::BF16> { static constexpr DotMode m = DotMode::BF16x2; };
template <> struct DotSel<Ty::F16, Ty::F16>   { static constexpr DotMode m = DotMode::F16x2; };
template <> struct DotSel<Ty::FP8, Ty::BF16>  { static constexpr DotMode m = DotMode::BF16x2; };
template <> struct DotSel<Ty::FP8, Ty::F16>   { static constexpr DotMode m = DotMode::F16x2; };
template <> struct DotSel<Ty::F32, Ty::F32>   { static constexpr DotMode m = DotMode::F32; };
template <> struct DotSel<Ty::FP8, Ty::F32>   { static constexpr DotMode m = DotMode::F32; };

template <Ty KV, Ty QT, int VEC>
struct QK {
  static constexpr DotMode mode = DotSel<KV, QT>::m;
  static constexpr int QW = (mode == DotMode::F32) ? VEC : VEC / 2;   // registers per head
  static constexpr int KDW = VEC * TyInfo<KV>::bytes / 4;             // raw dwords per token

  // q[h][c*VEC .. +VEC] -> registers
  __device__ static __forceinline__ void load_q(const void* qrow, int c, uint32_t* qr) {
    if constexpr (mode == DotMode::F32) {
      if constexpr (QT == Ty::F32) {
        gload<VEC>(reinterpret_cast<const uint32_t*>(qrow) + c * VEC, qr);
      } else {
        uint32_t w[VEC / 2];
        gload<VEC / 2>(reinterpret_cast<const uint32_t*>(qrow) + c * (VEC / 2), w);
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) {
          float f[2];
          if constexpr (QT == Ty::BF16) Widen<Ty::BF16>::run(w[i], f); else Widen<Ty::F16>::run(w[i], f);
          qr[2 * i] = f2u(f[0]);
          qr[2 * i + 1] = f2u(f[1]);
        }
      }
    } else {
      gload<VEC / 2>(reinterpret_cast<const uint32_t*>(qrow) + c * (VEC / 2), qr);
    }
  }

  // sum_e q[e] * k[e] over this lane's VEC dims
  __device__ static __forceinline__ float dot(const uint32_t* qr, const uint32_t* kr) {
    float acc = 0.f;
    if constexpr (mode == DotMode::F32) {
      float kf[VEC];
#pragma unroll
      for (int i = 0; i < KDW; ++i) Widen<KV>::run(kr[i], kf + i * Widen<KV>::per_word);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc = __builtin_fmaf(u2f(qr[e]), kf[e], acc);
    } else if constexpr (KV == Ty::FP8) {
      // 4 codes per word -> two packed 16-bit pairs (exact), then dot2
#pragma unroll
      for (int i = 0; i < KDW; ++i) {
        auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)kr[i], false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)kr[i], true);
        if constexpr (mode == DotMode::BF16x2) {
          uint32_t p0 = __builtin_amdgcn_perm(f2u(lo[1]), f2u(lo[0]), 0x07060302u);
          uint32_t p1 = __builtin_amdgcn_perm(f2u(hi[1]), f2u(hi[0]), 0x07060302u);
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qr[2 * i]),
                                                __builtin_bit_cast(bf16x2_t, p0), acc, false);
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qr[2 * i + 1]),
                                                __builtin_bit_cast(bf16x2_t, p1), acc, false);
        } else {
          half2_t h0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(lo[0], lo[1]));
          half2_t h1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(hi[0], hi[1]));
          acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qr[2 * i]), h0, acc, false);
          acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qr[2 * i + 1]), h1, acc, false);
        }
      }
    } else if constexpr (mode == DotMode::BF16x2) {
#pragma unroll
      for (int i = 0; i < KDW; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qr[i]),
                                              __builtin_bit_cast(bf16x2_t, kr[i]), acc, false);
    } else {
#pragma unroll
      for (int i = 0; i < KDW; ++i)
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qr[i]),
                                     __builtin_bit_cast(half2_t, kr[i]), acc, false);
    }
    return acc;
  }
};

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

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over lane bits 3 and 2 of the row (lanes c, c^4, c^8, c^12).
__device__ __forceinline__ float row_sum_bits32(float x) {
  x += dpp<DPP_ROW_ROR8>(x);
  x += dpp<DPP_ROW_ROR4>(x);
  return x;
}

__device__ __forceinline__ int ctx_status(const DecodeParams& a, int ctx) {
  // 0 = fine, 1 = invalid (NaN row)
  if (ctx < 0 || ctx > a.max_context_len) return 1;
  int64_t nb = ((int64_t)ctx + a.block_size - 1) >> a.log2_block_size;
  return nb > a.max_blocks_per_seq ? 1 : 0;
}

template <Ty KV, Ty QT, int D, int G, int NW>
__global__ void __launch_bounds__(NW * 64)
attend_kernel(const DecodeParams a) {
  static_assert(D % LPT == 0, "head_dim must split over 16 lanes");
  constexpr int VEC = D / LPT;                    // dims per lane
  using Q = QK<KV, QT, VEC>;
  constexpr int KDW = Q::KDW;
  constexpr int NV = NL * G;                      // (token slot, head) values per lane
  constexpr int LOGNV = (NV >= 32) ? 5 : (NV >= 16) ? 4 : (NV >= 8) ? 3 : 2;
  constexpr int H = LOGNV < 4 ? LOGNV : 4;        // halving stages of the reduce-scatter
  constexpr int NF = NV >= 16 ? NV / 16 : 1;      // complete values per lane afterwards
  constexpr int DUP = 4 - H;                      // low lane bits holding duplicates
  constexpr int PSTRIDE = NV + G + 1;             // LDS floats per row for p and alpha

  __shared__ int s_tbl[PA_MAX_PART_BLOCKS];
  __shared__ int s_bad;
  __shared__ float s_p[NW][ROWS][PSTRIDE];
  __shared__ float s_rowm[NW][ROWS][G];
  __shared__ float s_rowl[NW][ROWS][G];
  __shared__ float s_wm[NW][G];
  __shared__ float s_wl[NW][G];
  __shared__ float s_wo[NW][G][D];

  // Grid (sequence, KV head, partition): workgroups are dealt to the 8 XCDs
  // round-robin by linear id; rotating the sequence by the partition index
  // spreads the partitions of one sequence over the XCDs.
  const int part = blockIdx.z;
  const int kvh = blockIdx.y;
  const int seq = (int)((blockIdx.x + (unsigned)part) % (unsigned)a.num_seqs);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int c = lane & 15;

  const int ctx = a.context_lens[seq];
  const int P = a.part_tokens;
  const int bad_ctx = ctx_status(a, ctx);
  const int nparts = (bad_ctx || ctx == 0) ? 1 : (ctx + P - 1) / P;
  if (part >= nparts) return;

  const int hq0 = kvh * G;
  const int64_t out_row0 = ((int64_t)seq * a.num_q_heads + hq0) * D;

  if (bad_ctx || ctx == 0) {
    const float fill = bad_ctx ? __builtin_nanf("") : 0.f;
    for (int i = tid; i < G * D; i += NW * 64) store_out<QT>(a.out, out_row0 + i, fill);
    return;
  }

  const int p0 = part * P;
  const int pend = min(p0 + P, ctx);
  const int lg = a.log2_block_size;
  const int lb0 = p0 >> lg;
  const int nlb = ((pend - 1) >> lg) - lb0 + 1;

  // q registers for the G heads of this KV head
  uint32_t qr[G][Q::QW];
  {
    const char* qbase = reinterpret_cast<const char*>(a.q);
#pragma unroll
    for (int h = 0; h < G; ++h)
      Q::load_q(qbase + (out_row0 + (int64_t)h * D) * TyInfo<QT>::bytes, c, qr[h]);
  }

  if (tid == 0) s_bad = 0;
  __syncthreads();
  const int32_t* trow = a.block_tables + (int64_t)seq * a.max_blocks_per_seq + lb0;
  for (int i = tid; i < nlb; i += NW * 64) {
    int id = trow[i];
    if (id < 0 || id >= a.num_blocks) { s_bad = 1; id = 0; }
    s_tbl[i] = id;
  }
  __syncthreads();
  const bool bad_tbl = s_bad != 0;

  const uint32_t* kpool = reinterpret_cast<const uint32_t*>(a.k_pool);
  const uint32_t* vpool = reinterpret_cast<const uint32_t*>(a.v_pool);
  // element offset of (this kv head, slot 0, this lane's dims) inside a block
  const int64_t lane_off = a.layer_offset + (int64_t)kvh * a.block_size * D + c * VEC;
  constexpr int EB = TyInfo<KV>::bytes;

  float m[NF], l[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) { m[j] = -__builtin_inff(); l[j] = 0.f; }
  float acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;

  const int ntok = pend - p0;
  const int nchunks = (ntok + CHUNK - 1) / CHUNK;
  const float qk_scale = a.qk_scale_log2;

  // Issue the loads of one chunk: the 4 K rows first, then the 4 V rows, so
  // the scores can start while the values are still in flight.
  auto load_chunk = [&](int k, uint32_t (&kr)[NL][KDW], uint32_t (&vr)[NL][KDW]) {
    int64_t widx[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      int t = p0 + k * CHUNK + i * ROWS + row;
      t = min(t, pend - 1);                      // never look past the context
      const int lb = (t >> lg) - lb0;
      const int64_t eidx = (int64_t)s_tbl[lb] * a.block_stride + lane_off +
                           (int64_t)(t & (a.block_size - 1)) * D;
      widx[i] = eidx * EB / 4;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) gload<KDW>(kpool + widx[i], kr[i]);
#pragma unroll
    for (int i = 0; i < NL; ++i) gload<KDW>(vpool + widx[i], vr[i]);
  };

  // One chunk of 16 tokens: scores, online softmax, P.V.
  auto process_chunk = [&](int k, uint32_t (&kr)[NL][KDW], uint32_t (&vr)[NL][KDW]) {
    const int cbase = p0 + k * CHUNK;
    const bool tail = cbase + CHUNK > pend;

    // --- scores --------------------------------------------------------
    float sc[NV];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[i * G + h] = Q::dot(qr[h], kr[i]);
    ReduceScatter<3, NV>::run(sc, c);

    // --- online softmax on the values this lane owns --------------------
    float pj[NF], alj[NF];
    const int tok_i = c >> 2;                    // token slot of this lane's values
    const bool valid = cbase + tok_i * ROWS + row < pend;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      float z = valid ? sc[j] * qk_scale : -__builtin_inff();
      float bm = row_max_bits32(z);
      float mn = fmaxf(m[j], bm);
      float al = (mn == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m[j] - mn);
      float p = valid ? __builtin_amdgcn_exp2f(z - mn) : 0.f;
      l[j] = l[j] * al + p;
      m[j] = mn;
      pj[j] = p;
      alj[j] = al;
    }
    // share p (and the per-head rescale factors) inside the row
    if ((c & ((1 << DUP) - 1)) == 0) {
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int v = NF * (c >> DUP) + j;
        s_p[wave][row][v] = pj[j];
        if (v < G) s_p[wave][row][NV + v] = alj[j];
      }
    }
    wave_sync();
    float pp[NV], alpha[G];
#pragma unroll
    for (int v = 0; v < NV; ++v) pp[v] = s_p[wave][row][v];
#pragma unroll
    for (int h = 0; h < G; ++h) alpha[h] = s_p[wave][row][NV + h];
    wave_sync();

    bool rescale = false;
#pragma unroll
    for (int h = 0; h < G; ++h) rescale |= alpha[h] != 1.f;
    if (__any(rescale)) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha[h];
    }

    // --- P.V -------------------------------------------------------------
    if (tail) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (cbase + i * ROWS + row >= pend) {
#pragma unroll
          for (int w = 0; w < KDW; ++w) vr[i][w] = 0u;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[VEC];
#pragma unroll
      for (int w = 0; w < KDW; ++w) Widen<KV>::run(vr[i][w], vf + w * Widen<KV>::per_word);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = pp[i * G + h];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = __builtin_fmaf(p, vf[e], acc[h][e]);
      }
    }

  };

  if (!bad_tbl && wave < nchunks) {
    // Ping-pong register buffers: the loads of the next chunk are in flight
    // while the current one is processed. The prefetch is unconditional (its
    // chunk index is clamped to the last chunk, which is in bounds and cached)
    // so every iteration has the same loads outstanding and the compiler's
    // wait counts stay tight; no register copy forces an early wait.
    uint32_t ka[NL][KDW], va[NL][KDW], kb[NL][KDW], vb[NL][KDW];
    const int last = nchunks - 1;
    int k = wave;
    int n = (nchunks - wave + NW - 1) / NW;       // chunks of this wave (>= 1)
    load_chunk(k, ka, va);
    for (; n >= 2; n -= 2) {
      load_chunk(min(k + NW, last), kb, vb);
      process_chunk(k, ka, va);
      k += NW;
      load_chunk(min(k + NW, last), ka, va);
      process_chunk(k, kb, vb);
      k += NW;
    }
    if (n == 1) process_chunk(k, ka, va);
  }

  // --- merge the 4 rows of each wave ---------------------------------------
  // sum of l over the token-slot bits (lane bits 3, 2): lanes c < 4 then
  // hold the row's per-head sums (lanes that differ only in the low DUP bits
  // hold identical copies, so no correction is needed)
  float lrow[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) lrow[j] = row_sum_bits32(l[j]);
  if (c < 4 && (c & ((1 << DUP) - 1)) == 0) {
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int v = NF * (c >> DUP) + j;      // head index for token slot 0
      if (v < G) { s_rowm[wave][row][v] = m[j]; s_rowl[wave][row][v] = lrow[j]; }
    }
  }
  wave_sync();
  float rsc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mw = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < ROWS; ++r) mw = fmaxf(mw, s_rowm[wave][r][h]);
    float lw = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float mr = s_rowm[wave][r][h];
      const float f = (mr == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(mr - mw);
      lw += f * s_rowl[wave][r][h];
      if (r == row) rsc[h] = f;
    }
    if (lane == 0) { s_wm[wave][h] = mw; s_wl[wave][h] = lw; }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float x = acc[h][e] * rsc[h];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[h][e] = x;
    }
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_wo[wave][h][c * VEC + e] = acc[h][e];
  }
  __syncthreads();

  // --- merge the waves and write ------------------------------------------
  const bool single = nparts == 1;
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx - h * D;
    float mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_wm[w][h]);
    float o = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_wm[w][h];
      const float f = (mw == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(mw - mx);
      o += f * s_wo[w][h][d];
      lt += f * s_wl[w][h];
    }
    if (bad_tbl) { o = __builtin_nanf(""); lt = __builtin_nanf(""); mx = 0.f; }
    if (single) {
      store_out<QT>(a.out, out_row0 + idx, o * (a.v_scale / lt));
    } else {
      const int64_t pr = ((int64_t)seq * a.num_q_heads + hq0 + h) * a.num_parts + part;
      a.ws_o[pr * D + d] = o;
      if (d == 0) { a.ws_m[pr] = mx; a.ws_l[pr] = lt; }
    }
  }
}

// Phase 2: M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
template <Ty QT, int D>
__global__ void __launch_bounds__(64)
merge_kernel(const DecodeParams a) {
  const int seq = blockIdx.x;
  const int hq = blockIdx.y;
  const int ctx = a.context_lens[seq];
  if (ctx_status(a, ctx) || ctx == 0) return;
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const int64_t pr0 = ((int64_t)seq * a.num_q_heads + hq) * a.num_parts;
  float mx = -__builtin_inff();
  for (int p = 0; p < nparts; ++p) mx = fmaxf(mx, a.ws_m[pr0 + p]);
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float lt = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float mp = a.ws_m[pr0 + p];
    const float f = (mp == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(mp - mx);
    lt += f * a.ws_l[pr0 + p];
    const float* op = a.ws_o + (pr0 + p) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += f * op[threadIdx.x + 64 * e];
  }
  const float norm = a.v_scale / lt;
  const int64_t orow = ((int64_t)seq * a.num_q_heads + hq) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) store_out<QT>(a.out, orow + threadIdx.x + 64 * e, o[e] * norm);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
constexpr int NWAVES = 4;

template <Ty KV, Ty QT, int D, int G>
static hipError_t launch_attend_t(const DecodeParams& a, hipStream_t st) {
  dim3 grid(a.num_seqs, a.num_kv_heads, a.num_parts);
  hipLaunchKernelGGL((attend_kernel<KV, QT, D, G, NWAVES>), grid, dim3(NWAVES * 64), 0, st, a);
  return hipGetLastError();
}

template <Ty KV, Ty QT, int D>
static hipError_t launch_attend_g(const DecodeParams& a, int g, hipStream_t st) {
  switch (g) {
    case 1: return launch_attend_t<KV, QT, D, 1>(a, st);
    case 2: return launch_attend_t<KV, QT, D, 2>(a, st);
    case 4: return launch_attend_t<KV, QT, D, 4>(a, st);
    case 8: return launch_attend_t<KV, QT, D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <Ty KV, Ty QT>
static hipError_t launch_attend_d(const DecodeParams& a, int g, hipStream_t st) {
  if constexpr (KV == Ty::F32) {
    if (a.head_dim == 64) return launch_attend_g<KV, QT, 64>(a, g, st);
    return hipErrorInvalidValue;
  } else {
    if (a.head_dim == 64) return launch_attend_g<KV, QT, 64>(a, g, st);
    if (a.head_dim == 128) return launch_attend_g<KV, QT, 128>(a, g, st);
    return hipErrorInvalidValue;
  }
}

hipError_t launch_attend(const DecodeParams& a, int kv_ty, int q_ty, int g, hipStream_t st) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  if (kv == Ty::F32 && q == Ty::F32) return launch_attend_d<Ty::F32, Ty::F32>(a, g, st);
  if (kv == Ty::F16 && q == Ty::F16) return launch_attend_d<Ty::F16, Ty::F16>(a, g, st);
  if (kv == Ty::BF16 && q == Ty::BF16) return launch_attend_d<Ty::BF16, Ty::BF16>(a, g, st);
  if (kv == Ty::FP8 && q == Ty::BF16) return launch_attend_d<Ty::FP8, Ty::BF16>(a, g, st);
  if (kv == Ty::FP8 && q == Ty::F16) return launch_attend_d<Ty::FP8, Ty::F16>(a, g, st);
  if (kv == Ty::FP8 && q == Ty::F32) return launch_attend_d<Ty::FP8, Ty::F32>(a, g, st);
  return hipErrorInvalidValue;
}

template <Ty QT>
static hipError_t launch_merge_q(const DecodeParams& a, hipStream_t st) {
  dim3 grid(a.num_seqs, a.num_q_heads);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<QT, 64>), grid, dim3(64), 0, st, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<QT, 128>), grid, dim3(64), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeParams& a, int q_ty, hipStream_t st) {
  switch ((Ty)q_ty) {
    case Ty::F32: return launch_merge_q<Ty::F32>(a, st);
    case Ty::F16: return launch_merge_q<Ty::F16>(a, st);
    case Ty::BF16: return launch_merge_q<Ty::BF16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
