// pa_prefill.hip — paged prefill (whole, chunked, or recompute) attention on
// the gfx950 matrix cores: causal attention of each sequence's newest
// positions over the keys and values of all its positions, reached through
// its block table.
//
// A recomputed request runs its prompt and generated tokens again as one
// prefill pass ("When KV Capacity Runs Out", section "Recompute KV from token
// history"); the pass's keys and values are first written to the pool, then
// every position p attends to positions 0 .. p. Query rows are packed
// sequence by sequence (query_start_loc); the n_s rows of sequence s are its
// positions ctx_s - n_s .. ctx_s - 1.
//
// A column tile is 16/G consecutive query positions x the G query heads of a
// KV head; one wave owns 2 consecutive tiles of one (sequence, KV head), so
// each 16-key chunk of K and V it loads serves 32 columns, and the 4 waves of
// a workgroup own consecutive tiles of the same (sequence, KV head), so they
// stream the same key chunks at about the same time and share them in the
// caches. Per chunk the score tiles S[16 keys][16 columns] and P.V run on the
// matrix cores as in decode (pa_mfma.h), with the causal mask key <=
// position(column). A three-stage pipeline keeps the block ids of chunk j+2
// and the K/V of chunk j+1 in flight while chunk j is processed; every step
// issues the same loads. Workgroups launch last-first, so the longest causal
// ranges start first.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr int PW = 4;           // waves per workgroup
constexpr int PCH = 16;         // keys per chunk

template <Ty KV, int D>
constexpr int pf_waves_per_simd() { return D == 64 ? 3 : 2; }

// Column tiles per wave: each loaded key chunk serves NT x 16 columns.
constexpr int PNT = 2;

// K rows are loaded straight in the score product's operand layout (lane l:
// token l%16, dims 32k + 8(l/16) of step k): no lane exchange afterwards.
// The four waves of a workgroup read each chunk, mostly from the caches, so
// the whole-line reads that decode streams from memory with bring nothing
// here (measured slightly slower).
template <int D, int EB>
struct PfKLayout {
  static constexpr int KS = D / 32;
  static constexpr int KDW = 8 * EB / 4;
  static constexpr int KR = KS;
  static constexpr int KW = KDW;
};
template <int D, int EB>
__device__ __forceinline__ int pf_kdim(int k, int a) {
  return 32 * k + 8 * a;
}

template <Ty KV, Ty QT, int D, int G>
__global__ void __launch_bounds__(PW * 64)
__attribute__((amdgpu_waves_per_eu(pf_waves_per_simd<KV, D>())))
prefill_kernel(const PrefillParams a) {
  static_assert(QT == Ty::BF16 || QT == Ty::F16, "16-bit queries");
  static_assert(G >= 1 && G <= 16 && 16 % G == 0, "group divides the 16-column tile");
  constexpr int EB = TyInfo<KV>::bytes;
  using KL = PfKLayout<D, EB>;
  constexpr int KS = KL::KS;
  constexpr int KR = KL::KR;
  constexpr int KW = KL::KW;
  constexpr int VPL = D / 16;
  constexpr int VDW = VPL * EB / 4;
  constexpr int NT = PNT;
  constexpr int QTOK = 16 / G;              // query positions per column tile
  constexpr int WTOK = NT * QTOK;           // query positions per wave

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;                  // column: position n / G, head n % G
  const int H = a.num_kv_heads;
  const int s = (int)(blockIdx.x / H);
  const int kvh = (int)(blockIdx.x - (unsigned)s * H);
  // the workgroup's waves take consecutive position groups of one (sequence,
  // KV head): they stream the same key chunks at about the same time
  const int t0 = ((int)(gridDim.y - 1 - blockIdx.y) * PW + wave) * WTOK;
  const int r0 = a.query_start_loc[s];
  const int nq = a.query_start_loc[s + 1] - r0;
  // rows outside the packed query array are never touched
  if (nq <= 0 || t0 >= nq || r0 < 0 || (int64_t)r0 + nq > a.num_q_tokens) return;
  const int rows = min(WTOK, nq - t0);      // query positions of this wave
  const int ctx = a.context_lens[s];
  const int lg = a.log2_block_size;
  const bool ctx_ok = ctx >= nq && ctx <= a.max_context_len &&
                      (((int64_t)ctx + a.block_size - 1) >> lg) <= a.max_blocks_per_seq;

  f32x4_t acc[NT][VPL];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int m = 0; m < VPL; ++m) acc[t][m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  // output rows of tile t: column c = 4g + r of its accumulators
  auto store_rows = [&](int t, const float (&norm)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 4 * g + r;
      const int tok = t * QTOK + c / G;
      if (tok < rows) {
        const int64_t o = (((int64_t)r0 + t0 + tok) * a.num_q_heads + (int64_t)kvh * G + c % G) * D +
                          VPL * n;
#pragma unroll
        for (int m = 0; m < VPL; ++m) store_out<QT>(a.out, o + m, acc[t][m][r] * norm[r]);
      }
    }
  };
  if (!ctx_ok) {                            // invalid context or query count: NaN rows
    const float nan4[4] = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
    for (int t = 0; t < NT; ++t) store_rows(t, nan4);
    return;
  }

  // pools as bytes: element offsets (never negative) scale by EB, with no
  // signed division on the load path
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  auto dw = [](const char* p, int64_t e) __attribute__((always_inline)) {
    return reinterpret_cast<const uint32_t*>(p + e * EB);
  };
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.q);
  const int bmask = a.block_size - 1;
  const bool big_blocks = a.block_size >= PCH;
  const float qk_scale = a.qk_scale_log2;
  const int pos0 = ctx - nq + t0;           // position of the wave's first row
  const int p_last = pos0 + rows - 1;
  const int nch = p_last / PCH + 1;         // key chunks the wave needs
  const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int64_t head_off = a.layer_offset + (int64_t)kvh * a.block_size * D;

  // q of each tile as the B operand: lane l holds column l%16 (rows past the
  // wave's last repeat it; their scores are masked)
  uint4 qr[NT][KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t row = (((int64_t)r0 + t0 + min(t * QTOK + n / G, rows - 1)) * a.num_q_heads +
                         (int64_t)kvh * G + n % G) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint32_t w4[4];
      ld<4>(qw + ((row + pf_kdim<D, EB>(k, g)) >> 1), w4);
      qr[t][k] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }

  // block ids of chunk j (clamped to the last chunk): lane i holds the id of
  // the chunk's i-th block, lanes past its last block repeat the last one
  auto fetch_ids = [&](int j) __attribute__((always_inline)) -> int {
    j = min(j, nch - 1);
    const int cb = j * PCH;
    const int fb = cb >> lg;
    const int lb = (min(cb + PCH, ctx) - 1) >> lg;
    return trow[min(fb + lane, lb)];
  };
  bool bad = false;                         // a bad block id was seen
  auto load_kv = [&](int j, int idr, uint32_t (&kr)[KR][KW], uint32_t (&vr)[4][VDW])
      __attribute__((always_inline)) {
    j = min(j, nch - 1);
    const int cb = j * PCH;
    const int fb = cb >> lg;
    const bool badl = idr < 0 || idr >= a.num_blocks;
    bad = bad || __any(badl);
    const int idv = badl ? 0 : idr;

    auto elem_of = [&](int t) __attribute__((always_inline)) -> int64_t {   // element of token t, dim 0
      t = min(t, ctx - 1);
      const int id = big_blocks ? __builtin_amdgcn_readfirstlane(idv) : __shfl(idv, (t >> lg) - fb);
      return (int64_t)id * a.block_stride + head_off + (int64_t)(t & bmask) * D;
    };
    // K in the operand layout (lane l: token l%16, dims 32k + 8(l/16)); V
    // rows 4(l/16) .. +3, dims VPL*(l%16) .. +VPL
    int64_t ek, ev[4];
    if (big_blocks) {
      const int64_t base = elem_of(cb);
      ek = base + (int64_t)min(n, ctx - 1 - cb) * D + 8 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) ev[r] = base + (int64_t)min(4 * g + r, ctx - 1 - cb) * D + VPL * n;
    } else {
      ek = elem_of(cb + n) + 8 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) ev[r] = elem_of(cb + 4 * g + r) + VPL * n;
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) ld<KW>(dw(kpool, ek + 32 * k), kr[k]);
#pragma unroll
    for (int r = 0; r < 4; ++r) ld<VDW>(dw(vpool, ev[r]), vr[r]);
  };

  float m_ref[NT], l_sum[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_ref[t] = -__builtin_inff();           // reference max of the column (log2 units)
    l_sum[t] = 0.f;                         // this lane's share of the column's sum
  }
  auto process = [&](int j, const uint32_t (&kr)[KR][KW], const uint32_t (&vr)[4][VDW])
      __attribute__((always_inline)) {
    const int cb = j * PCH;
    uint32_t kraw[KS][KL::KDW];
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int x = 0; x < KL::KDW; ++x) kraw[k][x] = kr[k][x];
    uint32_t vb[VPL][2];                    // P.V B operands, shared by the tiles
    if constexpr (KV == Ty::FP8) {
      bool live[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) live[r] = cb + 4 * g + r < ctx;
      pv_operands_fp8<D>(vr, live, vb);
    } else {
      uint32_t vw[4][D / 32];
      if (cb + PCH <= ctx) {                // whole chunk: every value row is live
        const bool live[4] = {true, true, true, true};
        v_operand<KV, QT, D>(vr, live, vw);
      } else {
        bool live[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) live[r] = cb + 4 * g + r < ctx;
        v_operand<KV, QT, D>(vr, live, vw);
      }
      pv_operands<D>(vw, vb);
    }
    // a chunk wholly before the wave's first position needs no causal mask
    const bool below = cb + PCH - 1 <= pos0;
    const bool full_wave = rows == WTOK;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tok = t * QTOK + n / G;
      const int pcol = pos0 + tok;          // position of this column
      if (t * QTOK >= rows) break;          // tile past the wave's rows (uniform)
      const f32x4_t sc = chunk_scores_raw<KV, QT, D>(kraw, [&](int k) {
        return qr[t][k];
      });
      float z[4];
      if (below && full_wave) {
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = sc[r] * qk_scale;
      } else if (below) {
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = tok < rows ? sc[r] * qk_scale : -__builtin_inff();
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tk = cb + 4 * g + r;
          z[r] = (tok < rows && tk <= pcol) ? sc[r] * qk_scale : -__builtin_inff();
        }
      }
      softmax_pv_b<KV, QT, D>(z, vb, acc[t], m_ref[t], l_sum[t], lane);
    }
  };

  uint32_t kA[KR][KW], vA[4][VDW], kB[KR][KW], vB[4][VDW];
  int iA = fetch_ids(0);
  int iB = fetch_ids(1);
  load_kv(0, iA, kA, vA);
  // One exit, at the end of the pair: chunk nch (odd nch) is processed as a
  // no-op (its rows are past the context: V reads as zero, every score is
  // masked). A leave after the first chunk of the pair would reach the loop
  // latch with B's loads unread (the divergent loop is put in single-exit
  // form), and the wait analysis would then drain A's loads at the top of
  // every pair before B's registers are reused.
  for (int j = 0; j < nch; j += 2) {
    iA = fetch_ids(j + 2);
    load_kv(j + 1, iB, kB, vB);
    process(j, kA, vA);
    iB = fetch_ids(j + 3);
    load_kv(j + 2, iA, kA, vA);
    process(j + 1, kB, vB);
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float norm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float lt = l_sum[t] + __shfl_xor(l_sum[t], 16);
      lt += __shfl_xor(lt, 32);
      norm[r] = bad ? __builtin_nanf("") : a.v_scale / __shfl(lt, 4 * g + r);
    }
    store_rows(t, norm);
  }
}

template <Ty KV, Ty QT, int D>
hipError_t launch_g(const PrefillParams& a, int g, dim3 grid, hipStream_t st) {
  switch (g) {
    case 1: hipLaunchKernelGGL((prefill_kernel<KV, QT, D, 1>), grid, dim3(PW * 64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<KV, QT, D, 2>), grid, dim3(PW * 64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<KV, QT, D, 4>), grid, dim3(PW * 64), 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<KV, QT, D, 8>), grid, dim3(PW * 64), 0, st, a); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<KV, QT, D, 16>), grid, dim3(PW * 64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <Ty KV, Ty QT>
hipError_t launch_d(const PrefillParams& a, int g, dim3 grid, hipStream_t st) {
  if (a.head_dim == 64) return launch_g<KV, QT, 64>(a, g, grid, st);
  if (a.head_dim == 128) return launch_g<KV, QT, 128>(a, g, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int kv_ty, int q_ty, int head_dim, int g) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  const bool types = (kv == Ty::BF16 && q == Ty::BF16) || (kv == Ty::F16 && q == Ty::F16) ||
                     (kv == Ty::FP8 && (q == Ty::BF16 || q == Ty::F16));
  return types && (head_dim == 64 || head_dim == 128) &&
         (g == 1 || g == 2 || g == 4 || g == 8 || g == 16);
}

// Workgroups along the query rows: each covers PW * PNT * (16 / g) positions.
int prefill_tiles(int g, int max_query_len) {
  const int64_t per = PW * PNT * (16 / g);
  return (int)(((int64_t)max_query_len + per - 1) / per);
}

hipError_t launch_prefill(const PrefillParams& a, int kv_ty, int q_ty, int g, int max_query_len,
                          hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.num_seqs * a.num_kv_heads), (unsigned)prefill_tiles(g, max_query_len));
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  if (kv == Ty::BF16 && q == Ty::BF16) return launch_d<Ty::BF16, Ty::BF16>(a, g, grid, st);
  if (kv == Ty::F16 && q == Ty::F16) return launch_d<Ty::F16, Ty::F16>(a, g, grid, st);
  if (kv == Ty::FP8 && q == Ty::BF16) return launch_d<Ty::FP8, Ty::BF16>(a, g, grid, st);
  if (kv == Ty::FP8 && q == Ty::F16) return launch_d<Ty::FP8, Ty::F16>(a, g, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
