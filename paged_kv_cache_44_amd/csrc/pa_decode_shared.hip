// pa_decode_shared.hip — decode that reads a prefix shared by several
// sequences once per group of up to 32/G of them ("Efficient Memory
// Management for Large Language Model Serving with PagedAttention",
// sampling paragraph: parallel samples of one prompt share its blocks;
// "Continuous Batching and PagedAttention", section "Sharing, the part that
// goes beyond fixing what broke"). The result is that of ordinary decode.
//
// Sharing is read off the block tables, so it needs no description from the
// caller: two sequences hold the same tokens wherever their tables name the
// same block, up to the shorter context. Planning, two kernels:
//  1. share_lcp_kernel, one wave per sequence: the tokens sequence s shares
//     with sequence s - 1 (common leading table entries naming valid blocks,
//     times the block size, capped by both contexts; 0 for invalid rows).
//  2. share_plan_kernel, one workgroup: runs of consecutive sequences each
//     sharing at least 16 tokens with the one before; a run shares the
//     minimum of those lengths (the common prefix of all its members),
//     rounded down to a multiple of 16. Each member starts its own pass
//     after it (share_start), and each group of up to 32/G consecutive
//     members is one prefix slot, kept at its first member's index; every
//     member records its slot (share_desc).
// Then one launch of the matrix-core kernel runs the prefix pass and the
// suffix pass side by side (pa_decode_sk.h), and shared_combine_kernel
// finishes every row the suffix pass leaves open.
#include "pa_decode_sk.h"

namespace pa {
namespace {

__device__ __forceinline__ bool row_valid(const DecodeParams& a, int ctx) {
  if (ctx <= 0 || ctx > a.max_context_len) return false;
  return (((int64_t)ctx + a.block_size - 1) >> a.log2_block_size) <= a.max_blocks_per_seq;
}

__global__ void __launch_bounds__(256) share_lcp_kernel(const DecodeParams a) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= a.num_seqs) return;
  int shared = 0;
  const int c1 = a.context_lens[s];
  const int c0 = s > 0 ? a.context_lens[s - 1] : 0;
  if (s > 0 && row_valid(a, c0) && row_valid(a, c1)) {
    const int cmin = min(c0, c1);
    const int nb = (cmin + a.block_size - 1) >> a.log2_block_size;
    const int32_t* r0 = a.block_tables + (int64_t)(s - 1) * a.max_blocks_per_seq;
    const int32_t* r1 = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    int k = nb;                                  // first entry that differs (or is invalid)
    for (int base = 0; base < nb; base += 64) {
      const int e = base + lane;
      bool stop = false;
      if (e < nb) {
        const int32_t b0 = r0[e], b1 = r1[e];
        stop = b0 != b1 || b1 < 0 || b1 >= a.num_blocks;
      }
      const uint64_t m = __ballot(stop);
      if (m) {
        k = base + __builtin_ctzll(m);
        break;
      }
    }
    shared = min((int64_t)k << a.log2_block_size, (int64_t)cmin);
  }
  if (lane == 0) a.share_lcp[s] = shared;
}

constexpr int PT = 1024;                         // planning threads
constexpr int NOPEN = 0x7fffffff;

// Inclusive scans of one value per thread across the workgroup: forward max
// (over threads 0..t) and backward min (over t..PT-1). Each wave scans with
// lane shuffles; the waves' totals meet in LDS once.
__device__ __forceinline__ int scan_max_fwd(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v = max(v, y);
  }
  if (lane == 63) s_wave[wv] = v;
  __syncthreads();
  for (int u = 0; u < wv; ++u) v = max(v, s_wave[u]);
  __syncthreads();
  return v;
}
__device__ __forceinline__ int scan_min_bwd(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(v, o);
    if (lane + o < 64) v = min(v, y);
  }
  if (lane == 0) s_wave[wv] = v;
  __syncthreads();
  for (int u = wv + 1; u < PT / 64; ++u) v = min(v, s_wave[u]);
  __syncthreads();
  return v;
}

template <int G>
__global__ void __launch_bounds__(PT) share_plan_kernel(const DecodeParams a) {
  constexpr int NS = PA_PREFIX_COLS / G;         // sequences per prefix slot
  constexpr int E = (PA_SK_MAX_SEQS + PT - 1) / PT;   // sequences per thread at most
  extern __shared__ int s_min[];                 // [num_seqs]: run minimum, at its first member
  __shared__ int s_buf[PT];
  __shared__ int s_wave[PT / 64];
  const int S = a.num_seqs;
  const int t = threadIdx.x;
  const int per = (S + PT - 1) / PT;             // <= E
  const int s0 = min(t * per, S), s1 = min(s0 + per, S);
  // a sequence opens a run unless it shares a whole chunk with the one before
  int lcp[E];
  int last_open = -1, first_open = S;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int s = s0 + i;
    lcp[i] = s < s1 ? a.share_lcp[s] : 0;
    if (s < s1) {
      s_min[s] = NOPEN;
      if (lcp[i] < 16) {
        last_open = s;
        first_open = min(first_open, s);
      }
    }
  }
  // last opening before this thread's range, first one after it
  const int upto = scan_max_fwd(last_open, s_wave);
  const int from = scan_min_bwd(first_open, s_wave);
  s_buf[t] = upto;
  __syncthreads();
  const int open_before = t > 0 ? s_buf[t - 1] : -1;
  __syncthreads();
  s_buf[t] = from;
  __syncthreads();
  const int open_after = t + 1 < PT ? s_buf[t + 1] : S;
  // each member's run: its first member (lead) and end (next opening)
  int lead[E], end[E];
  {
    int cur = open_before;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (s0 + i < s1 && lcp[i] < 16) cur = s0 + i;
      lead[i] = cur;
    }
    int nxt = open_after;
#pragma unroll
    for (int i = E - 1; i >= 0; --i) {
      end[i] = nxt;
      if (s0 + i < s1 && lcp[i] < 16) nxt = s0 + i;
    }
  }
  // the run's shared length: the minimum over its members after the first
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (s0 + i < s1 && lead[i] != s0 + i) atomicMin(&s_min[lead[i]], lcp[i]);
  __syncthreads();
  // the sizes of the two passes, for the split of the launch that runs them:
  // prefix chunks of every slot, and every sequence's own chunks
  int cp = 0, cs = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int s = s0 + i;
    if (s >= s1) continue;
    const int L = lead[i];
    const int m = s_min[L];
    const int pre = (end[i] - L >= 2 && m >= 16 && m != NOPEN) ? (m & ~15) : 0;
    a.share_start[s] = pre;
    // the slot of s: the group of NS members it belongs to, kept at the
    // group's first member
    const int slot = pre > 0 ? L + (s - L) / NS * NS : s;
    int4 d = make_int4(slot, 0, 0, 0);
    if (pre > 0 && slot == s) {
      d = make_int4(s, min(NS, end[i] - s), pre, 0);
      cp += pre / 16;
    }
    reinterpret_cast<int4*>(a.share_desc)[s] = d;
    const int ctx = a.context_lens[s];
    if (row_valid(a, ctx)) cs += (ctx - pre + 15) / 16;
  }
  __shared__ int s_tot[2][PT / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    cp += __shfl_xor(cp, o);
    cs += __shfl_xor(cs, o);
  }
  if ((t & 63) == 0) {
    s_tot[0][t >> 6] = cp;
    s_tot[1][t >> 6] = cs;
  }
  __syncthreads();
  if (t == 0) {
    int tp = 0, tq = 0;
    for (int w = 0; w < PT / 64; ++w) {
      tp += s_tot[0][w];
      tq += s_tot[1][w];
    }
    a.share_tot[0] = tp;
    a.share_tot[1] = tq;
  }
}

// Every row the suffix pass does not finish: a sequence without a prefix
// whose segment was cut across teams (its pieces, combined as the plain
// decode's merge does), and every sequence with a prefix (the suffix pass's
// pieces, or the partial it left for a segment inside one team, plus the
// prefix pass's pieces of its columns), normalised and stored. One wave per
// (sequence, KV head), 64 / G lanes per head, every piece's loads of a batch
// of eight in flight before they are combined (M = max m_p,
// L = sum 2^(m_p - M) l_p, O likewise).
template <Ty QT, int G, int D>
__global__ void __launch_bounds__(256) shared_combine_kernel(const DecodeParams a) {
  constexpr int LPH = 64 / G;                    // lanes per head
  constexpr int DPL = D / LPH;                   // dims per lane
  constexpr int NB = 8;                          // pieces per batch
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = a.num_kv_heads, T = a.team, HG = H / T;
  if (w >= (int64_t)a.num_seqs * H) return;
  const int s = (int)(w / H), kvh = (int)(w - (int64_t)s * H);
  const int hg = kvh / T, ti = kvh % T;
  const int ctx = a.context_lens[s];
  const int st0 = own_start(a, s, ctx);
  // the suffix segment: its chunks and the teams holding its pieces
  const int nsuf = seq_chunks(a, ctx) > 0 ? (ctx - st0 + CH - 1) / CH : 0;
  int t0 = 0, t1 = -1, steams = 1;
  int64_t ccs = 0;
  bool own_partial = false, bad_record = false;
  if (nsuf > 0) {
    const int4 sg = reinterpret_cast<const int4*>(a.suf_seg)[(int64_t)s * HG + hg];
    if (!segment_record_ok(sg, a.suf_teams)) {
      bad_record = true;
    } else if (sg.x == sg.y) {
      if (st0 <= 0) return;                      // finished by the suffix pass
      own_partial = true;
    } else {
      t0 = sg.x;
      t1 = sg.y;
      ccs = sg.z;
      steams = sg.w;
    }
  } else if (st0 <= 0) {
    return;                                      // empty or invalid row: written by the suffix pass
  }
  const int hh = lane / LPH, d0 = (lane % LPH) * DPL;
  const int64_t pr = (int64_t)s * a.num_q_heads + (int64_t)kvh * G + hh;
  float M = -__builtin_inff(), L = 0.f, O[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) O[i] = 0.f;
  if (own_partial) {
    M = a.pre_m[pr];
    L = a.pre_l[pr];
#pragma unroll
    for (int i = 0; i < DPL; ++i) O[i] = a.pre_o[pr * D + d0 + i];
  }
  if (bad_record) L = __builtin_nanf("");
  // the pieces of teams ta .. tb of a pass (a team with an empty range holds
  // none) at slots ((team + cseg) * T + ti) * gc + col
  auto combine_pieces = [&](const float* wm, const float* wl, const float* wo, int64_t cseg, int ta,
                            int tb, int64_t cc, int teams, int gc, int col) __attribute__((always_inline)) {
    for (int tq = ta; tq <= tb; tq += NB) {
      float mv[NB], lv[NB], ov[NB][DPL];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int tm = tq + u;
        const bool ok = tm <= tb && team_begin(tm, cc, teams) != team_begin(tm + 1, cc, teams);
        const int64_t sl = ok ? ((tm + cseg) * T + ti) * gc + col : 0;
        mv[u] = ok ? wm[sl] : -__builtin_inff();
        lv[u] = ok ? wl[sl] : 0.f;
        const float* po = wo + sl * D + d0;
        if constexpr (DPL % 4 == 0) {
#pragma unroll
          for (int i = 0; i < DPL; i += 4) {
            const float4 x = ok ? *reinterpret_cast<const float4*>(po + i) : make_float4(0, 0, 0, 0);
            ov[u][i] = x.x; ov[u][i + 1] = x.y; ov[u][i + 2] = x.z; ov[u][i + 3] = x.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < DPL; ++i) ov[u][i] = ok ? po[i] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float mn = fmaxf(M, mv[u]);
        if (mn == -__builtin_inff()) continue;
        const float f1 = __builtin_amdgcn_exp2f(M - mn), f2 = __builtin_amdgcn_exp2f(mv[u] - mn);
        L = L * f1 + lv[u] * f2;
#pragma unroll
        for (int i = 0; i < DPL; ++i) O[i] = O[i] * f1 + ov[u][i] * f2;
        M = mn;
      }
    }
  };
  // the suffix pass's pieces of a cut segment
  combine_pieces(a.ws_m, a.ws_l, a.ws_o, (int64_t)s * HG + hg, t0, t1, ccs, steams, G, hh);
  // the prefix pass's pieces of the sequence's columns
  if (st0 > 0) {
    int64_t cs = 0, ccp = 0;
    int col0 = 0, p0 = 0, p1 = -1, pteams = 1;
    if (!prefix_segment(a, s, hg, HG, PA_PREFIX_COLS / G, G, cs, col0, p0, p1, ccp, pteams))
      L = __builtin_nanf("");
    combine_pieces(a.pre_ws_m, a.pre_ws_l, a.pre_ws_o, cs, p0, p1, ccp, pteams, PA_PREFIX_COLS,
                   col0 + hh);
  }
  const float norm = a.v_scale / L;
#pragma unroll
  for (int i = 0; i < DPL; ++i) store_out<QT>(a.out, pr * D + d0 + i, O[i] * norm);
}

}  // namespace

template <Ty QT>
static hipError_t launch_shared_combine_q(const DecodeParams& a, int g, hipStream_t st) {
  const int64_t waves = (int64_t)a.num_seqs * a.num_kv_heads;
  const dim3 grid((unsigned)((waves + 3) / 4));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  };
  if (a.head_dim == 128) {
    switch (g) {
      case 1: return go(shared_combine_kernel<QT, 1, 128>);
      case 2: return go(shared_combine_kernel<QT, 2, 128>);
      case 4: return go(shared_combine_kernel<QT, 4, 128>);
      case 8: return go(shared_combine_kernel<QT, 8, 128>);
    }
  } else if (a.head_dim == 64) {
    switch (g) {
      case 1: return go(shared_combine_kernel<QT, 1, 64>);
      case 2: return go(shared_combine_kernel<QT, 2, 64>);
      case 4: return go(shared_combine_kernel<QT, 4, 64>);
      case 8: return go(shared_combine_kernel<QT, 8, 64>);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_shared_combine(const DecodeParams& a, int q_ty, int g, hipStream_t st) {
  if ((Ty)q_ty == Ty::BF16) return launch_shared_combine_q<Ty::BF16>(a, g, st);
  if ((Ty)q_ty == Ty::F16) return launch_shared_combine_q<Ty::F16>(a, g, st);
  return hipErrorInvalidValue;
}

hipError_t launch_share_plan(const DecodeParams& a, int g, hipStream_t st) {
  if (a.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(share_lcp_kernel, dim3((a.num_seqs + 3) / 4), dim3(256), 0, st, a);
  const size_t lds = (size_t)a.num_seqs * sizeof(int);
  switch (g) {
    case 1: hipLaunchKernelGGL(share_plan_kernel<1>, dim3(1), dim3(PT), lds, st, a); break;
    case 2: hipLaunchKernelGGL(share_plan_kernel<2>, dim3(1), dim3(PT), lds, st, a); break;
    case 4: hipLaunchKernelGGL(share_plan_kernel<4>, dim3(1), dim3(PT), lds, st, a); break;
    case 8: hipLaunchKernelGGL(share_plan_kernel<8>, dim3(1), dim3(PT), lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {

// The shared-prefix decode's launch of both passes (attend_sk_dual_kernel):
// f(pool type, query type, head dim, group) for the runtime values, as
// integral constants; -1 for a combination it does not take.
template <Ty V> using TyC = std::integral_constant<Ty, V>;
template <int V> using IntC = std::integral_constant<int, V>;
template <typename F>
static int sk_dual_dispatch(int kv_ty, int q_ty, int head_dim, int g, F&& f) {
  auto by_g = [&](auto kv, auto q, auto d) -> int {
    switch (g) {
      case 1: return f(kv, q, d, IntC<1>{});
      case 2: return f(kv, q, d, IntC<2>{});
      case 4: return f(kv, q, d, IntC<4>{});
      case 8: return f(kv, q, d, IntC<8>{});
      default: return -1;
    }
  };
  auto by_d = [&](auto kv, auto q) -> int {
    if (head_dim == 64) return by_g(kv, q, IntC<64>{});
    if (head_dim == 128) return by_g(kv, q, IntC<128>{});
    return -1;
  };
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  if (kv == Ty::BF16 && q == Ty::BF16) return by_d(TyC<Ty::BF16>{}, TyC<Ty::BF16>{});
  if (kv == Ty::F16 && q == Ty::F16) return by_d(TyC<Ty::F16>{}, TyC<Ty::F16>{});
  if (kv == Ty::FP8 && q == Ty::BF16) return by_d(TyC<Ty::FP8>{}, TyC<Ty::BF16>{});
  if (kv == Ty::FP8 && q == Ty::F16) return by_d(TyC<Ty::FP8>{}, TyC<Ty::F16>{});
  return -1;
}

static int sk_blocks_dual(int kv_ty, int q_ty, int head_dim, int g, int num_seqs) {
  return sk_dual_dispatch(kv_ty, q_ty, head_dim, g, [&](auto kv, auto q, auto d, auto gg) -> int {
    constexpr Ty KV = decltype(kv)::value, QT = decltype(q)::value;
    constexpr int D = decltype(d)::value, G = decltype(gg)::value;
    return sk_resident_blocks(reinterpret_cast<const void*>(&attend_sk_dual_kernel<KV, QT, D, G>),
                              sk_lds_bytes(num_seqs, M_PREFIX), sk_waves_per_simd<KV, D, G, M_PREFIX>());
  });
}

static hipError_t sk_launch_dual(const DecodeParams& p, const DecodeParams& q, int kv_ty, int q_ty,
                                 int g, int blocks, hipStream_t st) {
  const int r = sk_dual_dispatch(kv_ty, q_ty, p.head_dim, g, [&](auto kv, auto qt, auto d, auto gg) -> int {
    constexpr Ty KV = decltype(kv)::value, QT = decltype(qt)::value;
    constexpr int D = decltype(d)::value, G = decltype(gg)::value;
    hipLaunchKernelGGL((attend_sk_dual_kernel<KV, QT, D, G>), dim3(blocks), dim3(NWM * 64),
                       sk_lds_bytes(p.num_seqs, M_PREFIX), st, p, q);
    return (int)hipGetLastError();
  });
  return r < 0 ? hipErrorInvalidValue : (hipError_t)r;
}

}  // namespace

int sk_blocks_shared_dual(int kv_ty, int q_ty, int head_dim, int g, int num_seqs) {
  return sk_blocks_dual(kv_ty, q_ty, head_dim, g, num_seqs);
}

hipError_t launch_attend_shared_dual(const DecodeParams& pre, const DecodeParams& suf, int kv_ty,
                                     int q_ty, int g, int blocks, hipStream_t st) {
  return sk_launch_dual(pre, suf, kv_ty, q_ty, g, blocks, st);
}


}  // namespace pa
