// pa_decode_shared.hip — decode that reads a prefix shared by several
// sequences once per group of up to 16/G of them ("Efficient Memory
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
//     after it (share_start), and each group of up to 16/G consecutive
//     members is one prefix slot, kept at its first member's index
//     (share_desc).
// Then the matrix-core kernel's prefix pass and suffix pass (pa_decode_sk.h).
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

// Inclusive scans of one value per thread across the workgroup, through
// LDS: forward max (over threads 0..t) and backward min (over t..PT-1).
__device__ __forceinline__ int scan_max_fwd(int v, int* s_buf) {
  const int t = threadIdx.x;
  for (int o = 1; o < PT; o <<= 1) {
    s_buf[t] = v;
    __syncthreads();
    if (t >= o) v = max(v, s_buf[t - o]);
    __syncthreads();
  }
  return v;
}
__device__ __forceinline__ int scan_min_bwd(int v, int* s_buf) {
  const int t = threadIdx.x;
  for (int o = 1; o < PT; o <<= 1) {
    s_buf[t] = v;
    __syncthreads();
    if (t + o < PT) v = min(v, s_buf[t + o]);
    __syncthreads();
  }
  return v;
}

template <int G>
__global__ void __launch_bounds__(PT) share_plan_kernel(const DecodeParams a) {
  constexpr int NS = 16 / G;                     // sequences per prefix slot
  constexpr int E = (PA_SK_MAX_SEQS + PT - 1) / PT;   // sequences per thread at most
  extern __shared__ int s_min[];                 // [num_seqs]: run minimum, at its first member
  __shared__ int s_buf[PT];
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
  const int upto = scan_max_fwd(last_open, s_buf);
  const int from = scan_min_bwd(first_open, s_buf);
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
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int s = s0 + i;
    if (s >= s1) continue;
    const int L = lead[i];
    const int m = s_min[L];
    const int pre = (end[i] - L >= 2 && m >= 16 && m != NOPEN) ? (m & ~15) : 0;
    a.share_start[s] = pre;
    int4 d = make_int4(s, 0, 0, 0);
    if (pre > 0 && (s - L) % NS == 0) d = make_int4(s, min(NS, end[i] - s), pre, 0);
    reinterpret_cast<int4*>(a.share_desc)[s] = d;
  }
}

}  // namespace

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

int sk_blocks_shared(int kv_ty, int q_ty, int head_dim, int g, int num_seqs, int mode) {
  return mode == M_PREFIX ? sk_blocks_mode<M_PREFIX>(kv_ty, q_ty, head_dim, g, num_seqs)
                          : sk_blocks_mode<M_SUFFIX>(kv_ty, q_ty, head_dim, g, num_seqs);
}

hipError_t launch_attend_shared(const DecodeParams& a, int kv_ty, int q_ty, int g, int blocks,
                                int mode, hipStream_t st) {
  return mode == M_PREFIX ? sk_launch_attend<M_PREFIX>(a, kv_ty, q_ty, g, blocks, st)
                          : sk_launch_attend<M_SUFFIX>(a, kv_ty, q_ty, g, blocks, st);
}

hipError_t launch_merge_shared(const DecodeParams& a, int q_ty, int g, int blocks, int mode,
                               hipStream_t st) {
  return mode == M_PREFIX ? sk_launch_merge<M_PREFIX>(a, q_ty, g, blocks, st)
                          : sk_launch_merge<M_SUFFIX>(a, q_ty, g, blocks, st);
}

}  // namespace pa
