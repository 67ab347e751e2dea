// pa_api.hip — the C ABI declared in include/pa.h: argument validation on
// the host, launch-size choices, and dispatch to the gfx950 kernels. Nothing
// here allocates device memory or synchronises the host.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

using pa::DecodeParams;

// Workspace of pa_decode_no_alloc: a fixed array in this library's device
// code, one copy on every GPU the library runs on, held until the process
// ends. Host code never passes `scratch` itself (in host code the name only
// stands for the symbol): it looks up the array's address on each device
// once and hands that address to the kernels.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_NO_ALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`: looked up with that device current
// on the first call that needs it, then kept.
pa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
      p = ptr;
    }
  }
  *out = p;
  return PA_OK;
}

int elem_bytes(pa_dtype t) {
  switch (t) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
  }
  return 0;
}

bool valid_dtype(int t) { return t >= PA_F32 && t <= PA_FP8_E4M3; }

// The integer a caller stored in an enum-typed argument or field, read
// without going through the enum type: a C caller may pass any int, and in
// C++ reading a value outside the enumerators' range through the enum type
// is undefined. Every enum input is checked this way before it is used.
template <class E>
int raw(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enums of the C ABI are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

bool valid_q_dtype(const pa_dtype& q) {
  const int v = raw(q);
  return v == PA_F32 || v == PA_F16 || v == PA_BF16;
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Geometry checks shared by every call. `need_ptrs` requires k and v.
pa_status check_cache(const pa_kv_cache* c, bool need_ptrs) {
  if (!c) return PA_ERR_INVALID_ARG;
  if (!valid_dtype(raw(c->dtype))) return PA_ERR_INVALID_ARG;
  if (need_ptrs && (!c->k || !c->v)) return PA_ERR_INVALID_ARG;
  if (c->num_blocks <= 0 || c->num_layers <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return PA_ERR_INVALID_ARG;
  if (!is_pow2(c->block_size) || c->block_size > 256) return PA_ERR_INVALID_ARG;
  if (c->layer_stride < 0 || c->block_stride < 0) return PA_ERR_INVALID_ARG;
  // sizes in 128-bit arithmetic: extreme strides must be refused, not wrap
  using i128 = __int128;
  const i128 slab = (i128)c->num_kv_heads * c->block_size * c->head_dim;
  // no two (block, layer) slabs may overlap: block-major (a block's layers
  // nested inside its stride) or layer-major (a layer's blocks nested inside
  // the layer stride)
  const bool one_l = c->num_layers == 1, one_b = c->num_blocks == 1;
  const bool block_major =
      (one_l || (i128)c->layer_stride >= slab) &&
      (one_b || (i128)c->block_stride >= (i128)(c->num_layers - 1) * c->layer_stride + slab);
  const bool layer_major =
      (one_b || (i128)c->block_stride >= slab) &&
      (one_l || (i128)c->layer_stride >= (i128)(c->num_blocks - 1) * c->block_stride + slab);
  if (!block_major && !layer_major) return PA_ERR_INVALID_ARG;
  const int eb = elem_bytes(c->dtype);
  // kernels address the pool with 64-bit byte offsets: its extent and both
  // strides in bytes must fit
  const i128 extent = ((i128)(c->num_blocks - 1) * c->block_stride +
                       (i128)(c->num_layers - 1) * c->layer_stride + slab) * eb;
  const i128 lim = (i128)INT64_MAX;
  if (extent > lim || (i128)c->block_stride * eb > lim || (i128)c->layer_stride * eb > lim)
    return PA_ERR_UNSUPPORTED;
  if ((c->block_stride * eb) % 16 || (c->layer_stride * eb) % 16) return PA_ERR_UNSUPPORTED;
  if (((int64_t)c->head_dim * eb) % 16) return PA_ERR_UNSUPPORTED;
  if (need_ptrs && (!aligned(c->k, 16) || !aligned(c->v, 16))) return PA_ERR_UNSUPPORTED;
  if (c->dtype == PA_FP8_E4M3) {
    if (!(c->k_scale > 0.f) || !isfinite(c->k_scale) || !(c->v_scale > 0.f) || !isfinite(c->v_scale))
      return PA_ERR_INVALID_ARG;
  } else if (c->k_scale != 1.0f || c->v_scale != 1.0f) {
    return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

// ---------------------------------------------------------------------------
// decode planning
// ---------------------------------------------------------------------------
struct DecodePlan {
  int g;
  bool mfma;           // evenly split matrix-core kernel (else the VALU kernel)
  int sk_blocks;       // matrix-core path: workgroups launched
  int part_tokens;     // VALU path: tokens per partition; matrix-core path: 16
  int num_parts;       // VALU path: partitions in the launch grid
  size_t ws_bytes;     // 0 when no workspace is needed
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace regions, in order: o, m, l (fp32), then (matrix-core path) one
// 16-byte merge descriptor per team.
struct WsLayout {
  size_t o, m, l, team, total;
};

WsLayout ws_layout(size_t rows, int head_dim, size_t teams) {
  WsLayout w;
  w.o = 0;
  w.m = align256(rows * head_dim * sizeof(float));
  w.l = w.m + align256(rows * sizeof(float));
  w.team = w.l + align256(rows * sizeof(float));
  w.total = w.team + align256(teams * 16);
  return w;
}

// fp32 partial rows of the workspace
size_t ws_rows(const DecodePlan& p, int num_seqs, int num_q_heads, int num_kv_heads) {
  return p.mfma ? pa::sk_slots(p.sk_blocks, num_seqs, num_kv_heads) * p.g
                : (size_t)num_seqs * num_q_heads * p.num_parts;
}

pa_status decode_supported(const pa_kv_cache* c, int num_q_heads, pa_dtype q_dtype, int* g_out) {
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads) return PA_ERR_INVALID_ARG;
  const int g = num_q_heads / c->num_kv_heads;
  // 16 only where the matrix-core path runs (checked by the callers)
  if (!(g == 1 || g == 2 || g == 4 || g == 8 || g == 16)) return PA_ERR_UNSUPPORTED;
  if (!(q_dtype == PA_F32 || q_dtype == PA_F16 || q_dtype == PA_BF16)) return PA_ERR_INVALID_ARG;
  const bool pair_ok = (c->dtype == q_dtype) || (c->dtype == PA_FP8_E4M3);
  if (!pair_ok) return PA_ERR_UNSUPPORTED;
  if (c->dtype == PA_F32) {
    if (c->head_dim != 64) return PA_ERR_UNSUPPORTED;
  } else if (!(c->head_dim == 64 || c->head_dim == 128)) {
    return PA_ERR_UNSUPPORTED;
  }
  *g_out = g;
  return PA_OK;
}

// Tokens per partition: large enough that the fp32 partial results stay a
// small fraction of the key/value bytes of a partition (about 4 * G / P /
// elem_bytes of them), small enough that long contexts still spread over
// many workgroups.
int choose_part_tokens(const pa_kv_cache* c, int g, int num_seqs, int max_ctx) {
  const int eb = elem_bytes(c->dtype);
  int p = 256;
  const int want = 256 * g / eb;
  while (p < want && p < 2048) p *= 2;
  const int64_t units = (int64_t)num_seqs * c->num_kv_heads;
  while (p > 256 && units * ((max_ctx + p - 1) / p) < 4096) p /= 2;
  // a partition may span at most PA_MAX_PART_BLOCKS table entries
  while (p / c->block_size > pa::PA_MAX_PART_BLOCKS && p > 64) p /= 2;
  return p;
}

pa_status plan_decode(const pa_kv_cache* c, int num_seqs, int num_q_heads, pa_dtype q_dtype,
                      int max_ctx, DecodePlan* plan) {
  pa_status st = check_cache(c, false);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_ctx < 0) return PA_ERR_INVALID_ARG;
  if (c->num_kv_heads > 65535 || num_q_heads > 65535) return PA_ERR_UNSUPPORTED;
  int g = 0;
  st = decode_supported(c, num_q_heads, q_dtype, &g);
  if (st != PA_OK) return st;
  plan->g = g;
  plan->mfma = pa::mfma_supported((int)c->dtype, (int)q_dtype, c->head_dim, g, num_seqs);
  if (plan->mfma) {
    // split chunk stream: partial slots for every piece that can exist, and
    // the teams' merge descriptors (at most one team per wave)
    plan->sk_blocks = pa::sk_blocks((int)c->dtype, (int)q_dtype, c->head_dim, g, num_seqs);
    plan->part_tokens = 16;
    plan->num_parts = 1;
    const size_t rows = ws_rows(*plan, num_seqs, num_q_heads, c->num_kv_heads);
    plan->ws_bytes =
        ws_layout(rows, c->head_dim, (size_t)plan->sk_blocks * 4).total;
    return PA_OK;
  }
  if (g > 8) return PA_ERR_UNSUPPORTED;                      // the VALU kernel's limit
  plan->sk_blocks = 0;
  plan->part_tokens = choose_part_tokens(c, g, num_seqs, max_ctx);
  plan->num_parts = std::max(1, (max_ctx + plan->part_tokens - 1) / plan->part_tokens);
  if (plan->num_parts > 65535) return PA_ERR_UNSUPPORTED;   // grid z limit
  if (plan->num_parts > 1) {
    plan->ws_bytes = ws_layout(ws_rows(*plan, num_seqs, num_q_heads, c->num_kv_heads),
                               c->head_dim, 0).total;
  } else {
    plan->ws_bytes = 0;
  }
  return PA_OK;
}

enum Phase { PHASE_ATTEND = 1, PHASE_MERGE = 2, PHASE_BOTH = 3 };

// Launch parameters common to every decode kernel.
DecodeParams decode_params(const pa_kv_cache* cache, int32_t layer, const void* q, void* out,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len,
                           int32_t num_seqs, int32_t num_q_heads, float scale) {
  DecodeParams a{};
  memset(&a, 0, sizeof(a));
  a.k_pool = cache->k;
  a.v_pool = cache->v;
  a.block_stride = cache->block_stride;
  a.layer_offset = (int64_t)layer * cache->layer_stride;
  a.num_blocks = cache->num_blocks;
  a.block_size = cache->block_size;
  a.log2_block_size = ilog2(cache->block_size);
  a.head_dim = cache->head_dim;
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  a.v_scale = fp8 ? cache->v_scale : 1.0f;
  const double log2e = 1.4426950408889634;
  a.qk_scale_log2 = (float)((double)scale * log2e * (fp8 ? (double)cache->k_scale : 1.0));
  a.q = q;
  a.out = out;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  return a;
}

// Shared-prefix decode: the suffix pass's pieces and merge descriptors (the
// usual decode workspace), the prefix pass's pieces (32 columns per slot),
// the plan (shared lengths, starts, slot records) and the team range of
// each prefix segment.
struct SharedLayout {
  WsLayout suf, pre;
  size_t pre_base, lcp, tot, start, desc, seg, sseg, pm, pl, po, total;
  int blocks, g;                 // resident workgroups of the launch holding both passes
};

pa_status shared_layout(const pa_kv_cache* c, int num_seqs, int num_q_heads, pa_dtype q_dtype,
                        SharedLayout* L) {
  pa_status st = check_cache(c, false);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return PA_ERR_INVALID_ARG;
  if (c->num_kv_heads > 65535 || num_q_heads > 65535) return PA_ERR_UNSUPPORTED;
  int g = 0;
  st = decode_supported(c, num_q_heads, q_dtype, &g);
  if (st != PA_OK) return st;
  if (!pa::mfma_supported((int)c->dtype, (int)q_dtype, c->head_dim, g, num_seqs) || g > 8)
    return PA_ERR_UNSUPPORTED;
  L->g = g;
  L->blocks = pa::sk_blocks_shared_dual((int)c->dtype, (int)q_dtype, c->head_dim, g, num_seqs);
  if (L->blocks < 16) return PA_ERR_UNSUPPORTED;   // both passes need a round of the XCDs
  const int H = c->num_kv_heads;
  // each pass runs on at most all of the launch's workgroups
  L->suf = ws_layout(pa::sk_slots(L->blocks, num_seqs, H) * g, c->head_dim, (size_t)L->blocks * 4);
  L->pre_base = L->suf.total;
  L->pre = ws_layout(pa::sk_slots(L->blocks, num_seqs, H) * pa::PA_PREFIX_COLS, c->head_dim,
                     (size_t)L->blocks * 4);
  const size_t S = (size_t)num_seqs;
  L->lcp = L->pre_base + L->pre.total;
  L->tot = L->lcp + align256(S * 4);
  L->start = L->tot + 256;
  L->desc = L->start + align256(S * 4);
  L->seg = L->desc + align256(S * 16);
  L->sseg = L->seg + align256(S * (size_t)H * 16);
  const size_t R = S * (size_t)num_q_heads;
  L->pm = L->sseg + align256(S * (size_t)H * 16);
  L->pl = L->pm + align256(R * 4);
  L->po = L->pl + align256(R * 4);
  L->total = L->po + align256(R * (size_t)c->head_dim * 4);
  return PA_OK;
}

// use_scratch: the workspace is the library's own `scratch` array (the
// workspace arguments are ignored); sizes that need more return
// PA_ERR_WORKSPACE before any HIP call.
pa_status decode_impl(int phases, const pa_kv_cache* cache, int32_t layer, const void* q,
                      pa_dtype q_dtype, void* out, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                      float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, bool use_scratch = false) {
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!q || !out || !context_lens || (!block_tables && max_blocks_per_seq > 0))
    return PA_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * cache->block_size < 0) return PA_ERR_INVALID_ARG;
  DecodePlan plan;
  st = plan_decode(cache, num_seqs, num_q_heads, q_dtype, max_context_len, &plan);
  if (st != PA_OK) return st;
  if (!aligned(q, 16) || !aligned(out, 4)) return PA_ERR_UNSUPPORTED;
  if (use_scratch) {
    if (plan.ws_bytes > PA_DECODE_NO_ALLOC_MAX_BYTES) return PA_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (plan.ws_bytes > 0) {
      st = scratch_of_current_device(&workspace);
      if (st != PA_OK) return st;
      workspace_bytes = PA_DECODE_NO_ALLOC_MAX_BYTES;
    }
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes || !aligned(workspace, 256))
      return PA_ERR_WORKSPACE;
  }

  DecodeParams a = decode_params(cache, layer, q, out, block_tables, max_blocks_per_seq,
                                 context_lens, max_context_len, num_seqs, num_q_heads, scale);
  a.part_tokens = plan.part_tokens;
  a.num_parts = plan.num_parts;
  a.team = plan.mfma ? pa::sk_team(cache->num_kv_heads) : 1;
  if (plan.ws_bytes > 0) {
    const size_t rows = ws_rows(plan, num_seqs, num_q_heads, cache->num_kv_heads);
    const WsLayout L = plan.mfma
        ? ws_layout(rows, cache->head_dim, (size_t)plan.sk_blocks * 4)
        : ws_layout(rows, cache->head_dim, 0);
    char* w = reinterpret_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(w + L.o);
    a.ws_m = reinterpret_cast<float*>(w + L.m);
    a.ws_l = reinterpret_cast<float*>(w + L.l);
    a.ws_team = reinterpret_cast<int32_t*>(w + L.team);

  }
  // the same launch size for both phases (a function of the call's sizes)
  const int blocks = plan.mfma ? pa::sk_launch_blocks(plan.sk_blocks, num_seqs, max_context_len,
                                                      cache->num_kv_heads)
                               : 0;
  if (phases & PHASE_ATTEND) {
    const hipError_t e =
        plan.mfma ? pa::launch_attend_mfma(a, (int)cache->dtype, (int)q_dtype, plan.g,
                                           blocks, stream)
                  : pa::launch_attend(a, (int)cache->dtype, (int)q_dtype, plan.g, stream);
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  if (phases & PHASE_MERGE) {
    if (plan.mfma) {
      if (pa::launch_merge_mfma(a, (int)q_dtype, plan.g, blocks, stream) != hipSuccess)
        return PA_ERR_HIP;
    } else if (plan.num_parts > 1) {
      if (pa::launch_merge(a, (int)q_dtype, stream) != hipSuccess) return PA_ERR_HIP;
    }
  }
  return PA_OK;
}

pa_status prefill_impl(const pa_kv_cache* cache, int32_t layer, const void* q, pa_dtype q_dtype,
                       void* out, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t max_context_len,
                       const int32_t* query_start_loc, int32_t max_query_len, int32_t num_seqs,
                       int32_t num_q_tokens, int32_t num_q_heads, float scale, hipStream_t stream) {
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_q_tokens < 0 || max_context_len < 0 || max_blocks_per_seq < 0 ||
      max_query_len < 0)
    return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads) return PA_ERR_INVALID_ARG;
  if (!(q_dtype == PA_F32 || q_dtype == PA_F16 || q_dtype == PA_BF16)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_q_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!q || !out || !context_lens || !query_start_loc || (!block_tables && max_blocks_per_seq > 0))
    return PA_ERR_INVALID_ARG;
  if (cache->num_kv_heads > 65535 || num_q_heads > 65535) return PA_ERR_UNSUPPORTED;
  const int g = num_q_heads / cache->num_kv_heads;
  if (!pa::prefill_supported((int)cache->dtype, (int)q_dtype, cache->head_dim, g))
    return PA_ERR_UNSUPPORTED;
  // one workgroup per (sequence, KV head, row tile), in a one-dimensional grid
  if (pa::prefill_grid(num_seqs, cache->num_kv_heads, pa::prefill_tiles(g, max_query_len)) > 0x7ffffff8)
    return PA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(out, 4)) return PA_ERR_UNSUPPORTED;
  pa::PrefillParams a;
  memset(&a, 0, sizeof(a));
  a.k_pool = cache->k;
  a.v_pool = cache->v;
  a.block_stride = cache->block_stride;
  a.layer_offset = (int64_t)layer * cache->layer_stride;
  a.num_blocks = cache->num_blocks;
  a.block_size = cache->block_size;
  a.log2_block_size = ilog2(cache->block_size);
  a.head_dim = cache->head_dim;
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  a.v_scale = fp8 ? cache->v_scale : 1.0f;
  const double log2e = 1.4426950408889634;
  a.qk_scale_log2 = (float)((double)scale * log2e * (fp8 ? (double)cache->k_scale : 1.0));
  a.q = q;
  a.out = out;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.query_start_loc = query_start_loc;
  a.num_q_tokens = num_q_tokens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  if (pa::launch_prefill(a, (int)cache->dtype, (int)q_dtype, g, max_query_len, stream) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

// True when K and V of a pool sit in pinned host memory that the current
// device reaches at the same addresses (hipHostMalloc memory under ROCm's
// unified addressing), so a kernel can read and write it directly.
bool host_pool_mapped(const pa_kv_cache* c) {
  void* p[2] = {c->k, c->v};
  for (void* q : p) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, q) != hipSuccess) {
      (void)hipGetLastError();   // pageable memory: not an error of this call
      return false;
    }
    if (at.type != hipMemoryTypeHost || at.devicePointer != q) return false;
  }
  return true;
}

// Launches of arg_copy_kernel over a host-side pair list, kArgCopyPairs at a
// time. Each side is described by its K and V bases and byte strides.
struct CopySide {
  char* k;
  char* v;
  int64_t block_bytes;
  int64_t layer_bytes;
};

CopySide side_of(const pa_kv_cache* c) {
  const int eb = elem_bytes(c->dtype);
  return {reinterpret_cast<char*>(c->k), reinterpret_cast<char*>(c->v), c->block_stride * eb,
          c->layer_stride * eb};
}

// pair i of the list is (src_of(i), dst_of(i))
template <typename SrcOf, typename DstOf>
pa_status launch_list_copy(const CopySide& dst, const CopySide& src, int64_t slab_bytes,
                           int32_t num_layers, int32_t n, SrcOf src_of, DstOf dst_of, int max_wgs,
                           hipStream_t stream) {
  pa::ArgCopyParams a;
  memset(&a, 0, sizeof(a));
  a.dst_k = dst.k;
  a.dst_v = dst.v;
  a.src_k = src.k;
  a.src_v = src.v;
  a.dst_block_bytes = dst.block_bytes;
  a.dst_layer_bytes = dst.layer_bytes;
  a.src_block_bytes = src.block_bytes;
  a.src_layer_bytes = src.layer_bytes;
  a.slab_bytes = slab_bytes;
  a.num_layers = num_layers;
  a.max_wgs = max_wgs;
  for (int32_t i = 0; i < n; i += pa::kArgCopyPairs) {
    const int32_t m = std::min<int32_t>(pa::kArgCopyPairs, n - i);
    a.num_pairs = m;
    for (int32_t j = 0; j < m; ++j) {
      a.pairs[2 * j] = src_of(i + j);
      a.pairs[2 * j + 1] = dst_of(i + j);
    }
    if (pa::launch_arg_copy(a, stream) != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

// grid caps: a few dozen workgroups saturate the host link; staging copies
// stay inside HBM and want the whole chip
constexpr int kHostLinkWgs = 64;
constexpr int kStagingWgs = 1024;

// Host pair list checks shared by the host-side copies: ids in range and
// destination ids distinct.
bool host_pairs_valid(const pa_kv_cache* dst, const pa_kv_cache* src, const int64_t* pairs,
                      int32_t num_pairs) {
  std::vector<int64_t> dsts(num_pairs);
  for (int i = 0; i < num_pairs; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= src->num_blocks || d < 0 || d >= dst->num_blocks) return false;
    dsts[i] = d;
  }
  std::sort(dsts.begin(), dsts.end());
  return std::adjacent_find(dsts.begin(), dsts.end()) == dsts.end();
}

bool same_shape(const pa_kv_cache* a, const pa_kv_cache* b) {
  return a->dtype == b->dtype && a->num_layers == b->num_layers &&
         a->num_kv_heads == b->num_kv_heads && a->block_size == b->block_size &&
         a->head_dim == b->head_dim;
}

}  // namespace

extern "C" {

pa_status pa_write_kv(const pa_kv_cache* cache, int32_t layer, const void* k, const void* v,
                      pa_dtype src_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                      hipStream_t stream) {
  if (!valid_dtype(raw(src_dtype))) return PA_ERR_INVALID_ARG;
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers) return PA_ERR_INVALID_ARG;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  const bool conv = src_dtype != cache->dtype;
  if (conv && !(cache->dtype == PA_FP8_E4M3 && src_dtype != PA_FP8_E4M3)) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16)) return PA_ERR_UNSUPPORTED;
  if (((int64_t)cache->head_dim * elem_bytes(src_dtype)) % 16) return PA_ERR_UNSUPPORTED;
  pa::WriteParams a;
  memset(&a, 0, sizeof(a));
  a.k_pool = cache->k;
  a.v_pool = cache->v;
  a.block_stride = cache->block_stride;
  a.layer_offset = (int64_t)layer * cache->layer_stride;
  a.num_blocks = cache->num_blocks;
  a.block_size = cache->block_size;
  a.log2_block_size = ilog2(cache->block_size);
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.k_src = k;
  a.v_src = v;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  if (pa::launch_write(a, (int)src_dtype, (int)cache->dtype, stream) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

size_t pa_decode_workspace_size(const pa_kv_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                int32_t max_context_len) {
  // the largest need over the query dtypes a pool of this dtype accepts
  if (!cache) return 0;
  size_t best = 0;
  const pa_dtype qs[3] = {PA_F32, PA_F16, PA_BF16};
  for (pa_dtype qd : qs) {
    DecodePlan plan;
    if (plan_decode(cache, num_seqs, num_q_heads, qd, max_context_len, &plan) == PA_OK)
      best = std::max(best, plan.ws_bytes);
  }
  return best;
}

int32_t pa_decode_partition_tokens(const pa_kv_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_context_len) {
  DecodePlan plan;
  if (!cache || check_cache(cache, false) != PA_OK) return 0;
  pa_dtype qd = cache->dtype == PA_FP8_E4M3 ? PA_BF16 : cache->dtype;
  if (plan_decode(cache, num_seqs, num_q_heads, qd, max_context_len, &plan) != PA_OK) return 0;
  return plan.part_tokens;
}

pa_status pa_prefill(const pa_kv_cache* cache, int32_t layer, const void* q, pa_dtype q_dtype,
                     void* out, const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len,
                     const int32_t* query_start_loc, int32_t max_query_len, int32_t num_seqs,
                     int32_t num_q_tokens, int32_t num_q_heads, float scale, hipStream_t stream) {
  if (!valid_q_dtype(q_dtype)) return PA_ERR_INVALID_ARG;
  return prefill_impl(cache, layer, q, q_dtype, out, block_tables, max_blocks_per_seq, context_lens,
                      max_context_len, query_start_loc, max_query_len, num_seqs, num_q_tokens,
                      num_q_heads, scale, stream);
}

pa_status pa_decode(const pa_kv_cache* cache, int32_t layer, const void* q, pa_dtype q_dtype,
                    void* out, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                    int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  if (!valid_q_dtype(q_dtype)) return PA_ERR_INVALID_ARG;
  return decode_impl(PHASE_BOTH, cache, layer, q, q_dtype, out, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, num_seqs, num_q_heads, scale, workspace,
                     workspace_bytes, stream);
}

pa_status pa_decode_no_alloc(const pa_kv_cache* cache, int32_t layer, const void* q,
                             pa_dtype q_dtype, void* out, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                             float scale, hipStream_t stream) {
  if (!valid_q_dtype(q_dtype)) return PA_ERR_INVALID_ARG;
  return decode_impl(PHASE_BOTH, cache, layer, q, q_dtype, out, block_tables, max_blocks_per_seq,
                     context_lens, max_context_len, num_seqs, num_q_heads, scale, nullptr, 0,
                     stream, true);
}

pa_status pa_decode_shared(const pa_kv_cache* cache, int32_t layer, const void* q,
                           pa_dtype q_dtype, void* out, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                           float scale, int32_t reuse_plan, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!valid_q_dtype(q_dtype)) return PA_ERR_INVALID_ARG;
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (layer < 0 || layer >= cache->num_layers) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale) || (reuse_plan != 0 && reuse_plan != 1)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!q || !out || !context_lens || (!block_tables && max_blocks_per_seq > 0))
    return PA_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * cache->block_size < 0) return PA_ERR_INVALID_ARG;
  SharedLayout L;
  st = shared_layout(cache, num_seqs, num_q_heads, q_dtype, &L);
  if (st != PA_OK) return st;
  if (!aligned(q, 16) || !aligned(out, 4)) return PA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256)) return PA_ERR_WORKSPACE;

  DecodeParams a = decode_params(cache, layer, q, out, block_tables, max_blocks_per_seq,
                                 context_lens, max_context_len, num_seqs, num_q_heads, scale);
  a.part_tokens = 16;
  a.num_parts = 1;
  a.team = pa::sk_team(cache->num_kv_heads);
  char* w = reinterpret_cast<char*>(workspace);
  a.share_lcp = reinterpret_cast<int32_t*>(w + L.lcp);
  a.share_start = reinterpret_cast<int32_t*>(w + L.start);
  a.share_desc = reinterpret_cast<int32_t*>(w + L.desc);
  a.share_seg = reinterpret_cast<int32_t*>(w + L.seg);
  a.suf_seg = reinterpret_cast<int32_t*>(w + L.sseg);
  a.share_tot = reinterpret_cast<int32_t*>(w + L.tot);
  a.pre_m = reinterpret_cast<float*>(w + L.pm);
  a.pre_l = reinterpret_cast<float*>(w + L.pl);
  a.pre_o = reinterpret_cast<float*>(w + L.po);
  // One launch runs both passes side by side (the kernel splits its
  // workgroups between them from the plan, see attend_sk_dual_kernel): all
  // the resident workgroups, or fewer for small batches as in the plain
  // decode, and never under two rounds of the XCDs.
  const int blocks = std::max(
      16, pa::sk_launch_blocks(L.blocks, num_seqs, max_context_len, cache->num_kv_heads));
  a.pre_teams = a.suf_teams = blocks * 4 / a.team;
  const int kv = (int)cache->dtype, qt = (int)q_dtype;
  if (!reuse_plan && pa::launch_share_plan(a, L.g, stream) != hipSuccess) return PA_ERR_HIP;
  // the prefix pass's pieces and the suffix pass's, each in its own region
  char* wp = w + L.pre_base;
  DecodeParams pre = a, suf = a;
  pre.ws_o = reinterpret_cast<float*>(wp + L.pre.o);
  pre.ws_m = reinterpret_cast<float*>(wp + L.pre.m);
  pre.ws_l = reinterpret_cast<float*>(wp + L.pre.l);
  pre.ws_team = reinterpret_cast<int32_t*>(wp + L.pre.team);
  suf.ws_o = reinterpret_cast<float*>(w + L.suf.o);
  suf.ws_m = reinterpret_cast<float*>(w + L.suf.m);
  suf.ws_l = reinterpret_cast<float*>(w + L.suf.l);
  suf.ws_team = reinterpret_cast<int32_t*>(w + L.suf.team);
  if (pa::launch_attend_shared_dual(pre, suf, kv, qt, L.g, blocks, stream) != hipSuccess)
    return PA_ERR_HIP;
  // every row the suffix pass left open: its pieces (or own partial) and,
  // with a prefix, the prefix pieces, combined
  DecodeParams fin = suf;
  fin.pre_ws_o = pre.ws_o;
  fin.pre_ws_m = pre.ws_m;
  fin.pre_ws_l = pre.ws_l;
  if (pa::launch_shared_combine(fin, qt, L.g, stream) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

size_t pa_decode_shared_workspace_size(const pa_kv_cache* cache, int32_t num_seqs,
                                       int32_t num_q_heads) {
  if (!cache) return 0;
  size_t best = 0;
  const pa_dtype qs[2] = {PA_F16, PA_BF16};
  for (pa_dtype qd : qs) {
    SharedLayout L;
    if (shared_layout(cache, num_seqs, num_q_heads, qd, &L) == PA_OK) best = std::max(best, L.total);
  }
  return best;
}

pa_status pa_decode_attend(const pa_kv_cache* cache, int32_t layer, const void* q,
                           pa_dtype q_dtype, void* out, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                           float scale, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (!valid_q_dtype(q_dtype)) return PA_ERR_INVALID_ARG;
  return decode_impl(PHASE_ATTEND, cache, layer, q, q_dtype, out, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                     scale, workspace, workspace_bytes, stream);
}

pa_status pa_decode_merge(const pa_kv_cache* cache, int32_t layer, const void* q,
                          pa_dtype q_dtype, void* out, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                          float scale, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!valid_q_dtype(q_dtype)) return PA_ERR_INVALID_ARG;
  return decode_impl(PHASE_MERGE, cache, layer, q, q_dtype, out, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                     scale, workspace, workspace_bytes, stream);
}

pa_status pa_copy_blocks(const pa_kv_cache* dst, const pa_kv_cache* src, const int64_t* pairs,
                         int32_t num_pairs, pa_copy_dir dir, hipStream_t stream) {
  const int d = raw(dir);
  if (!(d == PA_COPY_D2D || d == PA_COPY_H2D || d == PA_COPY_D2H || d == PA_COPY_H2D_KERNEL ||
        d == PA_COPY_D2H_KERNEL))
    return PA_ERR_INVALID_ARG;
  pa_status st = check_cache(dst, true);
  if (st != PA_OK) return st;
  st = check_cache(src, true);
  if (st != PA_OK) return st;
  if (!same_shape(dst, src)) return PA_ERR_INVALID_ARG;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (!(dir == PA_COPY_D2D || dir == PA_COPY_H2D || dir == PA_COPY_D2H ||
        dir == PA_COPY_H2D_KERNEL || dir == PA_COPY_D2H_KERNEL))
    return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!pairs) return PA_ERR_INVALID_ARG;
  const int eb = elem_bytes(dst->dtype);
  const int64_t slab = (int64_t)dst->num_kv_heads * dst->block_size * dst->head_dim * eb;

  if (dir == PA_COPY_D2D) {
    pa::CopyParams a;
    memset(&a, 0, sizeof(a));
    a.dst_k = reinterpret_cast<char*>(dst->k);
    a.dst_v = reinterpret_cast<char*>(dst->v);
    a.src_k = reinterpret_cast<const char*>(src->k);
    a.src_v = reinterpret_cast<const char*>(src->v);
    a.dst_block_bytes = dst->block_stride * eb;
    a.dst_layer_bytes = dst->layer_stride * eb;
    a.src_block_bytes = src->block_stride * eb;
    a.src_layer_bytes = src->layer_stride * eb;
    a.slab_bytes = slab;
    a.dst_num_blocks = dst->num_blocks;
    a.src_num_blocks = src->num_blocks;
    a.num_layers = dst->num_layers;
    a.pairs = pairs;
    a.num_pairs = num_pairs;
    if (dst->num_layers > 32767) return PA_ERR_UNSUPPORTED;
    if (pa::launch_copy(a, stream) != hipSuccess) return PA_ERR_HIP;
    return PA_OK;
  }

  // host pairs: validate everything before the first copy
  if (!host_pairs_valid(dst, src, pairs, num_pairs)) return PA_ERR_INVALID_ARG;

  const bool to_dev = dir == PA_COPY_H2D || dir == PA_COPY_H2D_KERNEL;
  if (dir == PA_COPY_H2D_KERNEL || dir == PA_COPY_D2H_KERNEL) {
    if (dst->num_layers > 32767 || !host_pool_mapped(to_dev ? src : dst)) return PA_ERR_UNSUPPORTED;
    return launch_list_copy(
        side_of(dst), side_of(src), slab, dst->num_layers, num_pairs,
        [&](int32_t i) { return pairs[2 * i]; }, [&](int32_t i) { return pairs[2 * i + 1]; },
        kHostLinkWgs, stream);
  }

  const hipMemcpyKind kind = to_dev ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  const int L = dst->num_layers;
  const int64_t block_bytes = slab * L;
  // a block is one contiguous range when its layers sit back to back; runs of
  // consecutive ids are one range when blocks are packed back to back too
  const bool dst_contig = L == 1 || dst->layer_stride * eb == slab;
  const bool src_contig = L == 1 || src->layer_stride * eb == slab;
  const bool packed = dst_contig && src_contig && dst->block_stride * eb == block_bytes &&
                      src->block_stride * eb == block_bytes;
  int i = 0;
  while (i < num_pairs) {
    const int64_t s0 = pairs[2 * i], d0 = pairs[2 * i + 1];
    int run = 1;
    if (packed) {
      while (i + run < num_pairs && pairs[2 * (i + run)] == s0 + run &&
             pairs[2 * (i + run) + 1] == d0 + run)
        ++run;
    }
    for (int kvsel = 0; kvsel < 2; ++kvsel) {
      const char* sb = reinterpret_cast<const char*>(kvsel ? src->v : src->k);
      char* db = reinterpret_cast<char*>(kvsel ? dst->v : dst->k);
      if (dst_contig && src_contig) {
        if (hipMemcpyAsync(db + d0 * dst->block_stride * eb, sb + s0 * src->block_stride * eb,
                           (size_t)run * (size_t)block_bytes, kind, stream) != hipSuccess)
          return PA_ERR_HIP;
        continue;
      }
      for (int l = 0; l < L; ++l)
        if (hipMemcpyAsync(db + d0 * dst->block_stride * eb + l * dst->layer_stride * eb,
                           sb + s0 * src->block_stride * eb + l * src->layer_stride * eb,
                           (size_t)slab, kind, stream) != hipSuccess)
          return PA_ERR_HIP;
    }
    i += run;
  }
  return PA_OK;
}

pa_status pa_copy_blocks_staged(const pa_kv_cache* dst, const pa_kv_cache* src,
                                const int64_t* pairs, int32_t num_pairs, pa_copy_dir dir,
                                void* staging, size_t staging_bytes, hipStream_t stream) {
  if (!(raw(dir) == PA_COPY_H2D || raw(dir) == PA_COPY_D2H)) return PA_ERR_INVALID_ARG;
  pa_status st = check_cache(dst, true);
  if (st != PA_OK) return st;
  st = check_cache(src, true);
  if (st != PA_OK) return st;
  if (!same_shape(dst, src)) return PA_ERR_INVALID_ARG;
  if (num_pairs < 0 || !(dir == PA_COPY_H2D || dir == PA_COPY_D2H)) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!pairs || !staging) return PA_ERR_INVALID_ARG;
  if (!aligned(staging, 16)) return PA_ERR_UNSUPPORTED;
  const bool to_dev = dir == PA_COPY_H2D;
  const pa_kv_cache* host = to_dev ? src : dst;
  const int eb = elem_bytes(dst->dtype);
  const int L = dst->num_layers;
  const int64_t slab = (int64_t)dst->num_kv_heads * dst->block_size * dst->head_dim * eb;
  const int64_t blk = slab * L;                       // one block's K (or V), every layer
  if (L > 1 && host->layer_stride * eb != slab) return PA_ERR_UNSUPPORTED;
  if (L > 32767) return PA_ERR_UNSUPPORTED;
  const int64_t cap64 = (int64_t)(staging_bytes / (size_t)(2 * blk));
  if (cap64 < 1) return PA_ERR_WORKSPACE;
  if (!host_pairs_valid(dst, src, pairs, num_pairs)) return PA_ERR_INVALID_ARG;

  const int32_t cap = (int32_t)std::min<int64_t>(cap64, num_pairs);
  char* sk = static_cast<char*>(staging);
  const CopySide stage = {sk, sk + (int64_t)cap * blk, blk, slab};
  const CopySide hs = side_of(host);
  const bool packed = host->num_blocks == 1 || hs.block_bytes == blk;
  const hipMemcpyKind kind = to_dev ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  for (int32_t c = 0; c < num_pairs; c += cap) {
    const int32_t m = std::min<int32_t>(cap, num_pairs - c);
    const int64_t* pc = pairs + 2 * (int64_t)c;
    if (!to_dev) {   // gather the device blocks into staging slots 0..m-1
      st = launch_list_copy(
          stage, side_of(src), slab, L, m, [&](int32_t i) { return pc[2 * i]; },
          [&](int32_t i) { return (int64_t)i; }, kStagingWgs, stream);
      if (st != PA_OK) return st;
    }
    // one DMA transfer per run of consecutive host ids, for K and for V
    for (int32_t i = 0; i < m;) {
      const int64_t h0 = pc[2 * i + (to_dev ? 0 : 1)];
      int32_t run = 1;
      while (packed && i + run < m && pc[2 * (i + run) + (to_dev ? 0 : 1)] == h0 + run) ++run;
      for (int kv = 0; kv < 2; ++kv) {
        char* hp = (kv ? hs.v : hs.k) + h0 * hs.block_bytes;
        char* sp = (kv ? stage.v : stage.k) + (int64_t)i * blk;
        if (hipMemcpyAsync(to_dev ? sp : hp, to_dev ? hp : sp, (size_t)run * (size_t)blk, kind,
                           stream) != hipSuccess)
          return PA_ERR_HIP;
      }
      i += run;
    }
    if (to_dev) {    // scatter staging slots 0..m-1 into the device blocks
      st = launch_list_copy(
          side_of(dst), stage, slab, L, m, [&](int32_t i) { return (int64_t)i; },
          [&](int32_t i) { return pc[2 * i + 1]; }, kStagingWgs, stream);
      if (st != PA_OK) return st;
    }
  }
  return PA_OK;
}

size_t pa_copy_staging_size(const pa_kv_cache* pool, int32_t num_pairs) {
  if (check_cache(pool, false) != PA_OK || num_pairs <= 0) return 0;
  return (size_t)num_pairs * 2 * (size_t)pool->num_layers * (size_t)pool->num_kv_heads *
         (size_t)pool->block_size * (size_t)pool->head_dim * (size_t)elem_bytes(pool->dtype);
}

int32_t pa_host_pool_mapped(const pa_kv_cache* pool) {
  if (check_cache(pool, true) != PA_OK) return 0;
  return host_pool_mapped(pool) ? 1 : 0;
}

const char* pa_status_string(pa_status s) {
  switch (raw(s)) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: unsupported size, dtype or alignment";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP launch or copy failed";
    case PA_ERR_NO_SPACE: return "PA_ERR_NO_SPACE: not enough free blocks";
  }
  return "unknown pa_status";
}

const char* pa_version(void) { return "0.1.0"; }

}  // extern "C"
