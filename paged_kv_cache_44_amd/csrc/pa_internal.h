// pa_internal.h — launch parameters shared between the C-ABI layer and the
// kernels. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Largest number of block-table entries one decode partition may span.
constexpr int PA_MAX_PART_BLOCKS = 1024;
// Largest batch the evenly split matrix-core decode takes (its per-workgroup
// chunk prefix sums live in LDS).
constexpr int PA_SK_MAX_SEQS = 8192;
// Query columns of a shared-prefix slot in the prefix pass: two 16-column
// matrix-core tiles, so a slot holds up to 32 / G sequences.
constexpr int PA_PREFIX_COLS = 32;

struct DecodeParams {
  const void* k_pool;
  const void* v_pool;
  int64_t block_stride;      // elements
  int64_t layer_offset;      // elements: layer * layer_stride
  int32_t num_blocks;
  int32_t block_size;
  int32_t log2_block_size;
  int32_t head_dim;
  float v_scale;             // applied to the output (1 unless FP8)
  float qk_scale_log2;       // scale * log2(e) (* k_scale for FP8)
  const void* q;
  void* out;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t part_tokens;       // tokens per partition
  int32_t num_parts;         // partitions per sequence in the launch grid
  float* ws_o;               // [num_seqs][num_q_heads][num_parts][head_dim]
  float* ws_m;               // [num_seqs][num_q_heads][num_parts]
  float* ws_l;               // [num_seqs][num_q_heads][num_parts]
  int32_t team;              // matrix-core path: waves per team (KV heads per head group)
  int32_t* ws_team;          // matrix-core path: merge descriptors, int4 per team
  // shared-prefix decode (matrix-core path only)
  int32_t* share_lcp;        // [num_seqs] tokens sequence s shares with s - 1 (from the tables)
  int32_t* share_start;      // [num_seqs] tokens of the shared prefix each sequence starts after
  int32_t* share_desc;       // [num_seqs] int4 {slot, members, prefix tokens, 0}: members and
                             // prefix are nonzero only at a slot's own index
  int32_t* share_seg;        // [num_seqs * head groups] int4 {first team, last team, Cc, teams}
                             // of each prefix segment, written by the prefix pass
  int32_t* suf_seg;          // the same for each suffix segment, written by the suffix pass
  int32_t* share_tot;        // [2] from the plan: prefix chunks of all slots, own chunks of all
                             // sequences (the split of the launch that runs both passes)
  int32_t suf_teams;         // most teams the suffix pass can have (records carry the count)
  const float* pre_ws_o;     // the prefix pass's pieces (its ws_o, ws_m, ws_l), combined
  const float* pre_ws_m;     // per sequence and head with the suffix pass's result
  const float* pre_ws_l;
  int32_t pre_teams;         // most teams the prefix pass can have (records carry the count)
  float* pre_m;              // [num_seqs][num_q_heads] partials of a prefixed sequence's own
  float* pre_l;              // tokens (after its shared prefix): running max (log2), sum of
  float* pre_o;              // weights, [head_dim] unnormalised output
};

struct PrefillParams {
  const void* k_pool;
  const void* v_pool;
  int64_t block_stride;      // elements
  int64_t layer_offset;      // elements: layer * layer_stride
  int32_t num_blocks;
  int32_t block_size;
  int32_t log2_block_size;
  int32_t head_dim;
  float v_scale;             // applied to the output (1 unless FP8)
  float qk_scale_log2;       // scale * log2(e) (* k_scale for FP8)
  const void* q;             // [num_q_tokens][num_q_heads][head_dim]
  void* out;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;
  const int32_t* query_start_loc;   // [num_seqs + 1]
  int32_t row_tiles;                // workgroups per (sequence, KV head) along the query rows
  int32_t num_q_tokens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
};

struct WriteParams {
  void* k_pool;
  void* v_pool;
  int64_t block_stride;
  int64_t layer_offset;
  int32_t num_blocks;
  int32_t block_size;
  int32_t log2_block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  float k_scale;
  float v_scale;
  const void* k_src;
  const void* v_src;
  const int64_t* slot_mapping;
  int32_t num_tokens;
};

struct CopyParams {
  char* dst_k;
  char* dst_v;
  const char* src_k;
  const char* src_v;
  int64_t dst_block_bytes;   // block stride in bytes
  int64_t dst_layer_bytes;   // layer stride in bytes
  int64_t src_block_bytes;
  int64_t src_layer_bytes;
  int64_t slab_bytes;        // bytes of one (block, layer): heads * slots * dim
  int32_t dst_num_blocks;
  int32_t src_num_blocks;
  int32_t num_layers;
  const int64_t* pairs;      // device [num_pairs][2]
  int32_t num_pairs;
};

// Block copies whose pairs travel in the kernel arguments (kArgCopyPairs
// per launch): between device memory and pinned, device-mapped host memory,
// and between device pools and a staging buffer. max_wgs caps the grid.
constexpr int kArgCopyPairs = 64;
struct ArgCopyParams {
  char* dst_k;
  char* dst_v;
  const char* src_k;
  const char* src_v;
  int64_t dst_block_bytes;
  int64_t dst_layer_bytes;
  int64_t src_block_bytes;
  int64_t src_layer_bytes;
  int64_t slab_bytes;
  int32_t num_layers;
  int32_t num_pairs;         // <= kArgCopyPairs
  int32_t max_wgs;
  int64_t pairs[2 * kArgCopyPairs];
};

hipError_t launch_attend(const DecodeParams& a, int kv_ty, int q_ty, int g, hipStream_t st);
hipError_t launch_merge(const DecodeParams& a, int q_ty, hipStream_t st);
bool mfma_supported(int kv_ty, int q_ty, int head_dim, int g, int num_seqs);
int sk_blocks(int kv_ty, int q_ty, int head_dim, int g, int num_seqs);
int sk_launch_blocks(int blocks_max, int num_seqs, int max_ctx, int num_kv_heads);
size_t sk_slots(int blocks, int num_seqs, int num_kv_heads);
int sk_team(int num_kv_heads);
hipError_t launch_attend_mfma(const DecodeParams& a, int kv_ty, int q_ty, int g, int blocks,
                              hipStream_t st);
hipError_t launch_merge_mfma(const DecodeParams& a, int q_ty, int g, int blocks, hipStream_t st);
// shared-prefix decode: planning (fills share_lcp, share_start, share_desc);
// the prefix (mode 1) and suffix (mode 2) passes in one launch; the combine
// of every row that is not finished by the suffix pass (cut segments, and
// every sequence with a prefix)
hipError_t launch_share_plan(const DecodeParams& a, int g, hipStream_t st);
int sk_blocks_shared_dual(int kv_ty, int q_ty, int head_dim, int g, int num_seqs);
hipError_t launch_attend_shared_dual(const DecodeParams& pre, const DecodeParams& suf, int kv_ty,
                                     int q_ty, int g, int blocks, hipStream_t st);
hipError_t launch_shared_combine(const DecodeParams& a, int q_ty, int g, hipStream_t st);
bool prefill_supported(int kv_ty, int q_ty, int head_dim, int g);
int prefill_tiles(int g, int max_query_len);
int64_t prefill_grid(int num_seqs, int num_kv_heads, int tiles);
hipError_t launch_prefill(const PrefillParams& a, int kv_ty, int q_ty, int g, int max_query_len,
                          hipStream_t st);
hipError_t launch_write(const WriteParams& a, int src_ty, int dst_ty, hipStream_t st);
hipError_t launch_copy(const CopyParams& a, hipStream_t st);
hipError_t launch_arg_copy(const ArgCopyParams& a, hipStream_t st);

}  // namespace pa
