/*
 * pa.h — C ABI of the paged KV-cache library (MI355X / gfx950).
 *
 * Three operations on a paged KV cache, as described in the pages on
 * PagedAttention:
 *
 *   pa_write_kv     slot-mapped writes of new keys/values into the block pool
 *                   ("When KV Capacity Runs Out", Figure 2: the KV of position
 *                   8 lands in the first slot of the newly attached block;
 *                   "Efficient Memory Management for Large Language Model
 *                   Serving with PagedAttention" (summary page), block-table
 *                   paragraph: logical blocks fill left to right).
 *   pa_decode       one decode query per sequence attending over the keys and
 *                   values of its context, fetched block by block through the
 *                   block table (same summary page, kernel paragraph: the
 *                   result is identical to ordinary attention; "Continuous
 *                   Batching and PagedAttention", section "The block table is
 *                   a page table").
 *   pa_prefill      causal attention of each sequence's newest positions over
 *                   its paged keys and values: prefill, chunked prefill, and
 *                   the prefill pass that recomputes a preempted request
 *                   ("When KV Capacity Runs Out", section "Recompute KV from
 *                   token history").
 *   pa_copy_blocks  whole-block copies: copy-on-write of a shared block inside
 *                   device memory (summary page, sampling and prefix
 *                   paragraphs) and swap between device and pinned host memory
 *                   ("When KV Capacity Runs Out", section "Restore KV stored
 *                   outside the GPU", Figure 4).
 *
 * Conventions shared by every call
 *  - Ownership: the caller owns every buffer (pools, tables, workspace). The
 *    library never allocates, never frees, never synchronises the host and
 *    keeps no pointer after a call returns. It holds no global state and is
 *    reentrant, except for pa_decode_no_alloc's fixed device array (see
 *    there).
 *  - Streams: all device work is enqueued on the caller's `stream` and is
 *    asynchronous with respect to the host; stream order gives the ordering
 *    between calls (e.g. a swap-out copy finishes before a later write that
 *    reuses the released block, as "Restore KV stored outside the GPU"
 *    requires).
 *  - Errors: argument problems that the host can see (null pointers, shapes,
 *    dtype combinations, unsupported sizes, a too-small workspace, host-side
 *    copy pairs) are reported before any HIP call is made and leave every
 *    buffer untouched. Launch failures return PA_ERR_HIP.
 *  - Alignment: pool base pointers, q and pa_write_kv's sources 16-byte,
 *    out 4-byte, workspaces 256-byte aligned; a misaligned pointer gives
 *    PA_ERR_UNSUPPORTED.
 *  - Bad values inside device arrays never cause an out-of-bounds access:
 *      * pa_write_kv skips a token whose slot lies beyond the pool;
 *      * pa_decode writes a NaN output row for a sequence whose context
 *        length is negative, exceeds max_context_len or max_blocks_per_seq *
 *        block_size, or whose block table names a block outside the pool;
 *      * pa_copy_blocks (device pairs) skips a pair naming a block outside
 *        either pool.
 *
 * Pool layout (one pool for K and one for V, same geometry)
 *   Element (layer l, block b, kv head h, slot o, dim d) lives at element index
 *       b * block_stride + l * layer_stride + (h * block_size + o) * head_dim + d
 *   Blocks are fixed-size and may sit anywhere in the pool ("Continuous
 *   Batching and PagedAttention", section "Fixed-size blocks make every free
 *   block usable"). The default, block-major layout has
 *       layer_stride = num_kv_heads * block_size * head_dim,
 *       block_stride = num_layers * layer_stride,
 *   so all layers of one block are one contiguous range, which makes a swap
 *   of a block a single transfer ("KV Cache Preemption in vLLM", section
 *   "Swap versus recompute", notes that a block's data spans every layer).
 *   A layer-major layout (one array of blocks per layer: block_stride = the
 *   slab, layer_stride >= num_blocks * slab) is accepted too. Either way no
 *   two (block, layer) slabs may overlap, else PA_ERR_INVALID_ARG.
 *   Positions are 0-based: token t of a sequence lives in logical block
 *   t / block_size at slot t % block_size ("When KV Capacity Runs Out",
 *   section "Running out of KV space during generation": positions count
 *   from 0).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, bad dtype combination   */
  PA_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (e.g. head_dim)  */
  PA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required  */
  PA_ERR_HIP = 4,         /* a HIP launch or copy call failed                 */
  PA_ERR_NO_SPACE = 5     /* block manager: not enough free blocks (nothing    */
                          /* was changed)                                      */
} pa_status;

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  /* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals
     m * 2^-9; largest finite 448 (0x7E); 0x7F / 0xFF are NaN; no infinity.
     The pages mention an FP8 KV cache only as a capacity lever ("KV Cache
     Preemption in vLLM", sections "How much KV cache a token costs" and "A
     worked example"); this format is the reading adopted for it. */
  PA_FP8_E4M3 = 3
} pa_dtype;

/* One KV pool: K and V tensors of identical geometry, in device memory or in
 * pinned host memory (host pools are only valid as a side of an H2D / D2H
 * pa_copy_blocks call). */
typedef struct {
  void* k;                /* K elements, layout above                           */
  void* v;                /* V elements, layout above                           */
  pa_dtype dtype;         /* storage type of both tensors                       */
  int32_t num_blocks;     /* physical blocks in the pool                        */
  int32_t num_layers;     /* layers held per block (>= 1)                       */
  int32_t num_kv_heads;   /* KV heads per layer                                 */
  int32_t block_size;     /* token slots per block: power of two, 1..256        */
  int32_t head_dim;       /* elements per head vector                           */
  int64_t block_stride;   /* elements between consecutive blocks               */
  int64_t layer_stride;   /* elements between consecutive layers of one block  */
  float k_scale;          /* FP8 only: value = code * k_scale (> 0, finite);    */
  float v_scale;          /*   must be exactly 1.0f for the other dtypes        */
} pa_kv_cache;

/* ------------------------------------------------------------------------ */
/* pa_write_kv — store the keys and values of num_tokens new tokens.         */
/*                                                                           */
/* For token i with slot_mapping[i] >= 0, block = slot / block_size and      */
/* offset = slot % block_size; K[i][h][:] and V[i][h][:] are stored at       */
/* (layer, block, h, offset, :) for every KV head h. Tokens with a negative  */
/* slot are skipped (padding). ("When KV Capacity Runs Out", Figure 2 and    */
/* section "Restore KV stored outside the GPU": the new position's KV is     */
/* written into the next free slot of the sequence's last block.)            */
/*                                                                           */
/*  k, v         device, [num_tokens][num_kv_heads][head_dim], dense, of     */
/*               src_dtype. src_dtype must equal cache->dtype, or, when the  */
/*               cache is PA_FP8_E4M3, be PA_F32 / PA_F16 / PA_BF16.         */
/*  slot_mapping device int64 [num_tokens]. Non-negative slots must be       */
/*               distinct within one call (undefined result otherwise); a    */
/*               slot >= num_blocks * block_size is skipped.                 */
/*  Same dtype: the stored bytes equal the source bytes.                     */
/*  FP8: code = RNE_e4m3(clamp(fp32(x) / scale, -448, 448)) with an IEEE     */
/*  correctly rounded fp32 division (scale = k_scale or v_scale); a NaN      */
/*  input gives the NaN code with the input's sign; -0 stays -0.             */
/*  num_tokens == 0 is a no-op.                                              */
/* ------------------------------------------------------------------------ */
pa_status pa_write_kv(const pa_kv_cache* cache, int32_t layer, const void* k,
                      const void* v, pa_dtype src_dtype,
                      const int64_t* slot_mapping, int32_t num_tokens,
                      hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* pa_decode — paged attention for one query token per sequence.             */
/*                                                                           */
/* For sequence s with n = context_lens[s] and query head h (group size      */
/* g = num_q_heads / num_kv_heads, KV head kvh = h / g):                     */
/*   z_t  = scale * <q[s][h], K[t][kvh]>,            t = 0 .. n-1            */
/*   out[s][h] = sum_t softmax(z)_t * V[t][kvh]                              */
/* where token t is read from block block_tables[s][t / block_size], slot    */
/* t % block_size ("Efficient Memory Management for Large Language Model     */
/* Serving with PagedAttention", kernel paragraph: fetch each block wherever */
/* it lives, score the query against it, combine with its values; the       */
/* result is that of ordinary attention). n counts the token written by  */
/* this step's pa_write_kv. n == 0 gives a zero output row. FP8 pools are    */
/* dequantised as code * k_scale / v_scale. No mask beyond the context      */
/* length is applied (the query is the last position).                       */
/*                                                                           */
/*  q, out        device, [num_seqs][num_q_heads][head_dim], dense, q_dtype  */
/*                (PA_F32, PA_F16 or PA_BF16); out has the same dtype and is */
/*                rounded to nearest-even from fp32 accumulation.            */
/*  block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries at    */
/*                index >= ceil(n / block_size) are never read.              */
/*  context_lens  device int32 [num_seqs], each in [0, max_context_len].     */
/*  max_context_len  host upper bound on context_lens; sizes the launch.     */
/*  workspace     device scratch of >= pa_decode_workspace_size(...) bytes,  */
/*                256-byte aligned; contents need no initialisation.         */
/* Supported today: head_dim 64 or 128 (PA_F32 pools: 64 only);             */
/* num_q_heads / num_kv_heads in {1, 2, 4, 8}, and 16 with PA_F16, PA_BF16   */
/* or PA_FP8_E4M3 pools and 16-bit queries for up to 8192 sequences; q_dtype */
/* equal to the pool dtype, or any of the three with a PA_FP8_E4M3 pool.     */
/* Others return PA_ERR_UNSUPPORTED.                                         */
/*                                                                           */
/* pa_decode is exactly pa_decode_attend followed by pa_decode_merge with    */
/* the same arguments. The split lets a caller time or schedule the two      */
/* launches separately; pa_decode_merge must follow pa_decode_attend on the  */
/* same stream with unchanged inputs and workspace (num_seqs and             */
/* max_context_len also set how many workgroups both launch: a merge given   */
/* other values gives undefined output rows, though it stays in bounds).     */
/* ------------------------------------------------------------------------ */
pa_status pa_decode(const pa_kv_cache* cache, int32_t layer, const void* q,
                    pa_dtype q_dtype, void* out, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t max_context_len, int32_t num_seqs,
                    int32_t num_q_heads, float scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* Phase 1: attention over each context partition. Writes out[s] directly    */
/* for sequences that fit one partition, partial results into workspace for  */
/* the others.                                                               */
pa_status pa_decode_attend(const pa_kv_cache* cache, int32_t layer,
                           const void* q, pa_dtype q_dtype, void* out,
                           const int32_t* block_tables,
                           int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len,
                           int32_t num_seqs, int32_t num_q_heads, float scale,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Phase 2: merge the partition partials of multi-partition sequences:       */
/* M = max_p m_p;  out = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p.      */
pa_status pa_decode_merge(const pa_kv_cache* cache, int32_t layer,
                          const void* q, pa_dtype q_dtype, void* out,
                          const int32_t* block_tables,
                          int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len,
                          int32_t num_seqs, int32_t num_q_heads, float scale,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Granularity at which pa_decode may split one sequence's context between  */
/* work units for these sizes: the partition length of the VALU kernel     */
/* (fp32 pools, fp32 queries), or 16 for the matrix-core kernel, which      */
/* splits the total work into equal runs of 16-token chunks per wave. 0 if  */
/* the arguments are invalid. Informational; callers need not use it.       */
int32_t pa_decode_partition_tokens(const pa_kv_cache* cache, int32_t num_seqs,
                                   int32_t num_q_heads,
                                   int32_t max_context_len);

/* Workspace bytes pa_decode needs for these sizes with any query dtype the  */
/* pool accepts (0 if none is needed or the arguments are invalid). The     */
/* size depends on the current device's compute-unit count; query it with   */
/* that device current.                                                      */
size_t pa_decode_workspace_size(const pa_kv_cache* cache, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_context_len);

/* ------------------------------------------------------------------------ */
/* pa_decode_no_alloc — pa_decode for callers that cannot allocate memory:    */
/* code under HIP graph capture, tight serving loops, and hosts that forbid  */
/* device allocation after start-up. Same arguments and result as pa_decode, */
/* without the workspace: the library keeps a fixed device array of          */
/* PA_DECODE_NO_ALLOC_MAX_BYTES on every GPU it runs on (held until the      */
/* process ends) and uses that instead. Nothing is allocated or freed.       */
/*                                                                           */
/*  - Sizes whose pa_decode_workspace_size exceeds                           */
/*    PA_DECODE_NO_ALLOC_MAX_BYTES return PA_ERR_WORKSPACE before any HIP    */
/*    call (use pa_decode with a workspace of your own for those).           */
/*  - The first call on a device that needs the array looks its address up  */
/*    (PA_ERR_HIP if that fails); later calls reuse it.                      */
/*  - All calls on one GPU share its array, and the array keeps whatever the */
/*    last call left (the kernels need no initialised workspace). Calls that */
/*    overlap on one GPU -- on different streams, or from several threads    */
/*    without ordering between them -- race on it and give undefined        */
/*    output rows; order them on one stream.                                 */
/* ------------------------------------------------------------------------ */
#define PA_DECODE_NO_ALLOC_MAX_BYTES ((size_t)64 << 20)

pa_status pa_decode_no_alloc(const pa_kv_cache* cache, int32_t layer, const void* q,
                             pa_dtype q_dtype, void* out, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, int32_t num_seqs,
                             int32_t num_q_heads, float scale, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* pa_decode_shared — pa_decode that reads a prefix shared by several        */
/* sequences once per group of up to 32 / g of them.                         */
/*                                                                           */
/* Same arguments and same result as pa_decode. Parallel samples of one      */
/* prompt share the prompt's blocks ("Efficient Memory Management ... with   */
/* PagedAttention", sampling paragraph; "Continuous Batching and             */
/* PagedAttention", section "Sharing, the part that goes beyond fixing what  */
/* broke"); pa_decode reads such a block once per sequence. Here sharing is  */
/* found in the block tables: a run of consecutive sequences, each naming    */
/* the same leading blocks as the one before for at least 16 tokens, shares */
/* the common prefix of all its members (rounded down to a multiple of 16   */
/* tokens and capped by every member's context). Up to 32 / g members at a   */
/* time attend to that prefix together, their queries side by side in two   */
/* matrix-core tiles, so each prefix block is read once per group, while,   */
/* in the same launch on the other workgroups, each member attends to the   */
/* rest of its context; a final combine joins the two partial results.     */
/* Put the samples of one prompt next to each other in the batch. The two   */
/* passes split the workgroups by the plan's chunk counts; a batch with no  */
/* sharing gives them all to the second pass and gets the right result,     */
/* though a few percent slower than pa_decode (planning and a combine).     */
/*                                                                           */
/*  reuse_plan   0: find the sharing from block_tables / context_lens and    */
/*               store it in the workspace (two small launches). 1: use the  */
/*               plan the previous call left in this workspace (another      */
/*               layer of the same step: same tables, lengths, num_seqs and  */
/*               pool geometry; anything else gives undefined results).      */
/*  workspace    >= pa_decode_shared_workspace_size(...) bytes, 256-byte     */
/*               aligned.                                                    */
/* Supported: the matrix-core configurations of pa_decode (PA_F16 / PA_BF16 */
/* pools with the same q_dtype, PA_FP8_E4M3 pools with PA_F16 / PA_BF16     */
/* queries; head_dim 64 or 128; g in {1, 2, 4, 8}; num_seqs <= 8192); others */
/* return PA_ERR_UNSUPPORTED (use pa_decode).                                */
/* ------------------------------------------------------------------------ */
pa_status pa_decode_shared(const pa_kv_cache* cache, int32_t layer, const void* q,
                           pa_dtype q_dtype, void* out, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, int32_t num_seqs,
                           int32_t num_q_heads, float scale, int32_t reuse_plan,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes pa_decode_shared needs for these sizes (0 if the          */
/* configuration is unsupported or invalid). Depends on the current         */
/* device's compute-unit count; query it with that device current.          */
size_t pa_decode_shared_workspace_size(const pa_kv_cache* cache, int32_t num_seqs,
                                       int32_t num_q_heads);

/* ------------------------------------------------------------------------ */
/* pa_prefill — paged prefill: causal attention of each sequence's newest    */
/* positions (a whole prompt, a later chunk of one, or the prompt plus the   */
/* generated tokens of a recomputed request, which "When KV Capacity Runs    */
/* Out", section "Recompute KV from token history", runs again as one        */
/* prefill pass).                                                            */
/*                                                                           */
/* Sequence s has n_s = query_start_loc[s+1] - query_start_loc[s] query rows */
/* (rows query_start_loc[s] .. +n_s-1 of q). Row j is position               */
/* p = context_lens[s] - n_s + j and, for query head h (KV head h / g),      */
/*   out[row][h] = sum_{t <= p} softmax(scale * <q[row][h], K[t][kvh]>)_t    */
/*                 * V[t][kvh]                                               */
/* with token t read through block_tables[s][t / block_size] as in          */
/* pa_decode. The keys and values of all positions, the new ones included,   */
/* must already be in the pool (pa_write_kv first). n_s = context_lens[s] is */
/* a whole prefill, n_s = 1 a decode step.                                   */
/*                                                                           */
/*  q, out           device [num_q_tokens][num_q_heads][head_dim], q_dtype   */
/*                   PA_F16 or PA_BF16 (out rounded to nearest-even).        */
/*  query_start_loc  device int32 [num_seqs + 1]: 0, nondecreasing, last =   */
/*                   num_q_tokens.                                           */
/*  max_query_len    host bound on the n_s; sizes the launch (rows of a      */
/*                   sequence beyond it are not computed).                   */
/*  context_lens, block_tables, max_context_len: as for pa_decode.           */
/* A sequence whose context is invalid (as for pa_decode) or shorter than   */
/* n_s gets NaN rows; a table entry naming a block outside the pool gives    */
/* NaN in every row that attends to that block (and may in other rows of    */
/* the same sequence: rows are computed in groups of 128 / g). Rows outside */
/* [0, num_q_tokens) are never written; a sequence whose query_start_loc     */
/* entries leave that range is skipped. No workspace is needed.             */
/* Supported: pools PA_F16 / PA_BF16 with the same q_dtype, or PA_FP8_E4M3   */
/* with either; head_dim 64 or 128; num_q_heads / num_kv_heads in           */
/* {1, 2, 4, 8, 16}. Others return PA_ERR_UNSUPPORTED.                       */
/* ------------------------------------------------------------------------ */
pa_status pa_prefill(const pa_kv_cache* cache, int32_t layer, const void* q,
                     pa_dtype q_dtype, void* out, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t max_context_len, const int32_t* query_start_loc,
                     int32_t max_query_len, int32_t num_seqs,
                     int32_t num_q_tokens, int32_t num_q_heads, float scale,
                     hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* pa_copy_blocks — copy whole blocks (K and V, every layer, head and slot). */
/*                                                                           */
/*  PA_COPY_D2D  copy-on-write inside device memory: a sequence about to     */
/*               write into a shared block first receives a private copy     */
/*               ("Efficient Memory Management ... with PagedAttention",     */
/*               sampling and prefix paragraphs;                             */
/*               "Continuous Batching and PagedAttention", section "Sharing, */
/*               the part that goes beyond fixing what broke"). `pairs` is   */
/*               in device memory. dst and src may be the same pool.         */
/*  PA_COPY_D2H  swap out: device `src` pool -> pinned host `dst` pool.      */
/*  PA_COPY_H2D  swap in: pinned host `src` pool -> device `dst` pool; the   */
/*               destination blocks may differ from the ones the data left   */
/*               ("When KV Capacity Runs Out", section "Restore KV stored    */
/*               outside the GPU").                                          */
/*               For D2H / H2D `pairs` is in host memory and is validated    */
/*               (ids in range, destination ids distinct) before any copy.   */
/*               The DMA engines copy, one transfer per run of consecutive   */
/*               ids (per layer unless a block's layers are contiguous on    */
/*               both sides); kernels on other streams run on undisturbed,   */
/*               so a swap on a copy stream overlaps decode.                 */
/*  PA_COPY_D2H_KERNEL, PA_COPY_H2D_KERNEL  the same moves by one kernel     */
/*               that reads and writes the host pool directly: the host link */
/*               runs at full speed whatever the block size ("41 ·           */
/*               Preemption, Recomputation & KV Pressure", section 3: many   */
/*               small transfers underuse it), but memory-bound kernels on   */
/*               other streams stall while it runs. The host pool must be    */
/*               pinned and device-mapped (pa_host_pool_mapped), else        */
/*               PA_ERR_UNSUPPORTED before any copy.                         */
/*  pairs        int64 [num_pairs][2] = {src_block, dst_block}.              */
/*  Both pools must have the same dtype, layers, heads, block size and head  */
/*  dim (strides may differ). Destination ids must be distinct and, for D2D  */
/*  within one pool, no id may be both a source and a destination in one     */
/*  call (undefined result otherwise). The copied bytes are identical.       */
/*  num_pairs == 0 is a no-op.                                               */
/* ------------------------------------------------------------------------ */
typedef enum {
  PA_COPY_D2D = 0,
  PA_COPY_H2D = 1,
  PA_COPY_D2H = 2,
  PA_COPY_H2D_KERNEL = 3,
  PA_COPY_D2H_KERNEL = 4
} pa_copy_dir;

pa_status pa_copy_blocks(const pa_kv_cache* dst, const pa_kv_cache* src,
                         const int64_t* pairs, int32_t num_pairs,
                         pa_copy_dir dir, hipStream_t stream);

/* pa_copy_blocks_staged — swap through a device staging buffer.            */
/*                                                                           */
/*  The moves of PA_COPY_D2H / PA_COPY_H2D, with the DMA engines moving a    */
/*  few large ranges: for D2H a kernel first gathers the scattered device    */
/*  blocks into `staging` (device memory the caller owns, 16-byte aligned),  */
/*  then one DMA transfer per run of consecutive host ids moves K and V;     */
/*  for H2D the transfers land in `staging` and a kernel scatters them into  */
/*  the device blocks. The DMA engines carry the host-link traffic, so a     */
/*  swap on a copy stream overlaps decode ("When KV Capacity Runs Out",      */
/*  section "Restore KV stored outside the GPU"), and large transfers keep   */
/*  the link busy whatever the block size or device layout ("41 ·           */
/*  Preemption, Recomputation & KV Pressure", section 3).                    */
/*  dir          PA_COPY_D2H or PA_COPY_H2D.                                 */
/*  staging      holds at least one block: 2 * num_layers * num_kv_heads *   */
/*               block_size * head_dim * element bytes; larger lists go in  */
/*               chunks of as many blocks as fit (pa_copy_staging_size gives */
/*               the size that moves a list in one chunk), else              */
/*               PA_ERR_WORKSPACE. Its contents afterwards are unspecified.  */
/*  The host pool's layers must be contiguous within a block (num_layers ==  */
/*  1 or layer_stride == num_kv_heads * block_size * head_dim), else        */
/*  PA_ERR_UNSUPPORTED; the device pool may have any valid layout. Pairs are */
/*  host memory, checked as for pa_copy_blocks before any device work.       */
/* ------------------------------------------------------------------------ */
pa_status pa_copy_blocks_staged(const pa_kv_cache* dst, const pa_kv_cache* src,
                                const int64_t* pairs, int32_t num_pairs, pa_copy_dir dir,
                                void* staging, size_t staging_bytes, hipStream_t stream);

/* Staging bytes that let pa_copy_blocks_staged move num_pairs blocks of     */
/* this pool's geometry in one chunk (0 for an invalid pool or count).       */
size_t pa_copy_staging_size(const pa_kv_cache* pool, int32_t num_pairs);

/* 1 when the pool's K and V arrays are pinned host memory that the current  */
/* device addresses directly (what PA_COPY_*_KERNEL needs), 0 otherwise,    */
/* including for an invalid pool. Leaves no pending HIP error behind.        */
int32_t pa_host_pool_mapped(const pa_kv_cache* pool);

/* Static, human-readable name of a status code. */
const char* pa_status_string(pa_status s);

/* Library version string, e.g. "0.1.0". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
