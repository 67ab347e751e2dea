/*
 * pa_blocks.h — host-side KV block manager (C ABI), the bookkeeping around
 * the three device calls of pa.h: it decides which physical block every
 * position of every sequence lives in, and produces the slot mappings, block
 * tables, copy-on-write pairs and swap pairs those calls take.
 *
 * What it implements, from the pages:
 *  - A pool of fixed-size blocks and a FIFO free list; any free block serves
 *    any sequence ("Continuous Batching and PagedAttention", section
 *    "Fixed-size blocks make every free block usable").
 *  - Per-sequence block tables that fill left to right; a block is taken
 *    only when the last one is full ("Efficient Memory Management for Large
 *    Language Model Serving with PagedAttention" (summary page), block-table
 *    paragraph; "When KV Capacity Runs Out", Figures 1 and 2).
 *  - Reference counts for shared blocks (forked samples, shared prompts) and
 *    copy-on-write before a sequence writes into a shared, partly filled
 *    block (same summary page, sampling and prefix paragraphs).
 *  - All-or-nothing release: a preempted or finished sequence gives up every
 *    block at once, contents untouched ("41 · Preemption, Recomputation & KV
 *    Pressure", section 2; "When KV Capacity Runs Out", section "Pause
 *    requests and release KV blocks").
 *  - Newest-first victim choice: the most recently admitted running sequence
 *    ("41 · Preemption, Recomputation & KV Pressure", section 2).
 *  - Swap: a victim's blocks are planned onto host blocks, released on the
 *    device once the copy is done, and restored into freshly allocated,
 *    possibly different, device blocks ("When KV Capacity Runs Out", section
 *    "Restore KV stored outside the GPU", Figure 4), with host-pool
 *    accounting ("KV Cache Preemption in vLLM", section "Swap versus
 *    recompute").
 *
 * Slots are encoded as physical_block * block_size + offset, as pa_write_kv
 * takes them. Sequences are named by caller-chosen int64 ids.
 *
 * Conventions: host only (no device memory, no HIP calls). A manager is
 * caller-owned (pa_bm_create / pa_bm_destroy) and not thread-safe; calls on
 * different managers are independent. Every call that fails returns a
 * non-OK status and changes nothing: PA_ERR_INVALID_ARG for null pointers,
 * unknown or duplicate ids, a sequence in the wrong state, or an output
 * array too small; PA_ERR_NO_SPACE when blocks are needed and not free.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;

/* A manager of num_blocks device blocks of block_size slots (their free list
 * in the order of `order`, a permutation of 0 .. num_blocks-1, or 0, 1, ...
 * when null) and num_host_blocks host blocks for swapped-out sequences (free
 * list 0, 1, ...). */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* order,
                       int32_t num_host_blocks, pa_bm** out);
void pa_bm_destroy(pa_bm* bm);

/* Free device blocks (host != 0: free host blocks). -1 for a null manager. */
int32_t pa_bm_num_free(const pa_bm* bm, int32_t host);

/* Admit a new running sequence holding no positions. */
pa_status pa_bm_add(pa_bm* bm, int64_t seq);

/* A new running sequence `child` mapping the same blocks as `parent`
 * (reference counts + 1): parallel samples of one prompt. */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* Reserve the next n positions of a running sequence. slots[i] receives the
 * slot of position num_tokens + i. When the last block is shared and partly
 * filled it is first copied: cow_pairs[2k], [2k+1] = (src, dst) block,
 * *num_cow the count (at most one per call). All or nothing: if the blocks
 * needed are not free, PA_ERR_NO_SPACE and nothing changes. slots needs n
 * entries, cow_pairs 2. */
pa_status pa_bm_append(pa_bm* bm, int64_t seq, int32_t n, int64_t* slots, int64_t* cow_pairs,
                       int32_t* num_cow);

/* Free device blocks the next n positions of `seq` would take (0 if the
 * sequence is unknown or not running). */
int32_t pa_bm_blocks_needed(const pa_bm* bm, int64_t seq, int32_t n);

/* Copy-on-write of the last block now, even if full (privatising a shared
 * last block up front; "Efficient Memory Management for Large Language Model
 * Serving with PagedAttention", sampling paragraph). pair[0], pair[1] =
 * (src, dst): dst is taken from the head of the free list and replaces src as
 * the sequence's last table entry; src loses this sequence's one reference.
 * The caller copies src into dst (pa_copy_blocks, PA_COPY_D2D) before writing
 * into it. PA_ERR_INVALID_ARG (nothing changed) when the sequence is unknown,
 * not running, holds no block, or is the only holder of its last block;
 * PA_ERR_NO_SPACE when no device block is free. */
pa_status pa_bm_copy_last_block(pa_bm* bm, int64_t seq, int64_t* pair);

/* Release every block of a sequence and forget it (finished, or preempted to
 * be recomputed later: its token history stays with the caller). */
pa_status pa_bm_release(pa_bm* bm, int64_t seq);

/* Block table of a sequence: table[0 .. *num_blocks-1] (capacity entries
 * available), *num_tokens its positions. For a swapped-out sequence the
 * table is empty and *num_tokens the saved count. */
pa_status pa_bm_table(const pa_bm* bm, int64_t seq, int32_t* table, int32_t capacity,
                      int32_t* num_blocks, int32_t* num_tokens);

/* Newest running sequence (the preemption victim), or PA_ERR_INVALID_ARG if
 * none is running. */
pa_status pa_bm_newest_running(const pa_bm* bm, int64_t* seq);

/* Swap-out plan of a running sequence: one host block per device block,
 * pairs[2i], [2i+1] = (device block, host block) for pa_copy_blocks
 * (PA_COPY_D2H), *n the count (capacity pairs available). The device blocks
 * stay held until pa_bm_swap_out_done, which the caller issues once the copy
 * has completed (its stream order), so no write can reuse them early.
 * PA_ERR_NO_SPACE if the host pool is short. */
pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* n);
pa_status pa_bm_swap_out_done(pa_bm* bm, int64_t seq);

/* Swap-in plan of a swapped-out sequence: fresh device blocks for its host
 * blocks, pairs[2i], [2i+1] = (host block, device block) for pa_copy_blocks
 * (PA_COPY_H2D); the host blocks are released and the sequence runs again,
 * admitted now. A later swap-out may be handed those host blocks at once:
 * issue its device-to-host copies on the same stream, after these, so they
 * never overwrite a host block before it has been read. PA_ERR_NO_SPACE if
 * the device pool is short. */
pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif  /* PA_BLOCKS_H_ */
