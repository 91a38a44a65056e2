/*
 * paged_block_manager.h -- host-side block manager of the paged KV cache, exported by libpagedattn.so.
 *
 * What it manages (vLLM PagedAttention, page 1 "LLM inference framework evaluation ... PagedAttention",
 * section 3.2; page 2 "vLLM-v0.11.0 ... how much memory does PagedAttention save", section 4.2):
 *  - a pool of `num_blocks` fixed-size physical blocks of `block_size` token slots, handed out from a free list
 *    and returned to it when no sequence uses them any more (the memory pool that reuses released blocks);
 *  - per sequence, the list of physical blocks that holds its tokens in logical order (its block-table row);
 *    a new block is taken only when a token needs one (on-demand allocation);
 *  - sharing: a forked sequence (beam search, parallel sampling) and sequences whose prompts start with the
 *    same full blocks of tokens (a common system prompt) reference the same physical blocks, counted by a
 *    per-block reference count; a sequence about to write into a block it shares first gets a private copy
 *    (copy-on-write), reported as a (src, dst) pair for copy_blocks().
 *
 * The manager never touches device memory: it hands out slots (slot = block * block_size + offset, the
 * slot_mapping of reshape_and_cache), copy pairs and block tables, and the caller moves the bytes with the
 * kernels of pa.h. Within one decode step the caller must apply the copy pairs
 * (copy_blocks) before writing the step's new tokens (reshape_and_cache).
 *
 * Conventions: host pointers only; the handle is not thread-safe (one caller at a time); every call either
 * succeeds completely or returns a negative status and changes nothing (short of the host itself running out
 * of memory, reported as PA_ERR_NOMEM). Status codes are those of pa.h plus PA_ERR_NOMEM and
 * PA_ERR_SEQ below.
 */
#ifndef PAGED_BLOCK_MANAGER_H
#define PAGED_BLOCK_MANAGER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ERR_NOMEM (-8) /* not enough free blocks for the request (nothing was allocated) */
#define PA_ERR_SEQ (-9)   /* unknown sequence id, or a sequence id that already exists */

typedef struct pa_block_manager pa_block_manager;

/*
 * A manager over blocks [0, num_blocks) of block_size slots; sequences may hold at most max_blocks_per_seq
 * blocks. Block `reserved_block` (or none when -1) is never handed out: callers use it to pad block tables.
 * Returns NULL on invalid sizes or when memory for the bookkeeping cannot be allocated.
 */
pa_block_manager *pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                               int32_t reserved_block);
void pa_bm_destroy(pa_block_manager *bm);

/*
 * Start sequence `seq_id` with a prompt of num_tokens tokens. With `tokens` non-NULL, every full block of
 * the prompt whose token contents (and everything before them) equal those of a full block already in the
 * pool is shared instead of allocated (prefix sharing; page 2 section 4.2 reuses shared blocks). The slot of
 * each prompt token is written to slots_out[num_tokens]: -1 for tokens that live in a shared block (their
 * K/V is already in the cache), else the slot to fill. Returns the number of newly allocated blocks.
 */
int32_t pa_bm_add_sequence(pa_block_manager *bm, int64_t seq_id, const int32_t *tokens, int32_t num_tokens,
                           int32_t *slots_out);

/* Child `child_id` starts as a copy of `parent_id` that shares all of its blocks (page 1 section 3.2). */
int32_t pa_bm_fork(pa_block_manager *bm, int64_t parent_id, int64_t child_id);

/*
 * Append one token to each of n sequences (a decode step): slots_out[i] receives the slot of sequence
 * seq_ids[i]'s new token. A sequence whose last block is full gets a new block; one whose last block is
 * shared gets a private copy of it first (copy-on-write), recorded as a pending copy pair. All or nothing:
 * PA_ERR_NOMEM if the step needs more free blocks than there are. Sequence ids must be distinct.
 */
int32_t pa_bm_append_slots(pa_block_manager *bm, const int64_t *seq_ids, int32_t n, int32_t *slots_out);

/*
 * Move the pending copy-on-write pairs ({src, dst} block ids, in the order they arose) to pairs_out
 * (capacity max_pairs pairs) and forget them. Returns the number of pairs, or PA_ERR_SHAPE if more are
 * pending than fit (nothing is taken then). Apply them with copy_blocks() before this step's cache writes.
 */
int32_t pa_bm_take_copies(pa_block_manager *bm, int32_t *pairs_out, int32_t max_pairs);

/* Release a finished sequence: blocks no longer referenced return to the free list. */
int32_t pa_bm_free_sequence(pa_block_manager *bm, int64_t seq_id);

/*
 * Block tables of n sequences: row i of table_out[n][max_blocks_per_seq] holds seq_ids[i]'s blocks in
 * logical order, padded with `pad`; lens_out[i] its length in tokens.
 */
int32_t pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seq_ids, int32_t n, int32_t *table_out,
                           int32_t *lens_out, int32_t pad);

/*
 * Swap (page 1 section 5: swap space on the host; page 2 section 7.2: inactive blocks moved to host memory).
 * The caller keeps a second pair of pools in host memory (pinned, so that swap_blocks of pa.h can
 * reach it) with num_host_blocks blocks of the device pools' shape; the manager hands out its block ids.
 *
 * pa_bm_set_host_pool: use host blocks [0, num_host_blocks). PA_ERR_SEQ while a sequence is swapped out.
 *
 * pa_bm_swap_out: move sequence seq_id out of the device pool. Each of its blocks, in logical order, is given
 * a host block: pairs_out[i] = {device block, host block}. Apply them with swap_blocks (host pools <- device
 * pools) before any freed device block is written again -- on one stream, enqueue the swap first. Device
 * blocks the sequence alone used return to the free list; shared ones stay with their other users. The
 * sequence keeps its length but is unknown to append/fork/block_tables (PA_ERR_SEQ) until swapped in;
 * free_sequence releases its host blocks. Returns the number of pairs; PA_ERR_NOMEM when the host pool lacks
 * blocks, PA_ERR_SHAPE when max_pairs is too small or copy-on-write pairs are still pending (take and apply
 * them first). Nothing changes on failure.
 *
 * pa_bm_swap_in: bring a swapped-out sequence back into fresh device blocks: pairs_out[i] = {host block,
 * device block}; apply them with swap_blocks (device pools <- host pools) before the sequence's next attention.
 * Its host blocks return to the host pool. PA_ERR_NOMEM when the device pool lacks free blocks.
 *
 * pa_bm_swap_stats: int64 stats_out[4] = free host blocks, host blocks in use, swapped-out sequences, blocks
 * moved so far (out and in).
 */
int32_t pa_bm_set_host_pool(pa_block_manager *bm, int32_t num_host_blocks);
int32_t pa_bm_swap_out(pa_block_manager *bm, int64_t seq_id, int32_t *pairs_out, int32_t max_pairs);
int32_t pa_bm_swap_in(pa_block_manager *bm, int64_t seq_id, int32_t *pairs_out, int32_t max_pairs);
int32_t pa_bm_swap_stats(const pa_block_manager *bm, int64_t *stats_out);

/*
 * Occupancy, as int64 stats_out[8]: free blocks, used blocks, blocks referenced by more than one sequence,
 * sequences, tokens summed over sequences, token slots in used blocks, slots holding a token (a shared slot
 * counted once), copy-on-write copies so far. Internal fragmentation = 1 - stats[6] / stats[5].
 */
int32_t pa_bm_stats(const pa_block_manager *bm, int64_t *stats_out);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_BLOCK_MANAGER_H */
