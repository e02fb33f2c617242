/*
 * pa_blockmgr.h -- host-side page allocator that feeds the paged-attention
 * kernels: it decides where every token's K/V row lives and produces the
 * inputs of pa_kv_append / pa_decode_append (slot_mapping), pa_decode
 * (block_tables, context_lens) and pa_copy_blocks (block_mapping).
 *
 * Behaviour [What is PagedAttention? (esaholic.com AI glossary),
 * "Step-by-Step Implementation Framework" and "Copy-on-Write Memory
 * Forking"; PagedAttention Internals (dailyaiworld.com), "How PagedAttention
 * Works" item 2, "Copy-on-Write and Prefix Sharing" and "Implementation:
 * Custom Block Manager Simulation"]:
 *   - the pool holds num_blocks physical pages of block_size tokens; free
 *     pages are handed out from the front of a free list and returned to its
 *     back, so reuse is first-in first-out;
 *   - a sequence of n tokens holds ceil(n / block_size) pages; token t lives
 *     in page pages[t / block_size] at offset t % block_size (its slot is
 *     page * block_size + offset);
 *   - every page carries a reference count (1 when taken); a forked sequence
 *     shares its parent's pages by reference; a page returns to the free
 *     list when its count reaches 0;
 *   - appending a token takes a new page when the token opens a block;
 *     appending into a partly filled page that is still shared first moves
 *     the sequence onto a fresh private page and reports the (old, new) pair
 *     for pa_copy_blocks (copy-on-write); the last holder writes in place;
 *   - running out of pages is an error status, never a partial result.
 *
 * Prefix caching [Paged Attention (AI terminology), "Key Points" (sharing
 * row) and "Common Usage Examples"; PagedAttention Internals, "Copy-on-Write and Prefix
 * Sharing" and "Architectural Recommendations" item 2]: prompts allocated
 * with pa_bm_allocate_prompt share every leading full page whose whole token
 * prefix an earlier prompt already stored, so the caller writes K/V only for
 * the tokens after the cached prefix.  Cached pages stay reusable after their
 * last holder frees them, until the free list hands them out again.
 *
 * Host memory only: the manager owns its state (allocated at create and as
 * sequences are added) and touches no device memory.  One manager must not
 * be used from two threads at once.  Sequence ids are caller-chosen int64.
 */
#ifndef PA_BLOCKMGR_H
#define PA_BLOCKMGR_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/*
 * Create a manager over pages 0 .. num_blocks - 1 (1 <= num_blocks <= 2^31)
 * of block_size tokens (>= 1).  free_order (host, num_blocks entries, or
 * NULL for 0, 1, 2, ...) is the initial order of the free list and must be a
 * permutation.  Returns PA_OK and *out, PA_ERR_NULL, PA_ERR_ARG or
 * PA_ERR_HOST_MEMORY.
 */
pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, const int64_t* free_order,
                       pa_block_manager** out);

/* Release the manager (NULL is a no-op). */
void pa_bm_destroy(pa_block_manager* bm);

/* Free pages, live sequences; -1 for a NULL manager. */
int64_t pa_bm_num_free(const pa_block_manager* bm);
int64_t pa_bm_num_seqs(const pa_block_manager* bm);

/* Token count of a sequence, or -1 if it does not exist. */
int64_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id);

/*
 * Copy up to `cap` page ids of a sequence (logical order) into `pages` (host)
 * and return how many pages it holds, or -1 if it does not exist.
 */
int64_t pa_bm_seq_pages(const pa_block_manager* bm, int64_t seq_id, int64_t cap, int32_t* pages);

/* Reference count of a page, or -1 for an id outside the pool. */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int64_t page);

/*
 * Copy up to `cap` entries of the free list, front first, into `pages`
 * (host) and return its length.
 */
int64_t pa_bm_free_list(const pa_block_manager* bm, int64_t cap, int32_t* pages);

/*
 * New sequence seq_id holding num_tokens (>= 0) tokens, e.g. a prompt:
 * ceil(num_tokens / block_size) pages from the front of the free list.
 * PA_ERR_ARG if seq_id exists or num_tokens < 0; PA_ERR_OUT_OF_PAGES if the
 * pool has fewer free pages (nothing is taken).
 */
pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, int64_t num_tokens);

/*
 * New sequence seq_id for a prompt of num_tokens (>= 0) token ids (host
 * int32 array `tokens`; NULL allowed when num_tokens is 0).
 *
 * Page k (k < num_tokens / block_size, i.e. a full page) is identified by
 * tokens[0 .. (k + 1) * block_size): the K/V it holds depends on that whole
 * prefix.  The leading run of full pages whose prefixes are cached is shared
 * (reference counts raised; a cached page on the free list is taken back off
 * it).  The remaining ceil(num_tokens / block_size) - hits pages come from
 * the front of the free list, and each of them that is full is registered
 * under its prefix (replacing an older page registered under the same
 * prefix).  *num_cached_tokens receives hits * block_size: the tokens whose
 * K/V is already in place; the caller writes tokens num_cached_tokens ..
 * num_tokens - 1 (pa_kv_append) before any kernel reads them, and a prompt
 * that hits pages registered by an earlier call in the same step reads them
 * only after that call's writes.
 *
 * Identity is a 128-bit hash of the prefix: two different prefixes share a
 * page only on a 128-bit collision.  A cached page is evicted (its entry
 * dropped) when the free list hands it out for any allocation.
 *
 * PA_ERR_NULL (num_cached_tokens NULL, or tokens NULL with num_tokens > 0),
 * PA_ERR_ARG (seq_id exists, num_tokens < 0), PA_ERR_OUT_OF_PAGES (fewer free
 * pages than the fresh pages plus the cached free pages it takes back);
 * every error changes no state.
 */
pa_status pa_bm_allocate_prompt(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                                int64_t num_tokens, int64_t* num_cached_tokens);

/* Pages registered in the prefix cache (held or free); -1 for a NULL manager. */
int64_t pa_bm_num_cached(const pa_block_manager* bm);

/* 1 if the page is registered in the prefix cache, 0 if not, -1 outside the pool. */
int32_t pa_bm_page_cached(const pa_block_manager* bm, int64_t page);

/*
 * New sequence child_id sharing every page of parent_id (reference counts
 * raised).  PA_ERR_NOT_FOUND for an unknown parent, PA_ERR_ARG if child_id
 * exists.
 */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id);

/*
 * Drop a sequence: each of its pages loses one reference and returns to the
 * back of the free list at zero (in the sequence's page order).  An unknown
 * id is a no-op (PA_OK).
 */
pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id);

/*
 * One decode step: append one token to each of seq_ids[0 .. n) in order (a
 * sequence may appear more than once).  slots[i] (host) receives the slot of
 * the i-th new token.  Copy-on-write page copies are written to copies
 * (host, [n][2] int64 (src, dst), at most one per token) in the order they
 * arise, their number to *num_copies; issue them with pa_copy_blocks before
 * writing the new rows.
 * tables / context_lens (host, optional, both or neither): a batch's
 * device-layout inputs as pa_bm_block_tables wrote them for these seq_ids
 * ([n][max_blocks_per_seq] int32 and [n] int32).  They are kept current:
 * only the entries this step changes are written (a page a new token opens,
 * a page copy-on-write replaces, the length), so a decode step costs O(n)
 * instead of a rebuild.  With tables, seq_ids must be distinct and every
 * sequence must still fit max_blocks_per_seq pages (else PA_ERR_ARG).
 * All or nothing: PA_ERR_OUT_OF_PAGES (pool too small for the whole batch),
 * PA_ERR_NOT_FOUND (unknown id) and PA_ERR_ARG change no state.
 */
pa_status pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, int32_t n, int64_t* slots,
                       int64_t* copies, int32_t* num_copies, int32_t max_blocks_per_seq,
                       int32_t* tables, int32_t* context_lens);

/*
 * Device-layout inputs for a batch: tables (host, [n][max_blocks_per_seq]
 * int32) receives each sequence's page ids followed by pad_page, and
 * context_lens (host, [n] int32) its token count.  PA_ERR_NOT_FOUND for an
 * unknown id, PA_ERR_ARG if a sequence holds more than max_blocks_per_seq
 * pages or more than 2^31 - 1 tokens.
 */
/*
 * Tokens that seq_ids[0 .. n) share in the same physical pages: the leading
 * pages that are one and the same page in every sequence (a forked prompt,
 * beams), in whole pages and capped by the shortest sequence.  That is the
 * shared_len pa_decode_shared_prefix takes for a batch of these sequences in
 * this order.  0 for n == 0; -1 for a NULL manager, n < 0, seq_ids NULL with
 * n > 0, or an unknown id.  [Internals, "Copy-on-Write and Prefix Sharing"]
 */
int64_t pa_bm_shared_prefix(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n);

/*
 * The group arrays pa_decode_shared_prefix_groups takes, for a batch in the
 * order seq_ids[0 .. n): each maximal run of two or more consecutive
 * sequences whose first pages are one and the same page, and that share at
 * least one whole page, is a group with the shared length
 * pa_bm_shared_prefix gives for it; the sequences between two such runs
 * (single sequences, runs sharing no whole page) form one group each of
 * shared length 0, read per sequence by the decode.  group_start (host,
 * n + 1 entries) receives the groups' first positions and then n,
 * group_shared_len (host, n entries) their shared lengths and
 * seq_shared_len (host, n entries) each sequence's group's shared length.
 * max_group_size and max_shared_len (host, may be NULL) receive the bounds
 * the decode call takes: the largest size of a group with a shared length
 * (1 when there is none; shared-nothing groups need no bound) and the
 * largest shared length.  Returns the number of groups, or -1 for a NULL
 * manager or output, n < 0, or an unknown id.  [Internals, "Copy-on-Write
 * and Prefix Sharing"]
 */
int32_t pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                            int32_t* group_start, int32_t* group_shared_len, int32_t* seq_shared_len,
                            int32_t* max_group_size, int32_t* max_shared_len);

pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                             int32_t max_blocks_per_seq, int32_t pad_page, int32_t* tables,
                             int32_t* context_lens);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKMGR_H */
