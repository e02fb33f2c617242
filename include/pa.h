/*
 * pa.h -- paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every tensor argument is a plain
 * device pointer owned by the caller; sizes are plain integers.  The library
 * allocates no memory, never synchronises and never throws: every call
 * validates its arguments on the host, then enqueues its kernels
 * asynchronously on `stream` (NULL = the null stream) and returns.  Its only
 * global state is pa_decode_noalloc's static scratch array and the cached
 * per-device address of it.
 *
 * Pages cited (title, then section):
 *   [Glossary]  "What is PagedAttention? Definition & Virtual Memory
 *               Architecture" (esaholic.com AI glossary)
 *   [Internals] "PagedAttention Internals: How Memory Fragmentation in LLM
 *               Serving Was Solved" (dailyaiworld.com)
 *
 * The pages fix the idea -- K/V vectors live in fixed-size blocks of 16 or 32
 * tokens scattered through one physical pool, a per-sequence block table maps
 * logical block i to a physical page, and the attention kernel reads K/V
 * through that table with no gather copy [Glossary, "Technical Architecture";
 * Internals, "How PagedAttention Works" items 1-3] -- but no memory layout.
 * The layouts below are this library's:
 *
 *   X = 16 / sizeof(element)        (8 for bf16, 4 for fp32)
 *   k_cache  [num_blocks][num_kv_heads][head_dim / X][block_size][X]
 *   v_cache  [num_blocks][num_kv_heads][head_dim][block_size]
 *   q, out   [num_seqs][num_heads][head_dim]
 *   k, v     [num_tokens][num_kv_heads][head_dim]          (new rows to append)
 *   block_tables [num_seqs][max_blocks_per_seq] int32      (physical page ids)
 *   context_lens [num_seqs] int32                          (tokens to attend over)
 *   slot_mapping [num_tokens] int64                        (page*block_size + offset)
 *   block_mapping [num_pairs][2] int64                     (src page, dst page)
 *
 * Token t of sequence b lives in page block_tables[b][t / block_size] at
 * offset t % block_size.  One (page, kv head) tile of K or V is one contiguous
 * run of head_dim * block_size elements (4 KiB for bf16, head_dim 128,
 * block 16).  All element types of one call are the same `pa_dtype`.
 *
 * Supported shapes: head_dim in {64, 128}; block_size in {16, 32};
 * num_heads a multiple of num_kv_heads with num_heads / num_kv_heads <= 16.
 *
 * Beyond the interface the library was specified with -- pa_kv_append(k, v,
 * slot_mapping, k_cache, v_cache), pa_decode(q, k_cache, v_cache,
 * block_tables, context_lens, block_size, num_kv_heads, scale, out, stream)
 * and pa_copy_blocks -- every added argument comes after those: sizes, the
 * pool size num_blocks (pa_decode and pa_copy_blocks clamp or skip ids
 * outside it), the dtype, the partition size, the kernel family and load
 * path (pa_decode, and num_kv_heads and reuse in pa_decode_workspace_size,
 * on which the default partition depends) and the workspace.
 *
 * Preconditions the library cannot check without reading device memory
 * (violating them gives unspecified output, never an out-of-bounds access):
 * table entries used by a sequence lie in [0, num_blocks); context_lens[b]
 * lies in [0, max_context_len]; non-negative append slots are unique; the
 * source and destination sets of a copy are disjoint and destinations are
 * unique.  Device-side guards clamp or skip anything out of range, so a bad
 * index never leaves the buffers the caller described.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL */
    PA_ERR_ARG = -2,         /* a size or count is out of range or inconsistent */
    PA_ERR_UNSUPPORTED = -3, /* valid request outside the shapes listed above */
    PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    PA_ERR_HIP = -5,         /* the HIP runtime refused a launch */
    PA_ERR_OUT_OF_PAGES = -6, /* block manager: the page pool is exhausted */
    PA_ERR_NOT_FOUND = -7,   /* block manager: no sequence with that id */
    PA_ERR_HOST_MEMORY = -8, /* block manager: host allocation failed */
    PA_ERR_SCRATCH = -9      /* pa_decode_noalloc: request exceeds the static scratch */
} pa_status;

/* Bytes of device scratch pa_decode_noalloc holds per GPU (32 MiB). */
#define PA_STATIC_SCRATCH_BYTES (32u * 1024u * 1024u)

typedef enum pa_dtype {
    PA_F32 = 0,
    PA_BF16 = 1
} pa_dtype;

/* Which decode kernel family runs.  AUTO picks the matrix-core kernel for
 * bf16 and the vector-ALU kernel for fp32; the two compute the same thing. */
typedef enum pa_kernel {
    PA_KERNEL_AUTO = 0,
    PA_KERNEL_VALU = 1,      /* vector ALU (fp32 and bf16) */
    PA_KERNEL_MFMA = 2       /* MFMA matrix cores for Q.K^T and P.V (bf16 only) */
} pa_kernel;

/* How the K/V pages of one decode call are reused across its sequences.
 * It picks the load path of the decode kernels; every choice computes the
 * same result.  Streaming loads pass pages by the caches (the fastest way to
 * read pages that only one sequence of the batch touches); cached loads let
 * sequences that share pages -- a common prompt prefix, forked beams --
 * serve each other from L2 [Internals, "Copy-on-Write and Prefix Sharing";
 * Glossary, "Copy-on-Write Memory Forking"]. */
typedef enum pa_kv_reuse {
    PA_KV_AUTO = 0,      /* library default: PA_KV_STREAM */
    PA_KV_STREAM = 1,    /* no page is read by more than one sequence */
    PA_KV_SHARED = 2     /* some pages are read by several sequences */
} pa_kv_reuse;

/* Human-readable text for a status code; never NULL, static storage. */
const char* pa_status_string(pa_status status);

/* ABI version of this header (major * 100 + minor). */
int32_t pa_version(void);

/*
 * pa_kv_append -- write each new token's key and value rows into its slot.
 *
 * For every token i with slot_mapping[i] >= 0: page = slot / block_size,
 * off = slot % block_size, and for every kv head h the row k[i][h][:] is
 * copied into k_cache at (page, h, :, off, :) and v[i][h][:] into v_cache at
 * (page, h, :, off).  A bit copy: no conversion, NaN payloads preserved.
 * Negative slots are skipped (padding).  Slots >= num_blocks * block_size are
 * skipped as well (out of range; documented precondition violation).
 * [Internals, "How PagedAttention Works" item 2: pages come from the pool on
 * demand as tokens are generated; Glossary, page-table figure: a token's
 * place is its page plus its offset inside the block]
 *
 *   k, v          device, [num_tokens][num_kv_heads][head_dim], read
 *   slot_mapping  device, [num_tokens] int64, read
 *   k_cache/v_cache device, layouts above, written at the given slots only
 *   num_blocks    pool size in pages (bounds the slots)
 * Returns PA_OK (num_tokens == 0 is a no-op), PA_ERR_NULL, PA_ERR_ARG,
 * PA_ERR_UNSUPPORTED or PA_ERR_HIP.
 */
pa_status pa_kv_append(const void* k, const void* v, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache,
                       int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                       hipStream_t stream);

/*
 * pa_decode -- one decode step of paged attention.
 *
 * For each sequence b (L = context_lens[b]) and query head h
 * (kv head g = h / (num_heads / num_kv_heads)):
 *     s_t = scale * q[b][h] . K_b[t][g]            for t in [0, L)
 *     out[b][h] = sum_t softmax(s)_t * V_b[t][g]
 * where K_b[t], V_b[t] are read in place from page block_tables[b][t / bs]
 * at offset t % bs.  L == 0 writes zeros.  Accumulation is fp32; the output
 * is rounded once (round-to-nearest-even for bf16).
 * [Internals, "How PagedAttention Works" item 3 (the fused kernel fetches
 * non-contiguous K/V through the block table and runs scaled dot-product
 * attention); Glossary, "On-the-Fly CUDA Block Fetching"]
 *
 * Long contexts are cut into partitions of `partition_size` tokens processed
 * by independent workgroups, each leaving its running max, running sum and
 * unnormalised accumulator in `workspace`; a second kernel merges them.
 *
 *   q             device, [num_seqs][num_heads][head_dim], read
 *   k_cache/v_cache device, layouts above, read
 *   block_tables  device, [num_seqs][max_blocks_per_seq] int32, read
 *   context_lens  device, [num_seqs] int32, read
 *   block_size    16 or 32;  num_kv_heads: kv heads per page
 *   scale         multiplies q . k (typically 1/sqrt(head_dim))
 *   out           device, [num_seqs][num_heads][head_dim], written
 *   max_context_len  host-side upper bound of context_lens (sizes the grid;
 *                 no device-to-host read is ever made)
 *   num_blocks    pool size in pages (device-side guard on table entries)
 *   partition_size 0 = library default, -1 = single pass (one workgroup per
 *                 sequence and kv head), otherwise a multiple of 32 >= 32
 *   kernel        PA_KERNEL_AUTO / _VALU / _MFMA
 *   reuse         PA_KV_AUTO / _STREAM / _SHARED (load path; same result)
 *   workspace     device scratch of at least pa_decode_workspace_size(...)
 *                 bytes when the split path runs (may be NULL otherwise);
 *                 owned by the caller, contents undefined afterwards
 * Returns PA_OK (num_seqs == 0 is a no-op), PA_ERR_NULL, PA_ERR_ARG,
 * PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE or PA_ERR_HIP.
 */
pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t block_size, int32_t num_kv_heads, float scale,
                    void* out, hipStream_t stream,
                    int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t max_context_len,
                    int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                    pa_kernel kernel, pa_kv_reuse reuse, void* workspace,
                    size_t workspace_bytes);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes pa_decode's arguments without the workspace;
 * when the split path runs, the partials go to a device array of
 * PA_STATIC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends.  The call itself allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine); its first call on
 * a device looks up that device's copy of the array once.
 *
 * Result, partition choice and status codes are those of pa_decode with a
 * workspace of pa_decode_workspace_size() bytes, bit for bit, plus
 * PA_ERR_SCRATCH (nothing launched) when that size exceeds
 * PA_STATIC_SCRATCH_BYTES; a single pass needs no scratch at all.  No
 * scratch content needs clearing between calls: a call writes every
 * partial it later reads.
 *
 * Calls that overlap on one GPU race: they share that GPU's array, so a
 * caller serialises them (one stream, or events between streams).
 */
pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t block_size, int32_t num_kv_heads, float scale,
                            void* out, hipStream_t stream,
                            int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                            pa_kernel kernel, pa_kv_reuse reuse);

/*
 * pa_decode_append -- the usual decode step in one pass: every sequence
 * appends its newest token and attends over all L = context_lens[b] tokens,
 * the new one included.  Sequence b's new rows k_new[b], v_new[b] are written
 * into the slot of position L - 1 (page block_tables[b][(L-1) / block_size],
 * offset (L-1) % block_size) by the workgroup that reads that position,
 * which uses the new rows directly.  The result -- cache contents and
 * output -- is bit-identical to pa_kv_append with those slots followed by
 * pa_decode with the same arguments, and saves one launch and the append's
 * dependent memory round trips.  One exception in how, not what: on a
 * single pass of 12-wave workgroups over >= 1024 pairs (see
 * pa_decode_partition_size), the rows are stored by a launch of their own
 * just before the decode, which measured faster there.  [Internals, "How
 * PagedAttention Works" items 2 and 3]
 *
 *   k_new, v_new  device, [num_seqs][num_kv_heads][head_dim], read
 *   slot_mapping  device, [num_seqs] int64, or NULL (every sequence with
 *                 L > 0 appends).  A negative entry means sequence b appends
 *                 nothing this step (it only attends); a non-negative entry
 *                 must be the slot of position L - 1 -- the slot written is
 *                 always the one the block table gives.
 *   k_cache/v_cache device, read, and written at one slot per appending
 *                 sequence
 * Other arguments and return values as for pa_decode.  Sequences with
 * L == 0 append nothing and get zeros.
 */
pa_status pa_decode_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           const void* q, void* k_cache, void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t block_size, int32_t num_kv_heads, float scale,
                           void* out, hipStream_t stream,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, int32_t max_context_len,
                           int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                           pa_kernel kernel, pa_kv_reuse reuse, void* workspace,
                           size_t workspace_bytes);

/*
 * Partition size pa_decode uses for a request: > 0 = split path with that
 * many tokens per partition, 0 = single pass, < 0 = invalid request
 * (PA_ERR_ARG, or an unknown `reuse`).  Pure host arithmetic.  An explicit
 * partition_size (a multiple of 32) is returned as is and -1 gives 0.
 * The library default (partition_size 0) depends on the load path `reuse`
 * selects, with pairs = num_seqs * num_kv_heads:
 *   streaming loads (PA_KV_AUTO, PA_KV_STREAM): a single pass when
 *     max_context_len <= 512, when pairs >= 2048, when pairs >= 1024 and
 *     max_context_len <= 4096, or when 512 <= pairs < 1024,
 *     num_seqs <= 256 and max_context_len <= 8192 (then the workgroups take
 *     the sequences longest first); otherwise the largest power of two P in
 *     [1024, 8192] with P < max_context_len and
 *     pairs * ceil(max_context_len / P) >= 768; otherwise the shared-page rule.
 *   shared pages (PA_KV_SHARED): a single pass when max_context_len <= 512;
 *     otherwise the largest power of two P in [512, 4096] with
 *     4 P <= max_context_len and pairs * ceil(max_context_len / P) >= 1024
 *     (512 if none qualifies), lowered to 256 when that leaves fewer than
 *     1024 workgroups.
 * On the streaming path, partitions of 2048 tokens or more, single passes
 * over >= 1024 pairs (contexts over 512) and the longest-first single pass
 * run 12-wave workgroups that fill a compute unit each; everything else runs
 * 4-wave workgroups.  These choices change speed only: every one gives
 * results within the same bounds, and the order in which workgroups take
 * sequences changes no bit.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                 int32_t partition_size, pa_kv_reuse reuse);

/*
 * Workspace bytes pa_decode needs (0 for the single pass):
 * num_seqs * num_heads * ceil(max_context_len / P) * (head_dim + 2) * 4,
 * P = pa_decode_partition_size(num_seqs, num_kv_heads, max_context_len,
 * partition_size, reuse).  Returns 0 for invalid arguments as well.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                                pa_kv_reuse reuse);

/*
 * pa_decode_partition -- first stage of the split path on its own: every
 * (sequence, kv head, partition) workgroup writes its partials to
 * `workspace` (fp32 running max in log2 units, running sum, unnormalised
 * accumulator).  Together with pa_decode_reduce it is exactly what
 * pa_decode does when partition_size > 0; callers that merge partials
 * themselves (for example a context split across devices) use the two
 * stages directly.  partition_size must be given explicitly here (a
 * multiple of 32, > 0); size the workspace with pa_decode_workspace_size()
 * for that same partition_size.  max_context_len == 0 launches nothing.
 * k_new, v_new, slot_mapping: NULL for a plain decode; otherwise the fused
 * append of pa_decode_append (then this stage plus pa_decode_reduce is
 * exactly pa_decode_append, and k_cache / v_cache are written).
 * Arguments otherwise as for pa_decode.
 */
pa_status pa_decode_partition(const void* q, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t block_size, int32_t num_kv_heads, float scale,
                              hipStream_t stream,
                              int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t max_blocks_per_seq, int32_t max_context_len,
                              int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                              pa_kernel kernel, pa_kv_reuse reuse, void* workspace,
                              size_t workspace_bytes, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping);

/*
 * pa_decode_reduce -- second stage: merge the partitions of every
 * (sequence, head) with M = max_p m_p,
 *     out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
 * and round once to the output dtype.  Sequences with L == 0 get zeros.
 * `workspace` must hold what pa_decode_partition wrote for the same
 * num_seqs, num_heads, head_dim, max_context_len and partition_size (> 0).
 */
pa_status pa_decode_reduce(const void* workspace, size_t workspace_bytes,
                           const int32_t* context_lens, void* out, hipStream_t stream,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t max_context_len, int32_t partition_size, pa_dtype dtype);

/*
 * pa_decode_shared_prefix -- pa_decode for a batch whose sequences all
 * begin with the same `shared_len` tokens in the same physical pages (their
 * block tables agree on the first shared_len / block_size entries), as
 * after forking one prompt.  [Internals, "Copy-on-Write and Prefix
 * Sharing"; Glossary, "Copy-on-Write Memory Forking"]
 *
 * The shared pages are read once per kv head for up to 128 (sequence,
 * query head) pairs at a time -- a matrix-core stage whose columns are the
 * decode queries of several sequences, each seeing all shared_len
 * positions -- instead of once per sequence; the rest of every context is
 * read per sequence by the split decode kernel from position shared_len
 * on, in the same launch (the two stages share the compute units), and a
 * merge launch follows.  With 64 or more columns per kv head the prefix
 * stage stages its pages in LDS and picks its own partition size; its
 * partials take the first slots of every (sequence, head) workspace row and
 * the per-sequence partitions follow, so the merge kernel combines one
 * contiguous run per row.  The result is the same attention as pa_decode,
 * within the same bounds.
 *
 *   shared_len      a multiple of block_size, 0 <= shared_len <=
 *                   max_context_len (0: the plain split path)
 *   partition_size  a multiple of 32, the partition of the per-sequence
 *                   stage (and of the prefix stage below 64 columns); 0
 *                   picks 2048, measured best on a 100-sequence forked
 *                   prompt and on 8 beams
 *   workspace       >= pa_decode_shared_prefix_workspace_size(num_seqs,
 *                   num_heads, num_kv_heads, head_dim, max_context_len,
 *                   shared_len, partition_size) bytes
 *   k_new, v_new, slot_mapping  NULL for a plain decode; otherwise each
 *                   sequence's newest rows are appended as by
 *                   pa_decode_append (position L - 1 must lie past
 *                   shared_len, which every appending sequence gives since
 *                   it owns its last page)
 * Other arguments as for pa_decode (bf16 only; it always uses the
 * matrix-core kernels and the shared-page load path).  Preconditions, not
 * checked: every context_lens[b] >= shared_len, and the first
 * shared_len / block_size table entries are equal in every row (the
 * shared pages are read through row 0); otherwise the output is
 * unspecified, and memory accesses stay in bounds as for pa_decode.
 * Returns PA_ERR_UNSUPPORTED for fp32 and for more than 1024 sequences.
 */
pa_status pa_decode_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t block_size, int32_t num_kv_heads, float scale,
                                  void* out, hipStream_t stream,
                                  int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int64_t num_blocks, pa_dtype dtype, int32_t shared_len,
                                  int32_t partition_size, void* workspace, size_t workspace_bytes,
                                  const void* k_new, const void* v_new, const int64_t* slot_mapping);

/*
 * Workspace bytes pa_decode_shared_prefix needs for these arguments:
 * num_seqs * num_heads * (slots per row) * (head_dim + 2) * 4, a row
 * holding the prefix launch's partials and then the per-sequence ones.
 * Returns 0 for invalid arguments.
 */
/*
 * pa_decode_shared_prefix_groups -- the same for a batch of several groups
 * of sequences, each group sharing its own prefix (several prompts forked
 * at once, multi-tenant batches).  [Internals, "Copy-on-Write and Prefix
 * Sharing"]
 *
 *   num_groups        >= 0
 *   group_start       device, [num_groups + 1] int32: group g is sequences
 *                     group_start[g] .. group_start[g + 1] - 1 (consecutive,
 *                     ascending); sequences in no group share nothing
 *   group_shared_len  device, [num_groups] int32: tokens group g's sequences
 *                     hold in the same pages, whole pages (their table rows
 *                     agree on the first group_shared_len[g] / block_size
 *                     entries; read through the group's first row)
 *   seq_shared_len    device, [num_seqs] int32: each sequence's group's
 *                     shared length (0 for a sequence in no group)
 *   max_group_size    host bound on group sizes, 1 .. 1024
 *   max_shared_len    host bound on group_shared_len, <= max_context_len
 *   partition_size    a multiple of 32 (0: 2048)
 *   workspace         >= pa_decode_shared_prefix_groups_workspace_size()
 * Each group's shared pages are read once per kv head and column group for
 * all its sequences' queries (with 64 or more query columns per group and kv
 * head, by the LDS-staged prefix stage in partitions of its own); the rest of
 * every context per sequence in the same launch; the merge as in the split
 * path.  Other arguments, preconditions and returns
 * as for pa_decode_shared_prefix (context_lens[b] >= seq_shared_len[b], an
 * appended position past it); inconsistent group arrays give unspecified
 * output with memory accesses in bounds.
 */
pa_status pa_decode_shared_prefix_groups(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int32_t block_size, int32_t num_kv_heads, float scale,
                                         void* out, hipStream_t stream,
                                         int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         int64_t num_blocks, pa_dtype dtype, int32_t num_groups,
                                         const int32_t* group_start, const int32_t* group_shared_len,
                                         const int32_t* seq_shared_len, int32_t max_group_size,
                                         int32_t max_shared_len, int32_t partition_size, void* workspace,
                                         size_t workspace_bytes, const void* k_new, const void* v_new,
                                         const int64_t* slot_mapping);

/*
 * Workspace bytes for pa_decode_shared_prefix_groups: the split path's
 * layout with room for the prefix partials in front of each (sequence, head)
 * row, num_seqs * num_heads * (ceil(max_context_len / P) + E) * (head_dim + 2)
 * * 4 with E = max(1, ceil(max_context_len / 256)) (P = partition_size, 0
 * meaning 2048; the prefix launch's partitions are at least 256 tokens).
 * The call itself needs only ceil(max_context_len / P) + ceil(max_shared_len
 * / Pp) slots (Pp its prefix partition), or + 1 on the multi-query prefix
 * kernel.  0 for invalid arguments.
 */
size_t pa_decode_shared_prefix_groups_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                                     int32_t max_context_len, int32_t partition_size);

size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_context_len, int32_t shared_len,
                                              int32_t partition_size);

/*
 * pa_copy_blocks -- copy whole pages (K and V, every kv head) for
 * copy-on-write forks: page block_mapping[i][1] becomes a bit-exact copy of
 * page block_mapping[i][0].  Pairs act as if applied at once (sources and
 * destinations must be disjoint, destinations unique).  Pairs naming a page
 * outside [0, num_blocks) are skipped.
 * [Glossary, "Copy-on-Write Memory Forking"; Internals, "Copy-on-Write and
 * Prefix Sharing": a request that starts writing its own tokens gets a page
 * of its own]
 *
 *   k_cache/v_cache device, layouts above, read and written
 *   block_mapping device, [num_pairs][2] int64 (src, dst), read
 * Returns PA_OK (num_pairs == 0 is a no-op), PA_ERR_NULL, PA_ERR_ARG,
 * PA_ERR_UNSUPPORTED or PA_ERR_HIP.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                         hipStream_t stream);

/*
 * pa_decode_multi -- attention for several new tokens per sequence at once:
 * the draft tokens speculative decoding verifies over paged memory
 * [Internals, "The Mathematical Cause of KV Cache Fragmentation", closing
 * link], or a chunk of a prompt, with the paging and attention of
 * [Internals, "How PagedAttention Works" items 1-3].
 *
 * Sequence b has n_b = query_start[b + 1] - query_start[b] new tokens whose
 * K and V rows are already in its pages (pa_kv_append, or pa_copy_blocks
 * and pa_kv_append) at positions L_b - n_b .. L_b - 1, L_b = context_lens[b]
 * counting them.  Row query_start[b] + j of q holds the queries of new token
 * j (0 <= j < n_b); it attends, head by head as in pa_decode, over positions
 * 0 .. L_b - n_b + j (causal among the new tokens), and the result goes to
 * the same row of out.
 *
 *   q, out       device, [num_tokens][num_heads][head_dim] bf16, 16-byte aligned
 *   query_start  device, [num_seqs + 1] int32, non-decreasing, query_start[0] = 0,
 *                query_start[num_seqs] <= num_tokens; read
 *   k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
 *   scale, num_heads, head_dim, max_blocks_per_seq, max_context_len,
 *   num_blocks, partition_size, reuse, workspace  as for pa_decode
 *   max_query_len  host bound on every n_b, 1 .. 1024
 *   workspace      pa_decode_multi_workspace_size() bytes when the split
 *                  path runs (else ignored); caller-owned
 *
 * Two kernels serve the call, chosen on the host from the head group G =
 * num_heads / num_kv_heads and max_query_len: below 64 query columns
 * (G * max_query_len) per (sequence, kv head), as in speculative
 * verification, each wave reads its chunks of K/V for up to 32 columns;
 * from 64 on (a prompt chunk), each K/V chunk is staged once in LDS for 128
 * columns, the product being dense enough for the matrix cores.  Either
 * gives the same result up to rounding order.
 *
 * Out-of-range device values are clamped (rows to [0, num_tokens), n_b to
 * max_query_len and to L_b); rows no sequence covers are not part of the
 * result (unspecified).  bf16 only: PA_ERR_UNSUPPORTED for fp32.  Returns
 * PA_OK (num_seqs == 0 or num_tokens == 0 is a no-op), PA_ERR_NULL,
 * PA_ERR_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE or PA_ERR_HIP.
 */
pa_status pa_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start, int32_t block_size, int32_t num_kv_heads,
                          float scale, void* out, hipStream_t stream, int32_t num_seqs,
                          int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                          int32_t max_blocks_per_seq, int32_t max_context_len, int32_t max_query_len,
                          int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                          pa_kv_reuse reuse, void* workspace, size_t workspace_bytes);

/*
 * pa_decode_multi_append -- the step's append and pa_decode_multi in one
 * call (no separate pa_kv_append; one launch below 64 query columns per
 * (sequence, kv head), where the attention kernel stores the rows itself,
 * and an append launch before the attention from 64 on).  k_new, v_new (device,
 * [num_tokens][num_kv_heads][head_dim] bf16, 16-byte aligned, read) are the
 * new tokens' K and V rows, row for row aligned with q: row
 * query_start[b] + j goes to position L_b - n_b + j of sequence b, i.e. to
 * page block_tables[b][pos / block_size] at offset pos % block_size, which
 * must already be the sequence's own page (allocated, copied on write).  A
 * page id outside [0, num_blocks) writes nothing there.  Every other
 * argument, the result and the status codes are those of pa_decode_multi
 * (PA_ERR_NULL also for a missing k_new / v_new); outputs and caches equal
 * pa_kv_append of the same rows followed by pa_decode_multi, bit for bit.
 */
pa_status pa_decode_multi_append(const void* k_new, const void* v_new, const void* q, void* k_cache,
                                 void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start, int32_t block_size, int32_t num_kv_heads,
                                 float scale, void* out, hipStream_t stream, int32_t num_seqs,
                                 int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t max_context_len, int32_t max_query_len,
                                 int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                                 pa_kv_reuse reuse, void* workspace, size_t workspace_bytes);

/* Partition size pa_decode_multi uses for these sizes (0 = single pass,
 * -1 = invalid request); partition_size as for pa_decode. */
int32_t pa_decode_multi_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t max_query_len,
                                       int32_t partition_size);

/* Workspace bytes pa_decode_multi needs (0 when it runs in one pass). */
size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                                      int32_t max_query_len, int32_t partition_size);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
