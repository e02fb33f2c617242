// Internal declarations shared by the host API and the kernel translation
// units of libpa.  Not installed; the public interface is include/pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa_impl {

// Everything a decode launch needs, resolved and validated on the host.
constexpr int kWideWaves = 12;   // decode workgroup that fills a compute unit (3 waves per SIMD)
constexpr int kPairWaves = 5;    // decode workgroup of the longest-first single pass
constexpr int kSortMax = 256;    // sequences the kernels rank for longest-first order

struct DecodeParams {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const void* k_new;     // fused append: new rows [num_seqs][num_kv_heads][head_dim], or null
    const void* v_new;
    const int64_t* append_mask;   // fused append: sequences with a negative entry append nothing (or null)
    void* out;             // final output (single pass)
    float* ws;             // partials (split): acc | m | l, see ws_* helpers
    float scale_log2;      // scale * log2(e): scores are kept in log2 units
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t group;         // num_heads / num_kv_heads
    int32_t head_dim;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int64_t num_blocks;
    int32_t partition;     // tokens per partition (single pass: covers max_context_len)
    int32_t max_parts;     // partitions per (seq, head) in the workspace (1 = single pass)
    int32_t split;         // 1: write partials to ws, 0: write out
    int32_t stream_kv;     // 1: no page is shared between sequences (streaming loads)
    int32_t waves;         // decode kernel: waves per workgroup (4, or 12 to fill a compute unit)
    int32_t order_by_length;  // 1: workgroups take sequences longest first (one-pass launches)
    int32_t first_token;   // decode_mfma split: positions below this are left to another launch (0: none)
    // multi-query launches only (null / 0 otherwise)
    const int32_t* query_start;   // [num_seqs + 1]: query rows of each sequence
    int32_t num_tokens;    // rows of q / out
    int32_t max_query_len; // bound on query rows per sequence
    int32_t col_groups;    // column groups of 16 * col_tiles (query token, head) pairs per kv head
    int32_t all_visible;   // 1: every query row sees all L positions (a shared prefix), 0: causal rows
    int32_t uniform_len;   // > 0: every sequence's context length (context_lens is not read)
    int32_t ws_parts;      // > 0: partial slots per workspace row (else max_parts)
    int32_t slot_shift;    // split: partition p writes workspace slot p + slot_shift
    // shared-prefix groups: sequence b's own first position (its group's
    // shared length; replaces first_token, and its slot shift is 1 when it
    // ends inside a partition), or null
    const int32_t* seq_first;
    int32_t table_rows_from_queries;  // multi-query: sequence b reads the table row of its first query row
    // decode_mfma, shared-page loads (partition p in slot p): partitions
    // below this one lie below first_token for every sequence; the grid
    // starts at it (0: every partition)
    int32_t first_part;
    // with seq_first: the partition the prefix launch used (0: partition)
    int32_t prefix_partition;
};

struct ReduceParams {
    const float* ws;
    const int32_t* context_lens;
    void* out;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t head_dim;
    int32_t max_context_len;
    int32_t partition;
    int32_t max_parts;
    // multi-query merge: rows are query tokens; a row's context is found
    // through query_start [num_groups + 1] and the per-sequence context_lens
    const int32_t* query_start;
    int32_t num_groups;
    int32_t max_query_len;
    // a row merges slots 0 .. ceil(L / partition) + slot_shift - 1 (a
    // shared prefix's partials come first, read in partitions of their own)
    int32_t slot_shift;
    const int32_t* seq_first;   // or per sequence (seq_slot_shift of its shared length)
    int32_t prefix_partition;   // with seq_first: the prefix launch's partition (0: partition)
};

// Slot shift of a sequence whose own positions start at `first`, after a
// prefix launch that wrote ceil(first / Pp) partials of its first positions
// (Pp = prefix_partition, or P when 0) to slots 0 ..: its own partitions of P
// tokens start with partition floor(first / P), which goes to the next slot.
__host__ __device__ inline int seq_slot_shift(int first, int P, int prefix_partition) {
    const int Pp = prefix_partition > 0 ? prefix_partition : P;
    return (first + Pp - 1) / Pp - first / P;
}

// Workspace layout for the split path (all fp32):
//   acc [num_seqs][num_heads][max_parts][head_dim]   unnormalised accumulator
//   m   [num_seqs][num_heads][max_parts]             running max (log2 units)
//   l   [num_seqs][num_heads][max_parts]             running sum of 2^(s - m)
__host__ __device__ inline size_t ws_rows(int32_t num_seqs, int32_t num_heads, int32_t max_parts) {
    return (size_t)num_seqs * (size_t)num_heads * (size_t)max_parts;
}

hipError_t launch_kv_append(const void* k, const void* v, const int64_t* slot_mapping,
                            void* k_cache, void* v_cache, int32_t num_tokens,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, pa_dtype dtype, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                              int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                              hipStream_t stream);

hipError_t launch_append_newest(const DecodeParams& p, pa_dtype dtype, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, pa_dtype dtype, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_reduce(const ReduceParams& p, pa_dtype dtype, hipStream_t stream);
hipError_t launch_decode_multi(const DecodeParams& p, int col_tiles, hipStream_t stream);
// Shared-prefix stage with LDS-staged K/V (`pre`, 4-wave workgroups) and
// the shared-page decode path over the rest of every context (`rest`, its
// first_part and slot shifts set) in one launch; the stage's query columns
// per workgroup, and the chunk its partition sizes must be a multiple of.
hipError_t launch_decode_prefix_rest(const DecodeParams& pre, const DecodeParams& rest, hipStream_t stream);
// the same with the multi-query kernel as the prefix stage (`pre` with
// shared-page loads, 4-wave workgroups, col_tiles 16-column tiles each)
hipError_t launch_decode_multi_rest(const DecodeParams& pre, int col_tiles, const DecodeParams& rest,
                                    hipStream_t stream);
// The LDS-staged kernel as the multi-query kernel of many columns per
// (sequence, kv head): causal rows, col_groups groups of
// decode_prefix_columns() columns, one pass (split 0) or partials.
hipError_t launch_decode_multi_wide(const DecodeParams& p, hipStream_t stream);
// A multi-query call's new rows (bf16) into their slots, before that kernel.
hipError_t launch_append_multi_rows(const DecodeParams& p, hipStream_t stream);
int decode_prefix_columns();
int decode_prefix_chunk();

}  // namespace pa_impl
