// Host side of libpa: argument validation, path selection and launches.
// Every entry point validates on the host before any HIP call, then enqueues
// asynchronously on the caller's stream.  Nothing is allocated, nothing is
// synchronised, no exception leaves the library.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pa_internal.h"

using pa_impl::DecodeParams;
using pa_impl::ReduceParams;

namespace {

constexpr int32_t kSplitAbove = 512;         // contexts up to this length run in one pass
constexpr int32_t kMinPartition = 256;       // library-default partition sizes: powers of two
constexpr int32_t kMaxPartition = 4096;      // in [kMinPartition, kMaxPartition]
constexpr int64_t kFillUnits = 1024;         // workgroups that keep 256 CUs busy (4 resident each)
constexpr int64_t kMinUnits = 1024;          // below this, fall back to the smallest partition
constexpr int32_t kChunk = 32;               // partitions are whole 32-token chunks
constexpr int32_t kMaxGroup = 16;            // query heads per kv head
constexpr uint64_t kMaxGrid = 1ull << 31;    // workgroups per launch
constexpr int32_t kMaxQueryLen = 1024;       // multi-query: new tokens per sequence
constexpr int64_t kMultiFill = 256;          // multi-query: workgroups that keep every CU busy
constexpr int64_t kMultiWideFill = 512;      // the same for the LDS-staged kernel (two per CU)
constexpr int32_t kMultiMaxPartition = 8192;
constexpr int64_t kPrefixFill = 512;         // shared-prefix launch: workgroups that fill the chip (two per CU)
// shared-prefix call, partition_size 0: measured best on 100 sequences over a
// 9,984-token prefix (91.5 us; 97.8 at 1024) and on 8 beams over 32,768
// tokens (35.5 us; 38.9 at 1024)
constexpr int32_t kSharedPrefixPartition = 2048;
// streaming-load decode default (see default_stream_partition)
constexpr int64_t kOnePassPairs = 2048;      // (sequence, kv head) pairs that make a single pass
constexpr int64_t kOnePassShortPairs = 1024; // ... or this many when no context exceeds
constexpr int32_t kOnePassShortContext = 4096;
constexpr int32_t kStreamMinPartition = 1024;
constexpr int32_t kStreamMaxPartition = 8192;
constexpr int64_t kStreamFillUnits = 768;    // three 12-wave workgroups per compute unit
constexpr int32_t kWidePartition = 2048;     // streaming partitions this long run 12-wave workgroups
constexpr int64_t kOrderedPairs = 512;       // one pass, longest sequences first, from this many pairs ...
constexpr int64_t kOrderedPairsEnd = 1024;   // ... up to (not including) this many: two to four rounds
constexpr int32_t kOrderedContext = 8192;    // and no context longer than this
constexpr int64_t kMultiOrderedUnits = 1024; // multi-query one pass: longest first up to this many workgroups
constexpr int32_t kSortMaxSeqs = pa_impl::kSortMax;   // the kernels rank at most this many sequences

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bool valid_dtype(pa_dtype d) { return d == PA_F32 || d == PA_BF16; }

size_t elem_bytes(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }

pa_status shape_status(int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    if (num_kv_heads <= 0) return PA_ERR_ARG;
    if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

int32_t parts_for(int32_t max_context_len, int32_t partition) {
    return (int32_t)(((int64_t)max_context_len + partition - 1) / partition);
}

// Library default for shared pages (and the streaming rule's fallback): the
// longest partition that still leaves at least 4 partitions in the longest
// context and kFillUnits (sequence, kv head, partition) workgroups; longer
// partitions mean fewer partials to write and merge and less per-workgroup
// set-up, shorter ones better balance over ragged lengths.  Tiny batches drop
// to kMinPartition for parallelism.
int32_t default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
    if (max_context_len <= kSplitAbove) return 0;
    const int64_t pairs = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
    auto units = [&](int32_t P) { return pairs * parts_for(max_context_len, P); };
    int32_t P = kMaxPartition;
    while (P > kSplitAbove && ((int64_t)P * 4 > max_context_len || units(P) < kFillUnits)) P /= 2;
    if (units(P) < kMinUnits) P = kMinPartition;
    return P;
}

// One pass with the workgroups taking sequences longest first: 512 to 1023
// (sequence, kv head) pairs (two to four rounds of 12-wave workgroups), at
// most kSortMaxSeqs sequences, no context past kOrderedContext.
bool ordered_one_pass(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    return pairs >= kOrderedPairs && pairs < kOrderedPairsEnd && num_seqs <= kSortMaxSeqs &&
           max_context_len > kSplitAbove && max_context_len <= kOrderedContext;
}

// Library default for streaming loads (no page shared between sequences).
// Measured on MI355X over uniform and ragged batches: when the (sequence,
// kv head) pairs alone give several rounds of 12-wave workgroups, a single
// pass wins -- no partials, no merge, and the unequal lengths even out over
// the rounds; with two to four rounds it wins when the workgroups take the
// longest sequences first.  Otherwise the longest power-of-two partition in
// [kStreamMinPartition, kStreamMaxPartition], shorter than the longest
// context, that still gives kStreamFillUnits workgroups; the shared-page
// rule when none does.
int32_t default_stream_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
    if (max_context_len <= kSplitAbove) return 0;
    const int64_t pairs = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
    if (pairs >= kOnePassPairs || (pairs >= kOnePassShortPairs && max_context_len <= kOnePassShortContext))
        return 0;
    if (ordered_one_pass(num_seqs, num_kv_heads, max_context_len)) return 0;
    for (int32_t P = kStreamMaxPartition; P >= kStreamMinPartition; P /= 2)
        if (P < max_context_len && pairs * parts_for(max_context_len, P) >= kStreamFillUnits) return P;
    return default_partition(num_seqs, num_kv_heads, max_context_len);
}

int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                          int32_t partition_size, bool stream) {
    if (max_context_len < 0) return -1;
    if (partition_size == -1) return 0;
    if (partition_size == 0)
        return stream ? default_stream_partition(num_seqs, num_kv_heads, max_context_len)
                      : default_partition(num_seqs, num_kv_heads, max_context_len);
    if (partition_size < kChunk || partition_size % kChunk != 0) return -1;
    return partition_size;
}

size_t workspace_bytes_for(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t max_context_len, int32_t partition) {
    if (partition <= 0) return 0;
    const int32_t parts = parts_for(max_context_len, partition);
    return pa_impl::ws_rows(num_seqs, num_heads, parts) * (size_t)(head_dim + 2) * sizeof(float);
}

// Shared-prefix call: the prefix launch reads positions [0, shared_len) in
// partitions of Pp tokens, whose partials take workspace slots 0 .. np - 1
// of every row; the per-sequence launch reads from shared_len on in
// partitions of P, partition p >= q0 = shared_len / P writing slot p + shift
// with shift = np - q0 (negative when Pp > P), so each row's partials stay
// contiguous and the merge takes slots 0 .. ceil(L / P) + shift - 1.  The
// per-wave-loads multi-query launch keeps Pp = P: prefix partitions of 1024
// or 512 tokens under P = 2048 measured no faster with it (100 sequences
// over 9,984 shared tokens: 94.5 and 113.8 us against 95.3; 8 beams: 39.7
// and 44.2 against 38.2); the LDS-staged launch sizes Pp for itself.
struct PrefixShape {
    int32_t Pp;
    int32_t np;
    int32_t shift;
    int32_t row;     // slots per workspace row
    int32_t tiles;   // 16-column tiles per prefix workgroup
    int32_t col_groups;
    bool wide;       // the LDS-staged prefix kernel (128 columns per workgroup)
};

// Many query columns per kv head (a prompt forked to many sequences): the
// LDS-staged prefix kernel, whose 4-wave workgroups stage each chunk of
// shared pages once for 128 columns, in one launch with the rest of every
// context (the two stages share the compute units).  Its partitions are
// multiples of its 64-token chunk, sized so that the launch starts about one
// prefix workgroup per compute unit (kPrefixWideFill waves), which leaves each
// unit's second workgroup slot to the rest of the contexts.  Measured on
// 100 sequences x 4 heads over a 9,984-token prefix and on 4 prompts x 25
// sequences, step in us, fill 768 / 1024 / 1280 / 1536 / 2048 waves:
// 58.8 / 51.8 / 51.1 / 51.2 / 57.3 and 39.4 / 41.5 / 42.8 / 43.9 / 48.6.
// (The two stages as separate launches, 8-wave prefix workgroups two
// waves per SIMD: 61.6 and 51.0.)
constexpr int32_t kPrefixWideMinCols = 64;
constexpr int64_t kPrefixWideFill = 1024;

int32_t prefix_wide_partition(int64_t units_per_part, int32_t shared_len) {
    const int32_t chunk = pa_impl::decode_prefix_chunk();
    const int64_t wgs = kPrefixWideFill / 4;
    const int64_t parts = (wgs + units_per_part - 1) / units_per_part;
    int64_t Pp = (shared_len + parts - 1) / parts;
    Pp = (Pp + chunk - 1) / chunk * chunk;
    if (Pp < 4 * chunk) Pp = 4 * chunk;
    return (int32_t)Pp;
}

int32_t multi_col_tiles(int32_t group, int32_t max_query_len);
int32_t multi_col_groups(int32_t group, int32_t max_query_len);

PrefixShape prefix_shape(int32_t num_seqs, int32_t group, int32_t num_kv_heads, int32_t max_context_len,
                         int32_t shared_len, int32_t P) {
    PrefixShape sh;
    // Two 16-column tiles per workgroup halve how often a shared page is
    // read; one tile runs three waves per SIMD instead of two and doubles
    // the workgroups.  One only when two would leave a single column group
    // and fewer than kPrefixFill workgroups (two per compute unit at this
    // kernel's occupancy).  Measured: 8 beams over 32,768 tokens (one group
    // of 32 columns) 41.2 us with two tiles, 37.3 with one; 100 sequences
    // over a 9,216-token prefix (13 groups) 108 us with two, 125 with one,
    // and at 416 workgroups still 111 against 138.
    sh.tiles = multi_col_tiles(group, num_seqs);
    const int32_t parts_at_P = (shared_len + P - 1) / P;
    if (sh.tiles == 2 && multi_col_groups(group, num_seqs) == 1 && (int64_t)num_kv_heads * parts_at_P < kPrefixFill)
        sh.tiles = 1;
    sh.col_groups = (int32_t)(((int64_t)group * num_seqs + 16 * sh.tiles - 1) / (16 * sh.tiles));
    sh.Pp = P;
    sh.wide = (int64_t)group * num_seqs >= kPrefixWideMinCols;
    if (sh.wide) {
        const int32_t cols = pa_impl::decode_prefix_columns();
        sh.col_groups = (int32_t)(((int64_t)group * num_seqs + cols - 1) / cols);
        sh.Pp = prefix_wide_partition((int64_t)num_kv_heads * sh.col_groups, shared_len);
    }
    sh.np = shared_len > 0 ? (shared_len + sh.Pp - 1) / sh.Pp : 0;
    sh.shift = sh.np - shared_len / P;
    sh.row = parts_for(max_context_len, P) + sh.shift;
    if (sh.row < 1) sh.row = 1;
    return sh;
}

struct Plan {
    DecodeParams p;
    pa_dtype dtype;
    bool use_mfma;
    int32_t partition;   // 0 = single pass
};

// Shared validation of pa_decode / pa_decode_partition.  Returns PA_OK with
// `plan` filled, or the first error found.  `need_out` is false for the
// partition-only stage; `force_split` requires the split path.
pa_status make_plan(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t block_size, int32_t num_kv_heads, float scale, void* out,
                    int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                    pa_dtype dtype, int32_t partition_size, pa_kernel kernel, pa_kv_reuse reuse,
                    void* workspace, size_t workspace_bytes, bool need_out, bool force_split,
                    Plan* plan, bool check_workspace = true) {
    if (!valid_dtype(dtype)) return PA_ERR_ARG;
    if (kernel != PA_KERNEL_AUTO && kernel != PA_KERNEL_VALU && kernel != PA_KERNEL_MFMA)
        return PA_ERR_ARG;
    if (reuse != PA_KV_AUTO && reuse != PA_KV_STREAM && reuse != PA_KV_SHARED) return PA_ERR_ARG;
    pa_status st = shape_status(num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (num_heads <= 0 || num_heads % num_kv_heads != 0) return PA_ERR_ARG;
    if (num_heads / num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0) return PA_ERR_ARG;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_ARG;
    if (num_blocks > (int64_t)INT32_MAX + 1) return PA_ERR_ARG;      // table entries are int32
    if (!isfinite(scale)) return PA_ERR_ARG;
    int32_t partition = resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size,
                                          reuse != PA_KV_SHARED);
    if (partition < 0) return PA_ERR_ARG;
    if (force_split && partition <= 0) return PA_ERR_ARG;
    if (!force_split && partition > 0 && max_context_len == 0) partition = 0;   // nothing to split
    if (kernel == PA_KERNEL_MFMA && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (num_seqs < 0) return PA_ERR_ARG;

    plan->dtype = dtype;
    plan->partition = partition;
    plan->use_mfma = kernel == PA_KERNEL_MFMA || (kernel == PA_KERNEL_AUTO && dtype == PA_BF16);
    if (num_seqs == 0) return PA_OK;

    if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
    if (need_out && !out) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ARG;
    if (need_out && !aligned16(out)) return PA_ERR_ARG;

    const int32_t parts = partition > 0 ? parts_for(max_context_len, partition) : 1;
    if ((uint64_t)num_seqs * (uint64_t)num_kv_heads * (uint64_t)parts >= kMaxGrid)
        return PA_ERR_UNSUPPORTED;
    if (partition > 0 && check_workspace) {
        const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, max_context_len, partition);
        if (need > 0) {
            if (!workspace) return PA_ERR_WORKSPACE;
            if (!aligned16(workspace)) return PA_ERR_ARG;
            if (workspace_bytes < need) return PA_ERR_WORKSPACE;
        }
    }

    DecodeParams& p = plan->p;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.k_new = nullptr;
    p.v_new = nullptr;
    p.append_mask = nullptr;
    p.out = out;
    p.ws = static_cast<float*>(workspace);
    p.scale_log2 = scale * 1.4426950408889634f;     // log2(e): scores in log2 units
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_heads / num_kv_heads;
    p.head_dim = head_dim;
    p.block_size = block_size;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = max_context_len;
    p.num_blocks = num_blocks;
    p.stream_kv = reuse != PA_KV_SHARED;
    // 12-wave workgroups for long streaming work units: partitions of
    // kWidePartition tokens or more, or a single pass over enough pairs.  A
    // longest-first single pass (two to four rounds of 12 waves) runs
    // 5-wave workgroups instead (8B-shaped launch, 512 pairs: 12 waves 94.4,
    // 8 waves 94.2, 6 waves 93.8, 5 waves 93.4 us; 4-wave workgroups capped
    // at three per SIMD 100.3).  Held to three waves per SIMD, two 5-wave
    // workgroups fit on one compute unit where two 6-wave ones do not (a
    // per-workgroup timeline of the 6-wave kernel shows 256 resident), so
    // the pairs go longest first with twice as many in flight.
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    const bool ordered = p.stream_kv && partition == 0 && ordered_one_pass(num_seqs, num_kv_heads, max_context_len);
    p.waves = p.stream_kv && (partition >= kWidePartition ||
                              (partition == 0 && pairs >= kOnePassShortPairs && max_context_len > kSplitAbove))
                  ? pa_impl::kWideWaves : (ordered ? pa_impl::kPairWaves : 4);
    p.order_by_length = ordered ? 1 : 0;
    p.query_start = nullptr;
    p.num_tokens = 0;
    p.max_query_len = 0;
    p.col_groups = 0;
    p.first_token = 0;
    p.all_visible = 0;
    p.uniform_len = 0;
    p.ws_parts = 0;
    p.slot_shift = 0;
    p.seq_first = nullptr;
    p.table_rows_from_queries = 0;
    p.first_part = 0;
    p.prefix_partition = 0;
    if (partition > 0) {
        p.partition = partition;
        p.max_parts = parts;
        p.split = 1;
    } else {
        const int32_t whole = max_context_len < 1 ? 1 : max_context_len;
        p.partition = (int32_t)(((int64_t)whole + kChunk - 1) / kChunk * kChunk);
        p.max_parts = 1;
        p.split = 0;
    }
    return PA_OK;
}

pa_status hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

pa_status launch_plan(const Plan& plan, hipStream_t stream) {
    if ((uint64_t)plan.p.num_seqs * plan.p.num_kv_heads * plan.p.max_parts == 0) return PA_OK;
    if (plan.use_mfma) return hip_status(pa_impl::launch_decode_mfma(plan.p, stream));
    return hip_status(pa_impl::launch_decode_valu(plan.p, plan.dtype, stream));
}

pa_status launch_reduce(const Plan& plan, const int32_t* context_lens, void* out, hipStream_t stream) {
    ReduceParams r;
    r.query_start = nullptr;
    r.num_groups = 0;
    r.max_query_len = 0;
    r.slot_shift = plan.p.slot_shift;
    r.seq_first = plan.p.seq_first;
    r.prefix_partition = plan.p.prefix_partition;
    r.ws = plan.p.ws;
    r.context_lens = context_lens;
    r.out = out;
    r.num_seqs = plan.p.num_seqs;
    r.num_heads = plan.p.num_heads;
    r.head_dim = plan.p.head_dim;
    r.max_context_len = plan.p.max_context_len;
    r.partition = plan.p.partition;
    r.max_parts = plan.p.ws_parts > 0 ? plan.p.ws_parts : plan.p.max_parts;
    return hip_status(pa_impl::launch_decode_reduce(r, plan.dtype, stream));
}

// Multi-query column tiling: (query token, head) pairs of one kv head, 16
// per MFMA tile, one tile per workgroup when they fit, else two.
int32_t multi_col_tiles(int32_t group, int32_t max_query_len) {
    return (int64_t)group * max_query_len <= 16 ? 1 : 2;
}

int32_t multi_col_groups(int32_t group, int32_t max_query_len) {
    const int64_t per = 16 * multi_col_tiles(group, max_query_len);
    return (int32_t)(((int64_t)group * max_query_len + per - 1) / per);
}

// Multi-query default: the fewest partitions that still give kMultiFill
// workgroups.  A multi-query workgroup writes a partial row per (query
// token, head) column, so partials and the merge cost several times what
// they cost a decode step, and long partitions win as soon as the chip is
// full: one pass when (sequence, column group, kv head) units alone fill it,
// else the longest power-of-two partition in [kMinPartition,
// kMultiMaxPartition] that does (kMinPartition when none does).
int32_t default_multi_partition(int64_t units, int32_t max_context_len, int64_t fill) {
    if (max_context_len <= kSplitAbove || units >= fill) return 0;
    for (int32_t P = kMultiMaxPartition; P >= kMinPartition; P /= 2) {
        if (P >= max_context_len) continue;         // one partition: a single pass does it without the merge
        if (units * parts_for(max_context_len, P) >= fill) return P;
    }
    return kMinPartition;
}

int32_t resolve_multi_partition(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t max_context_len, int32_t max_query_len, int32_t partition_size) {
    if (num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads != 0 || max_query_len < 1)
        return -1;
    if (partition_size != 0)
        return resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size, true);
    if (max_context_len < 0) return -1;
    // From kPrefixWideMinCols columns per (sequence, kv head) the LDS-staged
    // kernel runs, with 128-column groups and two workgroups per compute
    // unit.  Measured, 16 sequences x L U[512, 4096], 4 heads per kv head,
    // n = 16 / 32 / 64 new tokens: one pass (128 / 128 / 256 workgroups)
    // 135 / 138 / 142 us, split to reach 512 workgroups 62 / 72 / 123 us
    // (the per-wave kernel: 62 / 110 / 207 us).
    const int32_t group = num_heads / num_kv_heads;
    const bool wide = (int64_t)group * max_query_len >= kPrefixWideMinCols;
    const int64_t cols_per_group = wide ? pa_impl::decode_prefix_columns() : 16 * multi_col_tiles(group, max_query_len);
    const int64_t col_groups = ((int64_t)group * max_query_len + cols_per_group - 1) / cols_per_group;
    const int64_t units = (int64_t)(num_seqs > 0 ? num_seqs : 1) * col_groups * num_kv_heads;
    return default_multi_partition(units, max_context_len, wide ? kMultiWideFill : kMultiFill);
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_ARG: return "invalid argument (size, count, alignment or option out of range)";
        case PA_ERR_UNSUPPORTED: return "unsupported shape (head_dim 64/128, block_size 16/32, "
                                        "<= 16 query heads per kv head, bf16 for the MFMA kernel)";
        case PA_ERR_WORKSPACE: return "workspace missing or smaller than pa_decode_workspace_size()";
        case PA_ERR_HIP: return "HIP runtime error while launching";
        case PA_ERR_OUT_OF_PAGES: return "out of physical pages: the page pool is exhausted";
        case PA_ERR_NOT_FOUND: return "no sequence with that id";
        case PA_ERR_HOST_MEMORY: return "host memory allocation failed";
        case PA_ERR_SCRATCH: return "the split path needs more than the library's static scratch "
                                    "(PA_STATIC_SCRATCH_BYTES); pass a workspace to pa_decode instead";
    }
    return "unknown status";
}

int32_t pa_version(void) { return 331; }

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                 int32_t partition_size, pa_kv_reuse reuse) {
    if (reuse != PA_KV_AUTO && reuse != PA_KV_STREAM && reuse != PA_KV_SHARED) return -1;
    return resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size, reuse != PA_KV_SHARED);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                                pa_kv_reuse reuse) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
    if (reuse != PA_KV_AUTO && reuse != PA_KV_STREAM && reuse != PA_KV_SHARED) return 0;
    const int32_t partition = resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size,
                                                reuse != PA_KV_SHARED);
    if (partition <= 0) return 0;
    return workspace_bytes_for(num_seqs, num_heads, head_dim, max_context_len, partition);
}

pa_status pa_kv_append(const void* k, const void* v, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache,
                       int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                       hipStream_t stream) {
    if (!valid_dtype(dtype)) return PA_ERR_ARG;
    pa_status st = shape_status(num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (num_tokens < 0 || num_blocks <= 0) return PA_ERR_ARG;
    if ((uint64_t)num_tokens * (uint64_t)num_kv_heads >= (1ull << 33)) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ARG;
    return hip_status(pa_impl::launch_kv_append(k, v, slot_mapping, k_cache, v_cache, num_tokens,
                                                num_kv_heads, head_dim, block_size, num_blocks,
                                                dtype, stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                         hipStream_t stream) {
    if (!valid_dtype(dtype)) return PA_ERR_ARG;
    pa_status st = shape_status(num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (num_pairs < 0 || num_blocks <= 0) return PA_ERR_ARG;
    if (num_pairs >= (1 << 24)) return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_kv_heads * head_dim * block_size * (int64_t)elem_bytes(dtype) > (1ll << 30))
        return PA_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !block_mapping) return PA_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ARG;
    return hip_status(pa_impl::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs,
                                                  num_kv_heads, head_dim, block_size, num_blocks,
                                                  dtype, stream));
}

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t block_size, int32_t num_kv_heads, float scale,
                    void* out, hipStream_t stream,
                    int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t max_context_len,
                    int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                    pa_kernel kernel, pa_kv_reuse reuse, void* workspace,
                    size_t workspace_bytes) {
    Plan plan;
    pa_status st = make_plan(q, k_cache, v_cache, block_tables, context_lens, block_size,
                             num_kv_heads, scale, out, num_seqs, num_heads, head_dim,
                             max_blocks_per_seq, max_context_len, num_blocks, dtype,
                             partition_size, kernel, reuse, workspace, workspace_bytes,
                             /*need_out=*/true, /*force_split=*/false, &plan);
    if (st != PA_OK || num_seqs == 0) return st;
    st = launch_plan(plan, stream);
    if (st != PA_OK || plan.partition == 0) return st;
    return launch_reduce(plan, context_lens, out, stream);
}

}  // extern "C"

// ---- pa_decode_noalloc: the split path's partials in a static device array
//
// One array per GPU, in device memory the code object brings with it, so a
// call makes no allocation.  In host code `scratch` names a host-side shadow,
// not device memory: only the address hipGetSymbolAddress returns for the
// device that runs the call may reach a kernel.  That address is looked up
// once per device, with the device current, and kept.
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the device `stream` belongs to (the
// current device for the null stream); the lookup runs with that device
// current and restores the caller's current device afterwards.
pa_status scratch_on_stream_device(hipStream_t stream, void** ptr) {
    int dev = -1;
    if (stream != nullptr) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(stream, &sd) != hipSuccess) return PA_ERR_HIP;
        dev = (int)sd;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return PA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxScratchDevices) return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return PA_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return PA_ERR_HIP;
        void* found = nullptr;
        const hipError_t e = hipGetSymbolAddress(&found, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return PA_ERR_HIP;
        if (e != hipSuccess || found == nullptr) return PA_ERR_HIP;
        g_scratch_ptr[dev] = found;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t block_size, int32_t num_kv_heads, float scale,
                            void* out, hipStream_t stream,
                            int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                            pa_kernel kernel, pa_kv_reuse reuse) {
    Plan plan;
    pa_status st = make_plan(q, k_cache, v_cache, block_tables, context_lens, block_size,
                             num_kv_heads, scale, out, num_seqs, num_heads, head_dim,
                             max_blocks_per_seq, max_context_len, num_blocks, dtype,
                             partition_size, kernel, reuse, nullptr, 0,
                             /*need_out=*/true, /*force_split=*/false, &plan,
                             /*check_workspace=*/false);
    if (st != PA_OK || num_seqs == 0) return st;
    if (plan.partition > 0) {
        const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, max_context_len, plan.partition);
        if (need > (size_t)PA_STATIC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
        void* ws = nullptr;
        st = scratch_on_stream_device(stream, &ws);
        if (st != PA_OK) return st;
        plan.p.ws = static_cast<float*>(ws);
    }
    st = launch_plan(plan, stream);
    if (st != PA_OK || plan.partition == 0) return st;
    return launch_reduce(plan, context_lens, out, stream);
}

pa_status pa_decode_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           const void* q, void* k_cache, void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t block_size, int32_t num_kv_heads, float scale,
                           void* out, hipStream_t stream,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, int32_t max_context_len,
                           int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                           pa_kernel kernel, pa_kv_reuse reuse, void* workspace,
                           size_t workspace_bytes) {
    Plan plan;
    pa_status st = make_plan(q, k_cache, v_cache, block_tables, context_lens, block_size,
                             num_kv_heads, scale, out, num_seqs, num_heads, head_dim,
                             max_blocks_per_seq, max_context_len, num_blocks, dtype,
                             partition_size, kernel, reuse, workspace, workspace_bytes,
                             /*need_out=*/true, /*force_split=*/false, &plan);
    if (st != PA_OK || num_seqs == 0) return st;
    if (!k_new || !v_new) return PA_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return PA_ERR_ARG;
    plan.p.k_new = k_new;
    plan.p.v_new = v_new;
    plan.p.append_mask = slot_mapping;
    if (plan.use_mfma && plan.p.waves == pa_impl::kWideWaves && plan.partition == 0 && !plan.p.order_by_length) {
        // One pass of 12-wave workgroups over many rounds (a 70B-shaped
        // batch: 2,048 workgroups, eight rounds): the rows go to the cache in
        // a launch of their own first (decode 373.4 + append 7.8 us), because
        // stores inside this read stream slow every workgroup's reads.  The
        // fused append measured 416.6 us however it was done -- storing the
        // row alone and waiting for it, or patching the chunk's registers and
        // writing whole 64-byte blocks, with ordinary or non-temporal stores
        // -- and 374.5 us with the registers patched and the stores taken
        // out.  The stores in workgroups of their own in the same launch,
        // after the decode grid or before it, cost more than the separate
        // launch (385.4 and 393.0 us).  The longest-first pass (two to four
        // rounds) keeps the fused append (8B-shaped step 94.0 us).
        st = hip_status(pa_impl::launch_append_newest(plan.p, dtype, stream));
        if (st != PA_OK) return st;
        plan.p.k_new = nullptr;
        plan.p.v_new = nullptr;
        plan.p.append_mask = nullptr;
    }
    st = launch_plan(plan, stream);
    if (st != PA_OK || plan.partition == 0) return st;
    return launch_reduce(plan, context_lens, out, stream);
}

pa_status pa_decode_partition(const void* q, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t block_size, int32_t num_kv_heads, float scale,
                              hipStream_t stream,
                              int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                              int32_t max_blocks_per_seq, int32_t max_context_len,
                              int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                              pa_kernel kernel, pa_kv_reuse reuse, void* workspace,
                              size_t workspace_bytes, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping) {
    if (partition_size <= 0) return PA_ERR_ARG;
    Plan plan;
    pa_status st = make_plan(q, k_cache, v_cache, block_tables, context_lens, block_size,
                             num_kv_heads, scale, nullptr, num_seqs, num_heads, head_dim,
                             max_blocks_per_seq, max_context_len, num_blocks, dtype,
                             partition_size, kernel, reuse, workspace, workspace_bytes,
                             /*need_out=*/false, /*force_split=*/true, &plan);
    if (st != PA_OK || num_seqs == 0) return st;
    if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_ARG;
    plan.p.k_new = k_new;
    plan.p.v_new = v_new;
    plan.p.append_mask = k_new ? slot_mapping : nullptr;
    return launch_plan(plan, stream);
}

pa_status pa_decode_reduce(const void* workspace, size_t workspace_bytes,
                           const int32_t* context_lens, void* out, hipStream_t stream,
                           int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                           int32_t max_context_len, int32_t partition_size, pa_dtype dtype) {
    if (!valid_dtype(dtype)) return PA_ERR_ARG;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0 || partition_size <= 0) return PA_ERR_ARG;
    const int32_t partition = resolve_partition(num_seqs, 1, max_context_len, partition_size, true);
    if (partition <= 0) return PA_ERR_ARG;
    if ((uint64_t)num_seqs * (uint64_t)num_heads >= kMaxGrid) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!context_lens || !out) return PA_ERR_NULL;
    if (!aligned16(out)) return PA_ERR_ARG;
    const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, max_context_len, partition);
    if (need > 0) {
        if (!workspace) return PA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PA_ERR_ARG;
        if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    }
    Plan plan;
    plan.dtype = dtype;
    plan.p.ws = static_cast<float*>(const_cast<void*>(workspace));
    plan.p.num_seqs = num_seqs;
    plan.p.num_heads = num_heads;
    plan.p.head_dim = head_dim;
    plan.p.max_context_len = max_context_len;
    plan.p.partition = partition;
    plan.p.max_parts = parts_for(max_context_len, partition);
    plan.p.ws_parts = 0;
    plan.p.slot_shift = 0;
    plan.p.seq_first = nullptr;
    return launch_reduce(plan, context_lens, out, stream);
}

size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_context_len, int32_t shared_len,
                                              int32_t partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return 0;
    if (head_dim <= 0 || max_context_len < 0 || shared_len < 0 || shared_len > max_context_len) return 0;
    if (partition_size == 0) partition_size = kSharedPrefixPartition;
    if (partition_size < kChunk || partition_size % kChunk != 0) return 0;
    const PrefixShape sh = prefix_shape(num_seqs, num_heads / num_kv_heads, num_kv_heads, max_context_len,
                                        shared_len, partition_size);
    return pa_impl::ws_rows(num_seqs, num_heads, sh.row) * (size_t)(head_dim + 2) * sizeof(float);
}

pa_status pa_decode_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t block_size, int32_t num_kv_heads, float scale,
                                  void* out, hipStream_t stream,
                                  int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int64_t num_blocks, pa_dtype dtype, int32_t shared_len,
                                  int32_t partition_size, void* workspace, size_t workspace_bytes,
                                  const void* k_new, const void* v_new, const int64_t* slot_mapping) {
    if (!valid_dtype(dtype)) return PA_ERR_ARG;
    if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (partition_size == 0) partition_size = kSharedPrefixPartition;
    if (partition_size < 0) return PA_ERR_ARG;
    if (num_seqs > kMaxQueryLen) return PA_ERR_UNSUPPORTED;     // the prefix launch's query rows
    Plan plan;
    pa_status st = make_plan(q, k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
                             scale, out, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                             max_context_len, num_blocks, dtype, partition_size, PA_KERNEL_MFMA,
                             PA_KV_SHARED, workspace, workspace_bytes,
                             /*need_out=*/true, /*force_split=*/true, &plan,
                             /*check_workspace=*/false);      // its own row length, checked below
    if (st != PA_OK) return st;
    if (shared_len < 0 || shared_len % block_size != 0 || shared_len > max_context_len) return PA_ERR_ARG;
    if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_ARG;
    if (num_seqs == 0) return PA_OK;
    const int32_t P = plan.partition;
    const PrefixShape sh = prefix_shape(num_seqs, plan.p.group, num_kv_heads, max_context_len, shared_len, P);
    const size_t need = pa_impl::ws_rows(num_seqs, num_heads, sh.row) * (size_t)(head_dim + 2) * sizeof(float);
    if (!workspace) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ARG;
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;

    // Prefix positions: a stage over sequence 0's table row whose query rows
    // are all num_seqs decode queries, every row seeing all shared_len
    // positions, in partitions of sh.Pp written to slots 0 .. sh.np - 1 of
    // every row (the LDS-staged prefix body, or the multi-query body below 64
    // columns), launched together with the rest of every context.
    DecodeParams m{};
    bool fused = false;                       // prefix stage in the launch of the rest
    if (sh.np > 0) {
        m.q = q;
        m.k_cache = k_cache;
        m.v_cache = v_cache;
        m.block_tables = block_tables;
        m.context_lens = context_lens;        // not read: uniform_len
        m.out = out;
        m.ws = plan.p.ws;
        m.scale_log2 = plan.p.scale_log2;
        m.num_seqs = 1;
        m.num_heads = num_heads;
        m.num_kv_heads = num_kv_heads;
        m.group = plan.p.group;
        m.head_dim = head_dim;
        m.block_size = block_size;
        m.max_blocks_per_seq = max_blocks_per_seq;
        m.max_context_len = max_context_len;
        m.num_blocks = num_blocks;
        m.partition = sh.Pp;
        m.max_parts = sh.np;
        m.ws_parts = sh.row;
        m.split = 1;
        m.waves = 4;
        m.query_start = nullptr;              // rows 0 .. num_seqs - 1
        m.num_tokens = num_seqs;
        m.max_query_len = num_seqs;
        m.col_groups = sh.col_groups;
        m.stream_kv = 0;                      // ordinary loads: the pages are shared
        m.all_visible = 1;
        m.uniform_len = shared_len;
        if ((uint64_t)num_kv_heads * m.col_groups * (m.max_parts + 8) >= kMaxGrid) return PA_ERR_UNSUPPORTED;
        fused = true;
    }
    // The rest of every context, sequence by sequence, from shared_len on
    // (with the fused append of pa_decode_append when new rows are given:
    // position L - 1 lies past the shared prefix), its partitions shifted
    // past the prefix slots, then the usual merge.
    plan.p.first_token = shared_len;
    plan.p.ws_parts = sh.row;
    plan.p.slot_shift = sh.shift;
    // the partitions wholly inside the prefix are not launched
    plan.p.first_part = plan.p.stream_kv ? 0 : shared_len / P;
    plan.p.k_new = k_new;
    plan.p.v_new = v_new;
    plan.p.append_mask = k_new ? slot_mapping : nullptr;
    if (!fused) st = launch_plan(plan, stream);
    else if (sh.wide) st = hip_status(pa_impl::launch_decode_prefix_rest(m, plan.p, stream));
    else st = hip_status(pa_impl::launch_decode_multi_rest(m, sh.tiles, plan.p, stream));
    if (st != PA_OK) return st;
    return launch_reduce(plan, context_lens, out, stream);
}

// Grouped call: prefix slots per row beyond the split path's row.  A group's
// prefix launch in partitions of P leaves one partly shared partition (one
// slot more); the LDS-staged prefix launch writes ceil(S / Pp) partials of
// its own partitions Pp >= 4 chunks, at most ceil(max_context_len / 256).
int32_t groups_extra_slots(int32_t max_context_len) {
    const int32_t wide = parts_for(max_context_len, 4 * pa_impl::decode_prefix_chunk());
    return wide > 1 ? wide : 1;
}

size_t pa_decode_shared_prefix_groups_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                                     int32_t max_context_len, int32_t partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
    if (partition_size == 0) partition_size = kSharedPrefixPartition;
    if (partition_size < kChunk || partition_size % kChunk != 0) return 0;
    return pa_impl::ws_rows(num_seqs, num_heads,
                            parts_for(max_context_len, partition_size) + groups_extra_slots(max_context_len)) *
           (size_t)(head_dim + 2) * sizeof(float);
}

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
                                         const int64_t* slot_mapping) {
    if (!valid_dtype(dtype)) return PA_ERR_ARG;
    if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (partition_size == 0) partition_size = kSharedPrefixPartition;
    if (partition_size < 0) return PA_ERR_ARG;
    if (num_groups < 0 || max_group_size < 1 || max_shared_len < 0) return PA_ERR_ARG;
    if (max_group_size > kMaxQueryLen) return PA_ERR_UNSUPPORTED;   // query rows of one group
    Plan plan;
    pa_status st = make_plan(q, k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
                             scale, out, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                             max_context_len, num_blocks, dtype, partition_size, PA_KERNEL_MFMA,
                             PA_KV_SHARED, workspace, workspace_bytes,
                             /*need_out=*/true, /*force_split=*/true, &plan);
    if (st != PA_OK) return st;
    if (max_shared_len > max_context_len) return PA_ERR_ARG;
    if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_ARG;
    if (num_seqs == 0) return PA_OK;
    if (!seq_shared_len || (num_groups > 0 && (!group_start || !group_shared_len))) return PA_ERR_NULL;
    const int32_t P = plan.partition;
    const int32_t G = plan.p.group;
    // 64 or more columns per group and kv head: the LDS-staged prefix kernel
    // with partitions of its own (Pp), each sequence's slot shift following
    // from its shared length, in the launch of the rest of every context;
    // else the multi-query kernel in partitions of P
    const int64_t cols = (int64_t)G * max_group_size;
    const bool wide = num_groups > 0 && cols >= kPrefixWideMinCols;
    const int32_t wide_cg = (int32_t)((cols + pa_impl::decode_prefix_columns() - 1) /
                                      pa_impl::decode_prefix_columns());
    const int32_t Pp = wide ? prefix_wide_partition((int64_t)num_groups * num_kv_heads * wide_cg, max_shared_len)
                            : P;
    const int32_t row = parts_for(max_context_len, P) + (wide ? parts_for(max_shared_len, Pp) : 1);
    const size_t need = pa_impl::ws_rows(num_seqs, num_heads, row) * (size_t)(head_dim + 2) * sizeof(float);
    if (!workspace) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ARG;
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;

    // Each group's shared positions: one launch (the LDS-staged prefix kernel
    // or the multi-query kernel) whose virtual sequence g has query rows
    // group_start[g] .. group_start[g + 1] - 1 (the group's decode queries,
    // each seeing all group_shared_len[g] positions), reads the pages through
    // its first member's table row and writes the partials of partitions
    // 0 .. ceil(group_shared_len[g] / Pp) - 1 to those slots of its members'
    // rows.
    DecodeParams m{};
    bool fused = false;                       // prefix stage in the launch of the rest
    int32_t tiles = 1;                        // multi-query prefix stage: tiles per workgroup
    if (num_groups > 0 && max_shared_len > 0) {
        m.q = q;
        m.k_cache = k_cache;
        m.v_cache = v_cache;
        m.block_tables = block_tables;
        m.context_lens = group_shared_len;    // a group's context is its shared prefix
        m.out = out;
        m.ws = plan.p.ws;
        m.scale_log2 = plan.p.scale_log2;
        m.num_seqs = num_groups;
        m.num_heads = num_heads;
        m.num_kv_heads = num_kv_heads;
        m.group = plan.p.group;
        m.head_dim = head_dim;
        m.block_size = block_size;
        m.max_blocks_per_seq = max_blocks_per_seq;
        m.max_context_len = max_shared_len;
        m.num_blocks = num_blocks;
        m.partition = Pp;
        m.max_parts = parts_for(max_shared_len, Pp);
        m.ws_parts = row;
        m.split = 1;
        m.waves = 4;
        m.query_start = group_start;
        m.num_tokens = num_seqs;
        m.max_query_len = max_group_size;
        m.stream_kv = 0;                      // ordinary loads: the pages are shared
        m.all_visible = 1;
        m.table_rows_from_queries = 1;
        if (wide) {
            m.col_groups = wide_cg;
            if ((uint64_t)num_groups * num_kv_heads * m.col_groups * (m.max_parts + 8) >= kMaxGrid)
                return PA_ERR_UNSUPPORTED;
        } else {
            tiles = multi_col_tiles(m.group, max_group_size);
            m.col_groups = multi_col_groups(m.group, max_group_size);
            if ((uint64_t)num_groups * num_kv_heads * m.col_groups * m.max_parts >= kMaxGrid)
                return PA_ERR_UNSUPPORTED;
        }
        fused = true;
    }
    // The rest of every context from its own shared length on, partitions
    // shifted past its prefix slots (seq_slot_shift), then the merge.
    plan.p.seq_first = seq_shared_len;
    plan.p.prefix_partition = Pp;
    plan.p.ws_parts = row;
    plan.p.k_new = k_new;
    plan.p.v_new = v_new;
    plan.p.append_mask = k_new ? slot_mapping : nullptr;
    if (!fused) st = launch_plan(plan, stream);
    else if (wide) st = hip_status(pa_impl::launch_decode_prefix_rest(m, plan.p, stream));
    else st = hip_status(pa_impl::launch_decode_multi_rest(m, tiles, plan.p, stream));
    if (st != PA_OK) return st;
    return launch_reduce(plan, context_lens, out, stream);
}

}  // extern "C"

extern "C" {

int32_t pa_decode_multi_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t max_query_len,
                                       int32_t partition_size) {
    return resolve_multi_partition(num_seqs, num_heads, num_kv_heads, max_context_len, max_query_len,
                                   partition_size);
}

size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                                      int32_t max_query_len, int32_t partition_size) {
    if (num_seqs < 0 || num_tokens < 0 || head_dim <= 0) return 0;
    const int32_t partition = resolve_multi_partition(num_seqs, num_heads, num_kv_heads, max_context_len,
                                                      max_query_len, partition_size);
    if (partition <= 0) return 0;
    return workspace_bytes_for(num_tokens, num_heads, head_dim, max_context_len, partition);
}

}  // extern "C"

namespace {

pa_status decode_multi_impl(const void* k_new, const void* v_new, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* query_start, int32_t block_size, int32_t num_kv_heads,
                            float scale, void* out, hipStream_t stream, int32_t num_seqs,
                            int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t max_context_len, int32_t max_query_len,
                            int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                            pa_kv_reuse reuse, void* workspace, size_t workspace_bytes) {
    if (!valid_dtype(dtype)) return PA_ERR_ARG;
    if (reuse != PA_KV_AUTO && reuse != PA_KV_STREAM && reuse != PA_KV_SHARED) return PA_ERR_ARG;
    pa_status st = shape_status(num_kv_heads, head_dim, block_size);
    if (st != PA_OK) return st;
    if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (num_heads <= 0 || num_heads % num_kv_heads != 0) return PA_ERR_ARG;
    if (num_heads / num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0) return PA_ERR_ARG;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_ARG;
    if (num_blocks > (int64_t)INT32_MAX + 1) return PA_ERR_ARG;
    if (!isfinite(scale)) return PA_ERR_ARG;
    if (num_seqs < 0 || num_tokens < 0 || max_query_len < 1) return PA_ERR_ARG;
    if (max_query_len > kMaxQueryLen) return PA_ERR_UNSUPPORTED;
    int32_t partition = resolve_multi_partition(num_seqs, num_heads, num_kv_heads, max_context_len,
                                                 max_query_len, partition_size);
    if (partition < 0) return PA_ERR_ARG;
    if (partition > 0 && max_context_len == 0) partition = 0;
    if (num_seqs == 0 || num_tokens == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
        return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PA_ERR_ARG;
    if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_NULL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PA_ERR_ARG;

    const int32_t group = num_heads / num_kv_heads;
    const int32_t tiles = multi_col_tiles(group, max_query_len);
    const int32_t col_groups = multi_col_groups(group, max_query_len);
    const int32_t parts = partition > 0 ? parts_for(max_context_len, partition) : 1;
    if ((uint64_t)num_seqs * num_kv_heads * col_groups * parts >= kMaxGrid) return PA_ERR_UNSUPPORTED;
    if ((uint64_t)num_tokens * num_heads >= kMaxGrid) return PA_ERR_UNSUPPORTED;
    if (partition > 0) {
        const size_t need = workspace_bytes_for(num_tokens, num_heads, head_dim, max_context_len, partition);
        if (!workspace) return PA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PA_ERR_ARG;
        if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    }

    DecodeParams p{};
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.out = out;
    p.ws = static_cast<float*>(workspace);
    p.scale_log2 = scale * 1.4426950408889634f;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = group;
    p.head_dim = head_dim;
    p.block_size = block_size;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = max_context_len;
    p.num_blocks = num_blocks;
    p.stream_kv = reuse != PA_KV_SHARED;
    p.query_start = query_start;
    p.num_tokens = num_tokens;
    p.max_query_len = max_query_len;
    p.col_groups = col_groups;
    p.k_new = k_new;
    p.v_new = v_new;
    // one pass of at most four rounds of workgroups: longest sequences first
    p.order_by_length = partition == 0 && num_seqs <= kSortMaxSeqs &&
                        (int64_t)num_seqs * col_groups * num_kv_heads <= kMultiOrderedUnits;
    if (partition > 0) {
        p.partition = partition;
        p.max_parts = parts;
        p.split = 1;
    } else {
        const int32_t whole = max_context_len < 1 ? 1 : max_context_len;
        p.partition = (int32_t)(((int64_t)whole + kChunk - 1) / kChunk * kChunk);
        p.max_parts = 1;
        p.split = 0;
    }
    if ((int64_t)group * max_query_len >= kPrefixWideMinCols) {
        // Many query columns per (sequence, kv head) -- a prompt chunk: the
        // LDS-staged kernel stages each K/V chunk once for 128 columns, where
        // the kernel below reads it once per 32 (and the product is dense
        // enough for the matrix cores to matter).  The fused append stores
        // the new rows in a launch of its own first, so it stays bit-identical
        // to pa_kv_append + pa_decode_multi.
        if (k_new) {
            st = hip_status(pa_impl::launch_append_multi_rows(p, stream));
            if (st != PA_OK) return st;
        }
        p.k_new = nullptr;
        p.v_new = nullptr;
        p.order_by_length = 0;
        p.col_groups = (int32_t)(((int64_t)group * max_query_len + pa_impl::decode_prefix_columns() - 1) /
                                 pa_impl::decode_prefix_columns());
        st = hip_status(pa_impl::launch_decode_multi_wide(p, stream));
    } else {
        // 4-wave workgroups.  8 (one per compute unit at this kernel's two
        // waves per SIMD) measured faster without the fused append
        // (speculative verification, 64 sequences x 5 queries: 104.6 against
        // 108.2 us) and slower with it (116.9 against 114.9);
        // pa_decode_multi_append must stay bit-identical to pa_kv_append +
        // pa_decode_multi, so both keep 4.
        p.waves = 4;
        st = hip_status(pa_impl::launch_decode_multi(p, tiles, stream));
    }
    if (st != PA_OK || partition == 0) return st;

    ReduceParams r;
    r.ws = p.ws;
    r.context_lens = context_lens;
    r.out = out;
    r.num_seqs = num_tokens;              // merge rows are query tokens
    r.num_heads = num_heads;
    r.head_dim = head_dim;
    r.max_context_len = max_context_len;
    r.partition = partition;
    r.max_parts = parts;
    r.query_start = query_start;
    r.num_groups = num_seqs;
    r.max_query_len = max_query_len;
    r.slot_shift = 0;
    r.seq_first = nullptr;
    r.prefix_partition = 0;
    return hip_status(pa_impl::launch_decode_reduce(r, dtype, stream));
}

}  // namespace

extern "C" {

pa_status pa_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start, int32_t block_size, int32_t num_kv_heads,
                          float scale, void* out, hipStream_t stream, int32_t num_seqs,
                          int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                          int32_t max_blocks_per_seq, int32_t max_context_len, int32_t max_query_len,
                          int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                          pa_kv_reuse reuse, void* workspace, size_t workspace_bytes) {
    return decode_multi_impl(nullptr, nullptr, q, k_cache, v_cache, block_tables, context_lens, query_start,
                             block_size, num_kv_heads, scale, out, stream, num_seqs, num_tokens, num_heads,
                             head_dim, max_blocks_per_seq, max_context_len, max_query_len, num_blocks, dtype,
                             partition_size, reuse, workspace, workspace_bytes);
}

pa_status pa_decode_multi_append(const void* k_new, const void* v_new, const void* q, void* k_cache,
                                 void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start, int32_t block_size, int32_t num_kv_heads,
                                 float scale, void* out, hipStream_t stream, int32_t num_seqs,
                                 int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t max_context_len, int32_t max_query_len,
                                 int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                                 pa_kv_reuse reuse, void* workspace, size_t workspace_bytes) {
    if (num_seqs > 0 && num_tokens > 0 && (!k_new || !v_new)) return PA_ERR_NULL;
    return decode_multi_impl(k_new, v_new, q, k_cache, v_cache, block_tables, context_lens, query_start,
                             block_size, num_kv_heads, scale, out, stream, num_seqs, num_tokens, num_heads,
                             head_dim, max_blocks_per_seq, max_context_len, max_query_len, num_blocks, dtype,
                             partition_size, reuse, workspace, workspace_bytes);
}

}  // extern "C"
