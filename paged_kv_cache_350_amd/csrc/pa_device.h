// Device-side helpers shared by the libpa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa_impl {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kXcds = 8;       // MI355X: 8 accelerator complex dies, one L2 each

// Third word of a raw buffer resource on gfx9-family chips (32-bit data
// format, no swizzle); the range check then compares byte offsets against
// the record count and returns zeros past it.
constexpr int kBufferFlags = 0x00020000;

// Cache-policy bits of a vector memory instruction on gfx950 (sc0 = 1,
// nt = 2, sc1 = 16).  K/V pages that no other workgroup reads again are
// streamed with nt; pages shared between sequences keep the default policy
// so that concurrent readers hit in L2.
constexpr int kPolicyReuse = 0;
constexpr int kPolicyStream = 2;

// Reinterpret a 32-bit pattern as float.  Always goes through a scalar: a
// bit cast applied directly to an element of a vector value (v[i]) has been
// seen to read the wrong element with this compiler.
__device__ __forceinline__ float u32_as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return u32_as_f32((uint32_t)h << 16); }

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (bf16_t)x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Cross-lane reductions over lane pairs (l, l ^ 16) and (l, l ^ 32) of a
// wave without LDS: v_permlane16_swap / v_permlane32_swap (gfx950) leave each
// lane holding {x[l], x[l ^ k]} in its two results (order depending on the
// lane), so a commutative operation on the two is exactly the reduction a
// __shfl_xor would give, with no LDS round trip.
__device__ __forceinline__ float max_xor16(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(u32_as_f32(r[0]), u32_as_f32(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(u32_as_f32(r[0]), u32_as_f32(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return u32_as_f32(r[0]) + u32_as_f32(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return u32_as_f32(r[0]) + u32_as_f32(r[1]);
}

// 16-byte global load/store through a plain vector type.
__device__ __forceinline__ u32x4_t ld16(const void* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}
// 16-byte K/V load: non-temporal when the pages are streamed (read by one
// workgroup per call), ordinary when other workgroups read them too.
template <bool STREAM>
__device__ __forceinline__ u32x4_t ld16_kv(const void* p) {
    if constexpr (STREAM)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    else
        return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
    *reinterpret_cast<u32x4_t*>(p) = v;
}
// Non-temporal stores for K/V rows appended by pa_kv_append: the rows are
// read by a later kernel, and lines left dirty in L2 by scattered row writes
// measurably slow that kernel's read stream (a decode over 2,048 (sequence,
// kv head) pairs ran 20 us slower after an append kernel with ordinary
// stores, and not measurably slower with these).  The fused appends keep
// ordinary stores: their own workgroup reads the row back at once, and
// non-temporal stores made that 5% slower on an 8B-shaped step.
__device__ __forceinline__ void st16_nt(void* p, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T v) {
    __builtin_nontemporal_store(v, p);
}

// Longest-first order: the sequence with the k-th longest context (ties:
// lower index first; negative lengths count as 0), for batches of at most
// kSortMax sequences (s_lens holds kSortMax entries).  Every workgroup
// derives it the same way from context_lens, so the map is a bijection of
// [0, num_seqs): it changes which workgroup runs which sequence, never what
// any workgroup computes.  The host turns it on for one-pass launches of
// two to four rounds of workgroups, where a random order leaves the longest
// sequences for the last round or puts two of them on one compute unit
// (measured: 8B-shaped decode 101.2 -> 92.7 us, 64 ragged speculative-
// verification sequences 120.5 -> 107.7 us).  Each workgroup pays a load of
// every length and a rank loop, which costs more than it gains once there
// are many rounds of short work.
template <int THREADS>
__device__ __forceinline__ int seq_by_length(const int32_t* lens, int num_seqs, int k, int* s_lens, int* s_pick) {
    const int tid = threadIdx.x;
    const int padded = (num_seqs + 3) & ~3;
    for (int i = tid; i < padded; i += THREADS) {
        const int v = i < num_seqs ? lens[i] : 0;
        s_lens[i] = i < num_seqs ? (v < 0 ? 0 : v) : INT_MIN;     // padding ranks last
    }
    __syncthreads();
    for (int c = tid; c < num_seqs; c += THREADS) {
        const int lc = s_lens[c];
        int rank = 0;
        const int4* s4 = reinterpret_cast<const int4*>(s_lens);
        for (int j4 = 0; j4 < padded / 4; ++j4) {
            const int4 v = s4[j4];
            const int j = 4 * j4;
            rank += (v.x > lc) | ((v.x == lc) & (j < c));
            rank += (v.y > lc) | ((v.y == lc) & (j + 1 < c));
            rank += (v.z > lc) | ((v.z == lc) & (j + 2 < c));
            rank += (v.w > lc) | ((v.w == lc) & (j + 3 < c));
        }
        if (rank == k) *s_pick = c;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_pick);
}

// Decode work items are (partition-major group q = part * num_kv_heads + g,
// sequence b).  Workgroups are handed to the XCDs round-robin (id i runs on
// XCD i % 8).  When the number of groups nq is a multiple of 8, XCD x is given
// exactly the groups q = x, x + 8, x + 16, ...: every XCD then sees the same
// mix of partitions (balanced even when most late partitions are empty), and
// all sequences of one (partition, kv head) run back to back on one XCD, so
// pages they share (a common prefix) are served from that XCD's L2.  Other
// grids keep the natural order, which spreads consecutive sequences across
// the XCDs.  Both maps are bijections of [0, num_seqs * nq).
struct WorkItem {
    int b;
    int q;
};

__device__ __forceinline__ WorkItem decode_work_item(uint32_t hw_id, uint32_t num_seqs, uint32_t nq) {
    WorkItem w;
    if (nq % kXcds == 0) {
        const uint32_t k = hw_id / kXcds;
        w.q = (int)(hw_id % kXcds + kXcds * (k / num_seqs));
        w.b = (int)(k % num_seqs);
    } else {
        w.q = (int)(hw_id / num_seqs);
        w.b = (int)(hw_id % num_seqs);
    }
    return w;
}

// Partition handled by work-item slot `slot` (0 .. max_parts - 1, the order
// in which slots are dispatched) of a sequence with L tokens and partitions
// of P tokens; -1 when the sequence has no such partition.
//   from_start: slot s is partition s.  Sequences that share a prompt prefix
//     read the same pages in the same slot, at about the same time.
//   from_end: slots count partitions back from each sequence's end, largest
//     distance first, so the last partition of every sequence -- the only
//     partial, shorter one -- is dispatched last and the grid drains on
//     small work units instead of full ones.
__device__ __forceinline__ int partition_of(int slot, int max_parts, int L, int P, bool from_end) {
    if (!from_end) return slot * P < L ? slot : -1;
    const int nparts = (L + P - 1) / P;
    const int k = max_parts - 1 - slot;          // distance from the last partition
    return k < nparts ? nparts - 1 - k : -1;
}

// Partition handled by slot `slot` when positions below `first` are read by
// another launch: slots count from the partition that holds `first`; -1 past
// the sequence's end.
__device__ __forceinline__ int own_partition(int slot, int first, int L, int P) {
    const int part = (first > 0 ? first : 0) / P + slot;
    return (int64_t)part * P < L ? part : -1;
}

// Multi-query launches: the query rows of sequence b are row0 .. row0 + n - 1,
// taken from query_start[b] and query_start[b + 1] (or, with no query_start,
// rows b * max_query_len onwards) and clamped so that every row lies in
// [0, num_tokens), n <= max_query_len and n <= L (the sequence's clamped
// context length).  The partition and merge kernels both go through
// this function, so they agree on which rows a sequence covers even when the
// offsets are inconsistent.
struct QueryRows {
    int row0;
    int n;
};

__device__ __forceinline__ QueryRows query_rows(const int32_t* query_start, int b, int L, int num_tokens,
                                                int max_query_len) {
    int r0 = query_start ? query_start[b] : b * max_query_len;
    int r1 = query_start ? query_start[b + 1] : r0 + max_query_len;
    r0 = r0 < 0 ? 0 : r0;
    r1 = r1 > num_tokens ? num_tokens : r1;
    int n = r1 - r0;
    n = n < 0 ? 0 : n;
    n = n > max_query_len ? max_query_len : n;
    n = n > L ? L : n;
    return QueryRows{r0, n};
}

}  // namespace pa_impl
