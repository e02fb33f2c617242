// KV-append scatter: each new token's K and V rows go to the slot its
// sequence's block table gives it (page * block_size + offset).
// [PagedAttention Internals, "How PagedAttention Works" item 2: pages are
// taken on demand as the model generates tokens; What is PagedAttention?,
// page-table figure: a token's place is its page plus its offset]
//
// Two kernels, the same bit copy.  Few rows (a decode step's newest tokens,
// one per sequence, each in a page of its own): one wavefront per (token, kv
// head) row pair; the K row moves as 16-byte chunks (one lane per chunk) into
// k_cache[page][h][chunk][off][:], the V row element by element into
// v_cache[page][h][d][off].  Many rows (a prompt's prefill): one workgroup per
// run of consecutive tokens and one kv head, rows staged in LDS and stored
// with lanes running over the tokens, so that tokens in consecutive slots of
// a page fill whole memory sectors in one store instruction.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {

namespace {

constexpr int kRowsPerBlock = 4;   // four wavefronts, one row pair each
constexpr int kTileMinTokens = 512;   // from this many tokens on, the LDS-staged bulk kernel
constexpr int kMaxVPerLane = 2;    // V elements per lane: head_dim <= 128

// A row pair's source values, loaded before the destination is known: the
// loads go out together with the slot (or length and table) loads instead
// of after them, so a launch waits for one memory round trip less.
template <typename E>
struct SourceRow {
    u32x4_t k;                 // lane's 16-byte K chunk (lanes < head_dim * sizeof(E) / 16)
    E v[kMaxVPerLane];         // V elements lane, lane + 64
};

template <typename E>
__device__ __forceinline__ SourceRow<E> load_source(const E* krow, const E* vrow, int lane, int head_dim) {
    constexpr int X = 16 / sizeof(E);
    SourceRow<E> src;
    src.k = lane < head_dim / X ? ld16(krow + lane * X) : u32x4_t{0u, 0u, 0u, 0u};
    for (int i = 0; i < kMaxVPerLane; ++i) {
        const int d = lane + kWave * i;
        src.v[i] = d < head_dim ? vrow[d] : E{};
    }
    return src;
}

// Store a row pair into slot `off` of page tile `tile` (bit copy): K as
// 16-byte chunks into [chunk][off][X], V element by element into [d][off].
template <typename E>
__device__ __forceinline__ void store_row(E* k_cache, E* v_cache, int64_t tile, int off, int block_size,
                                          int head_dim, int lane, const SourceRow<E>& src) {
    constexpr int X = 16 / sizeof(E);
    if (lane < head_dim / X) st16_nt(k_cache + tile + ((int64_t)lane * block_size + off) * X, src.k);
    for (int i = 0; i < kMaxVPerLane; ++i) {
        const int d = lane + kWave * i;
        if (d < head_dim) st_nt(&v_cache[tile + (int64_t)d * block_size + off], src.v[i]);
    }
}

template <typename E>
__global__ __launch_bounds__(kRowsPerBlock * kWave)
void kv_append_kernel(const E* __restrict__ k, const E* __restrict__ v,
                      const int64_t* __restrict__ slot_mapping,
                      E* __restrict__ k_cache, E* __restrict__ v_cache,
                      int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int64_t num_blocks) {
    const int lane = threadIdx.x % kWave;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (row >= (int64_t)num_tokens * num_kv_heads) return;
    const int64_t tok = row / num_kv_heads;
    const int h = (int)(row % num_kv_heads);
    const SourceRow<E> src = load_source(k + row * head_dim, v + row * head_dim, lane, head_dim);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0 || slot >= num_blocks * block_size) return;   // padding / out of range
    const int64_t page = slot / block_size;
    const int off = (int)(slot % block_size);
    const int64_t tile = (page * num_kv_heads + h) * (int64_t)head_dim * block_size;
    store_row(k_cache, v_cache, tile, off, block_size, head_dim, lane, src);
}

// Bulk append.  The tokens are cut into page segments: maximal runs of
// tokens in consecutive slots of one page (a token whose slot is invalid is a
// segment of its own).  A workgroup takes kv head blockIdx.y of the segments
// that start among tokens TG * blockIdx.x .. + TG - 1 (TG = 32) -- the last
// of them may run up to 31 tokens past that window -- so every page segment
// is written by one workgroup: a prefill run that starts inside a page leaves
// no page row split between two workgroups' partial stores.  Measured, bf16,
// 8 kv heads, D 128, block 32: the prefix workload's suffix prefill (25,484
// tokens in 100 runs starting at page offset 16) 70.3 us with fixed 64-token
// windows, 42.4 us with segments over 64-token windows, 36.2 us over 32-token
// ones (16: 50.9); a 32,768-token prompt 45.9, 47.2 and 40.9 us.
// The rows come in as 16-byte loads along each row (coalesced) into LDS, one
// chunk of padding per row.  How they are stored depends on the slots,
// decided once per workgroup:
//  * most neighbouring tokens in consecutive slots of one page (a prefill
//    run): lane j of a lane group stores token j, so one store instruction
//    writes the same K chunk or the same V dim of consecutive tokens -- a V
//    page row of block_size elements and a K run of block_size 16-byte
//    chunks land whole, where one row at a time leaves each 32-byte sector
//    of a dim-major V page to block_size separate 2-byte writes (measured:
//    32,768 prompt tokens, 8 kv heads, D 128, bf16, in 46-53 us against
//    1,100-1,140 us one row per wavefront);
//  * otherwise (tokens scattered over pages): consecutive lanes store
//    consecutive chunks and dims of one token, as the one-row kernel does,
//    which keeps each store instruction inside one page tile (storing
//    scattered tokens lane by lane measured 3x slower than that).
// Any slot mapping is handled by both; only the speed depends on it.
constexpr int kTileThreads = 256;
constexpr int kTileWindow = 32;

// Where token t's rows go, as its slot (page * block_size + offset; negative
// or past the pool: nowhere): pa_kv_append's slot mapping ...
struct SlotsFromMapping {
    const int64_t* slots;
    __device__ int64_t operator()(int64_t t) const { return slots[t]; }
};

// ... or a multi-query call's new rows: row t belongs to the last sequence b
// with query_start[b] <= t and goes to position L - n + (t - row0) if it is
// one of b's n rows (n clamped as the multi-query kernels clamp it), through
// b's table row; a page id outside the pool writes nothing.
struct SlotsFromQueries {
    const int32_t* query_start;
    const int32_t* context_lens;
    const int32_t* block_tables;
    int32_t num_seqs, num_tokens, max_query_len, max_blocks_per_seq, max_context_len, block_size;
    int64_t num_blocks;
    __device__ int64_t operator()(int64_t t) const {
        int lo = 0, hi = num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (query_start[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int cap = min(max_context_len, max_blocks_per_seq * block_size);
        int L = context_lens[lo];
        L = L < 0 ? 0 : (L > cap ? cap : L);
        const QueryRows qr = query_rows(query_start, lo, L, num_tokens, max_query_len);
        if (t < qr.row0 || t >= qr.row0 + qr.n) return -1;
        const int pos = L - qr.n + (int)(t - qr.row0);
        const int page = block_tables[(size_t)lo * max_blocks_per_seq + pos / block_size];
        if ((uint32_t)page >= (uint64_t)num_blocks) return -1;
        return (int64_t)page * block_size + pos % block_size;
    }
};

template <typename E, int D, typename Slots>
__global__ __launch_bounds__(kTileThreads)
void kv_append_tile_kernel(const E* __restrict__ k, const E* __restrict__ v, Slots slot_of,
                           E* __restrict__ k_cache, E* __restrict__ v_cache,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t block_size,
                           int64_t num_blocks) {
    constexpr int X = 16 / (int)sizeof(E);         // elements per 16-byte chunk
    constexpr int CH = D / X;                      // chunks per row
    constexpr int TG = kTileWindow;                // tokens per window
    constexpr int TGX = TG + 32;                   // the window and the rest of a segment (block_size <= 32)
    constexpr int RS = CH + 1;                     // LDS row stride in chunks
    constexpr int NG = kTileThreads / TG;          // lane groups over chunks / dims
    static_assert(TGX <= kTileThreads && TGX <= 2 * kWave, "one thread of the first two waves per examined token");
    __shared__ u32x4_t sk[TGX * RS];
    __shared__ u32x4_t sv[TGX * RS];
    __shared__ int64_t s_base[TGX];                // element offset of the token's (page, head) tile, -1: skip
    __shared__ int s_off[TGX];
    __shared__ uint64_t s_starts[2];               // per token of the first two waves: starts a segment

    const int tid = threadIdx.x;
    const int h = (int)blockIdx.y;
    const int64_t w0 = (int64_t)blockIdx.x * TG;
    const int64_t nslots = num_blocks * block_size;
    // token w0 + tid (tid < TGX): its slot and its predecessor's, both loaded
    // at once, and whether it starts a page segment (a token past the last
    // counts as a start, so the last segment ends there)
    const int64_t t = w0 + tid;
    int64_t slot = -1, prev = -1;
    if (tid < TGX && t < num_tokens) {
        slot = slot_of(t);
        if (t > 0) prev = slot_of(t - 1);
    }
    const bool valid = slot >= 0 && slot < nslots;            // padding / out of range: skipped
    const bool starts = t >= num_tokens || !valid || t == 0 || slot % block_size == 0 || prev < 0 ||
                        prev >= nslots || prev + 1 != slot;
    if (tid < 2 * kWave) {                                     // whole waves: the ballot's lanes are all live
        const uint64_t m = __builtin_amdgcn_ballot_w64(tid < TGX && starts);
        if (tid % kWave == 0) s_starts[tid / kWave] = m;
    }
    __syncthreads();
    const uint64_t m0 = s_starts[0];
    const uint64_t m1 = s_starts[1];
    // the starts among tokens [lo, hi) (hi - lo <= 64) as bits 0 .. hi - lo - 1
    auto starts_in = [&](int lo, int hi) -> uint64_t {
        const unsigned __int128 all = ((unsigned __int128)m1 << 64) | m0;
        const uint64_t m = (uint64_t)(all >> lo);
        return hi - lo >= 64 ? m : m & ((1ull << (hi - lo)) - 1);
    };
    // first start in [0, TG) and first start in [TG, TGX) (there is one when
    // block_size <= 32: a segment is at most block_size tokens)
    const uint64_t mb = starts_in(0, TG);
    const uint64_t me = starts_in(TG, TGX);
    const int begin = mb ? __builtin_ctzll(mb) : TG;
    const int end = me ? TG + __builtin_ctzll(me) : TGX;
    if (begin >= TG || w0 + begin >= num_tokens) return;      // no segment starts in this window
    const int ntok = end - begin;                             // <= TGX
    // pairs of neighbouring tokens in consecutive slots of one page: the
    // tokens after the first that start no segment
    const int runs = ntok - 1 - (int)__builtin_popcountll(starts_in(begin + 1, end > begin + 65 ? begin + 65 : end)) -
                     (end > begin + 65 ? (int)__builtin_popcountll(starts_in(begin + 65, end)) : 0);
    // token w0 + begin + j, j < ntok, in row j
    if (tid >= begin && tid < end) {
        const int j = tid - begin;
        s_base[j] = valid ? (slot / block_size * num_kv_heads + h) * (int64_t)D * block_size : -1;
        s_off[j] = valid ? (int)(slot % block_size) : 0;
    }
    for (int i = tid; i < ntok * CH; i += kTileThreads) {
        const int j = i / CH;
        const int c = i % CH;
        // rows past the last token (one-token segments of their own) are
        // never stored: nothing to load for them
        if (w0 + begin + j >= num_tokens) continue;
        const int64_t src = ((w0 + begin + j) * num_kv_heads + h) * (int64_t)D + (int64_t)c * X;
        sk[j * RS + c] = ld16(k + src);
        sv[j * RS + c] = ld16(v + src);
    }
    __syncthreads();

    if (2 * runs >= ntok - 1) {
        const int g = tid / TG;
        for (int j = tid % TG; j < ntok; j += TG) {
            const int64_t base = s_base[j];
            if (base < 0) continue;
            const int off = s_off[j];
            for (int c = g; c < CH; c += NG)
                st16_nt(k_cache + base + ((int64_t)c * block_size + off) * X, sk[j * RS + c]);
            const E* vrow = reinterpret_cast<const E*>(&sv[j * RS]);
            for (int d = g; d < D; d += NG) st_nt(&v_cache[base + (int64_t)d * block_size + off], vrow[d]);
        }
        return;
    }
    for (int i = tid; i < ntok * CH; i += kTileThreads) {
        const int j = i / CH;
        const int c = i % CH;
        const int64_t base = s_base[j];
        if (base >= 0) st16_nt(k_cache + base + ((int64_t)c * block_size + s_off[j]) * X, sk[j * RS + c]);
    }
    for (int i = tid; i < ntok * D; i += kTileThreads) {
        const int j = i / D;
        const int d = i % D;
        const int64_t base = s_base[j];
        if (base >= 0)
            st_nt(&v_cache[base + (int64_t)d * block_size + s_off[j]], reinterpret_cast<const E*>(&sv[j * RS])[d]);
    }
}

// The newest row of each sequence (pa_decode_append's rows, [num_seqs]
// [num_kv_heads][head_dim]) to position L - 1, with L clamped as the decode
// kernels clamp it; sequences with L == 0, a negative mask entry or a page
// id outside the pool store nothing -- the fused append's rules exactly.
template <typename E>
__global__ __launch_bounds__(kRowsPerBlock * kWave)
void append_newest_kernel(DecodeParams p) {
    const int lane = threadIdx.x % kWave;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (row >= (int64_t)p.num_seqs * p.num_kv_heads) return;
    const int b = (int)(row / p.num_kv_heads);
    const int h = (int)(row % p.num_kv_heads);
    const int bs = p.block_size;
    const int D = p.head_dim;
    const SourceRow<E> src = load_source(reinterpret_cast<const E*>(p.k_new) + row * D,
                                         reinterpret_cast<const E*>(p.v_new) + row * D, lane, D);
    const int cap = min(p.max_context_len, p.max_blocks_per_seq * bs);
    int L = p.context_lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    if (L == 0 || (p.append_mask != nullptr && p.append_mask[b] < 0)) return;
    const int page = p.block_tables[(size_t)b * p.max_blocks_per_seq + (L - 1) / bs];
    if ((uint32_t)page >= (uint64_t)p.num_blocks) return;
    const int off = (L - 1) % bs;
    const int64_t tile = ((int64_t)page * p.num_kv_heads + h) * (int64_t)D * bs;
    store_row(const_cast<E*>(reinterpret_cast<const E*>(p.k_cache)), const_cast<E*>(reinterpret_cast<const E*>(p.v_cache)),
              tile, off, bs, D, lane, src);
}

}  // namespace

hipError_t launch_append_newest(const DecodeParams& p, pa_dtype dtype, hipStream_t stream) {
    const int64_t rows = (int64_t)p.num_seqs * p.num_kv_heads;
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    const dim3 block(kRowsPerBlock * kWave);
    if (dtype == PA_BF16)
        hipLaunchKernelGGL(append_newest_kernel<uint16_t>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(append_newest_kernel<uint32_t>, grid, block, 0, stream, p);
    return hipGetLastError();
}

template <typename E, int D, typename Slots = SlotsFromMapping>
hipError_t launch_tile(const void* k, const void* v, Slots slots, void* k_cache,
                       void* v_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t block_size,
                       int64_t num_blocks, hipStream_t stream) {
    constexpr int TG = kTileWindow;
    const dim3 grid((unsigned)(((int64_t)num_tokens + TG - 1) / TG), (unsigned)num_kv_heads);
    hipLaunchKernelGGL((kv_append_tile_kernel<E, D, Slots>), grid, dim3(kTileThreads), 0, stream,
                       (const E*)k, (const E*)v, slots, (E*)k_cache, (E*)v_cache, num_tokens,
                       num_kv_heads, block_size, num_blocks);
    return hipGetLastError();
}

hipError_t launch_kv_append(const void* k, const void* v, const int64_t* slot_mapping,
                            void* k_cache, void* v_cache, int32_t num_tokens,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, pa_dtype dtype, hipStream_t stream) {
    if (num_tokens >= kTileMinTokens && num_kv_heads <= 65535) {
        if (dtype == PA_BF16)
            return head_dim == 128 ? launch_tile<uint16_t, 128>(k, v, SlotsFromMapping{slot_mapping}, k_cache, v_cache, num_tokens,
                                                               num_kv_heads, block_size, num_blocks, stream)
                                   : launch_tile<uint16_t, 64>(k, v, SlotsFromMapping{slot_mapping}, k_cache, v_cache, num_tokens,
                                                              num_kv_heads, block_size, num_blocks, stream);
        return head_dim == 128 ? launch_tile<uint32_t, 128>(k, v, SlotsFromMapping{slot_mapping}, k_cache, v_cache, num_tokens,
                                                           num_kv_heads, block_size, num_blocks, stream)
                               : launch_tile<uint32_t, 64>(k, v, SlotsFromMapping{slot_mapping}, k_cache, v_cache, num_tokens,
                                                          num_kv_heads, block_size, num_blocks, stream);
    }
    const int64_t rows = (int64_t)num_tokens * num_kv_heads;
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    const dim3 block(kRowsPerBlock * kWave);
    if (dtype == PA_BF16) {
        hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, block, 0, stream,
                           (const uint16_t*)k, (const uint16_t*)v, slot_mapping,
                           (uint16_t*)k_cache, (uint16_t*)v_cache, num_tokens,
                           num_kv_heads, head_dim, block_size, num_blocks);
    } else {
        hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, block, 0, stream,
                           (const uint32_t*)k, (const uint32_t*)v, slot_mapping,
                           (uint32_t*)k_cache, (uint32_t*)v_cache, num_tokens,
                           num_kv_heads, head_dim, block_size, num_blocks);
    }
    return hipGetLastError();
}

// A multi-query call's new rows (bf16, k_new / v_new aligned with the query
// rows) into their slots: the page-segment tile kernel, each row's slot
// found from query_start and the block table, so a prompt chunk's rows --
// runs of consecutive positions -- land in whole page rows.
hipError_t launch_append_multi_rows(const DecodeParams& p, hipStream_t stream) {
    if (p.num_tokens == 0 || p.num_seqs == 0) return hipSuccess;
    const SlotsFromQueries slots{p.query_start, p.context_lens, p.block_tables, p.num_seqs, p.num_tokens,
                                 p.max_query_len, p.max_blocks_per_seq, p.max_context_len, p.block_size,
                                 p.num_blocks};
    return p.head_dim == 128
               ? launch_tile<uint16_t, 128>(p.k_new, p.v_new, slots, const_cast<void*>(p.k_cache),
                                            const_cast<void*>(p.v_cache), p.num_tokens, p.num_kv_heads,
                                            p.block_size, p.num_blocks, stream)
               : launch_tile<uint16_t, 64>(p.k_new, p.v_new, slots, const_cast<void*>(p.k_cache),
                                           const_cast<void*>(p.v_cache), p.num_tokens, p.num_kv_heads,
                                           p.block_size, p.num_blocks, stream);
}

}  // namespace pa_impl
