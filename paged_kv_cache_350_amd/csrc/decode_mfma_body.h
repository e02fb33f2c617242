#pragma once
// Paged decode attention on the MFMA matrix cores (bf16 caches, gfx950).
//
// Same contract as the vector-ALU kernel: one workgroup per (sequence, kv
// head, partition), all G <= 16 query heads of the kv head at once, K/V read
// in place through the block table.  A workgroup has 4 or 12 waves (the
// template parameter WAVES); its waves take the partition's 32-token chunks
// in turn and merge their partial softmax states in LDS at the end.  [PagedAttention Internals, "How
// PagedAttention Works" item 3; What is PagedAttention?, "On-the-Fly CUDA
// Block Fetching"]
//
// Why matrix cores: with grouped-query attention the G query heads of one kv
// head share every K and V row, so Q.K^T over a tile of tokens is a genuine
// [tokens x D] . [D x G] product and P.V a [D x tokens] . [tokens x G] one.
// On the vector ALU they cost ~2G FMAs per cached element plus lane
// reductions, which approaches the VALU rate at G = 8; one 16x16x32 bf16
// MFMA retires 8192 of them.  G is padded to 16 columns; a padding column
// repeats head 0's query, so it takes exactly column 0's rescale decisions
// and is never stored.
//
// Work unit: a chunk of 32 tokens, tau = 0..31.  Per chunk:
//   Q.K^T  v_mfma_f32_16x16x32_bf16 on two 16-token row tiles t = 0, 1:
//          A = K rows (tokens), B = Q^T (columns = heads), D/32 k-steps.
//          K pages are [D/8 chunks][BS][8]: lane (r = lane % 16, j = lane / 16)
//          of k-step s loads the 16 bytes of chunk 4 s + j of its row's token.
//          The result gives lane (h = lane % 16, j) rows 4 j .. 4 j + 3 of
//          each tile, i.e. 8 scores of head h.
//   softmax per head: chunk max over the lane's 8 scores, then across the
//          four lane groups; the running sum and accumulator are rescaled by
//          2^(m_old - m_new) only when the max grows by more than 8 (log2
//          units), so normally no accumulator is touched by the vector ALU.
//   P.V    v_mfma_f32_16x16x32_bf16, A = V^T (rows = 16 dims), B = P^T.  The
//          k-slots of lane group j are the tokens of its 8 scores, so lane
//          (h, j) already holds its B operand; V pages are dim-major [D][BS],
//          so the A operand is that lane's 8 tokens of dim 16 dc + r.
//          Nothing goes through LDS inside the loop.  Page ids come through
//          the scalar cache, one chunk ahead of their use.
//
// Two ways to assign tokens to rows, chosen by how the pages are reused:
//   split (streaming: each page read by one workgroup per step) -- tile t is
//          the 16-token half t of the chunk (two pages at block 16, two halves
//          of one page at block 32), row r is token 16 t + r.  Every load
//          instruction reads one half, so it is a raw buffer load whose base
//          address (the half's page tile) sits in scalar registers and whose
//          per-lane offset never changes: no 64-bit address math, and the
//          loads carry the non-temporal bit.  Lane group j holds tokens
//          4 j .. 4 j + 3 of each half; its V operand is two 8-byte loads.
//   interleaved (shared pages: many workgroups read the same page, mostly
//          from L2) -- row r of tile t is token 8 (r / 4) + 4 t + r % 4, so
//          lane group j holds tokens 8 j .. 8 j + 7 and its V operand is one
//          16-byte load.  Loads are ordinary global loads from a per-lane page
//          base computed once per chunk; fewer, wider load instructions is
//          what counts when the data comes from cache.
// Masking of a partly valid chunk selects -inf scores and zero V values
// (never multiplies a possibly-NaN slot by zero).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {


namespace mfma_detail {

constexpr int kChunk = 32;            // tokens per MFMA step (k of the P.V product)
constexpr int kHalf = 16;             // tokens per row tile
constexpr float kRescaleSlack = 8.f;  // log2 units: weights stay <= 256 between rescales

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Buffer resource over `bytes` bytes at `base` (raw buffer, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}

// Raw buffer loads with the streaming policy: per-lane byte offset `off` plus
// a wave-uniform byte offset `soff` (a scalar register, so constant strides
// cost no VGPR).
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, kPolicyStream);
}
__device__ __forceinline__ u32x2_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, kPolicyStream);
}

// Chunk-relative token of score slot 4 t + i held by lane group j: split
// halves, or interleaved.
template <bool IL>
__device__ __forceinline__ int slot_token(int t, int i, int j) {
    return IL ? 8 * j + 4 * t + i : kHalf * t + 4 * j + i;
}

// One workgroup's work: `bid` is its index in the launch's grid of
// (sequence, kv head, partition) units, `smem` the launch's dynamic LDS
// (the wave-merge area below).
template <int D, int BS, bool SPLIT, int WAVES>
__device__ __forceinline__ void decode_mfma_body(const DecodeParams& p, uint32_t bid, float* smem) {
    constexpr int kWaves = WAVES;
    constexpr int kThreads = kWaves * kWave;
    constexpr int KSTEPS = D / 32;   // Q.K^T k-steps
    constexpr int DC = D / 16;       // 16-dim output tiles of P.V
    constexpr uint32_t kTileBytes = (uint32_t)D * BS * 2;
    static_assert(BS == 16 || BS == 32, "block size");
    // token order inside a chunk: split halves on the streaming path at
    // block 16, interleaved otherwise
    constexpr bool IL = !SPLIT || BS == 32;

    float* sm_m = smem;                          // [kWaves][16]
    float* sm_l = sm_m + kWaves * 16;            // [kWaves][16]
    float* sacc = sm_l + kWaves * 16;            // [kWaves][G][D]

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int hl = lane % 16;        // head (column) of this lane
    const int j = lane / 16;         // lane group
    const int r = lane % 16;         // A-operand row of this lane

    const int part0 = SPLIT ? 0 : p.first_part;              // slots below it are not launched
    const WorkItem wi = decode_work_item(bid, (uint32_t)p.num_seqs,
                                         (uint32_t)(p.num_kv_heads * (p.max_parts - part0)));
    __shared__ __align__(16) int s_lens[kSortMax];
    __shared__ int s_pick;
    const int b = p.order_by_length ? seq_by_length<kThreads>(p.context_lens, p.num_seqs, wi.b, s_lens, &s_pick)
                                    : wi.b;                  // launch-uniform choice
    const int g = wi.q % p.num_kv_heads;
    const int slot = wi.q / p.num_kv_heads + part0;
    const int G = p.group;

    int L = p.context_lens[b];
    const int cap = min(p.max_context_len, p.max_blocks_per_seq * BS);
    L = L < 0 ? 0 : (L > cap ? cap : L);
    // With a shared length per sequence (the grouped call, shared-page loads)
    // slot s is the s-th partition from the one holding the sequence's first
    // private position: the host knows no lower bound on those lengths, so
    // the grid keeps every slot, and this order puts each sequence's own
    // work first and the slots past its end (which return at once) last.
    const int part = (!SPLIT && p.seq_first)
                         ? own_partition(slot, p.seq_first[b], L, p.partition)
                         : partition_of(slot, p.max_parts, L, p.partition, SPLIT);
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
    const size_t head0 = (size_t)b * p.num_heads + (size_t)g * G;
    if (part < 0) {
        if (!p.split && slot == 0) {          // single pass, empty context: zeros
            for (int e = tid; e < G * D; e += kThreads) out[head0 * D + e] = 0;
        }
        return;
    }
    // positions below first_token are read by a shared-prefix launch
    const int first = p.seq_first ? p.seq_first[b] : p.first_token;
    const int shift = p.seq_first ? seq_slot_shift(first, p.partition, p.prefix_partition) : p.slot_shift;
    const int pstart = part * p.partition;
    if (pstart + p.partition <= first) return;
    const int start = max(pstart, first);
    const int end = min(pstart + p.partition, L);

    // Q^T as the B operand: lane (hl, j) holds head hl, dims 32 s + 8 j .. + 8.
    bf16x8_t qf[KSTEPS];
    {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                               (head0 + (hl < G ? hl : 0)) * D;
        // no select on the loaded values: the first wait on them is the
        // first MFMA, after the first chunk's K/V loads are in flight
        for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(ld16(qrow + 32 * s + 8 * j));
    }

    // interleaved order: this lane's K row (tile 0) and V token group
    const int tk = 8 * (r / 4) + (r % 4);
    const int tv = 8 * j;
    // streaming path: per-lane byte offsets inside a K / V page tile (a
    // half's at block 16; loop invariant); the tile, k-step and dim-tile
    // strides are scalar offsets.
    const uint32_t kofs = (uint32_t)((j * BS + (IL ? tk : r)) * 16);
    const uint32_t vofs = (uint32_t)((r * BS + (IL ? tv : 4 * j)) * 2);
    constexpr uint32_t kStepBytes = 4u * BS * 16;     // K chunk 4 s + j -> 4 (s + 1) + j
    constexpr uint32_t kTileStep = 16u * BS * 2;      // V dim 16 dc + r -> 16 (dc + 1) + r

    const int* row = p.block_tables + (size_t)b * p.max_blocks_per_seq;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(p.k_cache);
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(p.v_cache);
    const size_t tile_elems = (size_t)D * BS;
    const size_t kv_heads = (size_t)p.num_kv_heads;

    float m_run = neg_inf();
    float l_run = 0.f;
    f32x4_t acc[DC];
    for (int dc = 0; dc < DC; ++dc) acc[dc] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (end - start + kChunk - 1) / kChunk;

    // Fused append (pa_decode_append): the workgroup that reads position
    // L - 1 stores kv head g's new K and V rows into that slot, and the wave
    // that reads it (the one whose last chunk holds L - 1) stores them
    // itself.  Its loads of the new row go out with its first loads and the
    // stores follow its first chunk's K/V loads.
    //  * Streaming path: the wave never waits for its stores.  It loads its
    //    last chunk as usual -- the slot of L - 1 may still hold what was
    //    there before -- and puts the new row into that chunk's operand
    //    registers itself, lane to lane (ds_bpermute), before any MFMA reads
    //    them; then it writes the row back inside whole 64-byte blocks.
    //    (8B-shaped step 95.4 -> 94.0 us against storing the row alone and
    //    waiting for it before the last chunk's loads.)
    //  * Shared-page path: it waits for its stores before its last chunk's
    //    loads (before any load when its only chunk holds L - 1).
    // No other workgroup reads that page: without sharing it belongs to this
    // (sequence, kv head) alone, and a sequence only appends into a page it
    // owns (copy-on-write happens before).  A page id outside the pool
    // writes nothing, as pa_kv_append skips an out-of-range slot.
    //
    // Only the appending wave reads the mask and the page id, through the
    // scalar cache (both are read-only here).
    typedef const __attribute__((address_space(4))) int* const_row_t;
    typedef const __attribute__((address_space(4))) int64_t* const_mask_t;
    const const_row_t rowc = (const_row_t)row;
    // The wave that reads L - 1 (wave-uniform).  The streaming path reads
    // the mask, the page id and the new row only with that last chunk's
    // loads, so nothing delays the wave before then (it runs the longest of
    // its workgroup's waves: the last chunk makes its share the largest).
    const bool append_cand = p.k_new != nullptr && end == L && w == (nchunks - 1) % kWaves;
    bool append_wave = false;                                // shared-page path, decided here
    if (!SPLIT && append_cand) {
        const bool masked_out = p.append_mask != nullptr && ((const_mask_t)p.append_mask)[b] < 0;
        append_wave = !masked_out && (uint32_t)rowc[(L - 1) / BS] < (uint64_t)p.num_blocks;
    }
    const bool store_first = !SPLIT && append_wave && nchunks - 1 < kWaves;   // its only chunk holds L - 1
    // lane c < D / 8 holds K bytes 16 c .. 16 c + 15 of the new row; lane
    // l holds V dims l and l + 64 (D = 128) or l (D = 64)
    u32x4_t new_k = u32x4_t{0u, 0u, 0u, 0u};
    uint16_t new_v[D / kWave];
    for (int i = 0; i < D / kWave; ++i) new_v[i] = 0;
    auto load_new_row = [&]() {
        const size_t src = ((size_t)b * kv_heads + g) * D;
        const uint16_t* kn = reinterpret_cast<const uint16_t*>(p.k_new) + src;
        const uint16_t* vn = reinterpret_cast<const uint16_t*>(p.v_new) + src;
        if (lane < D / 8) new_k = ld16(kn + 8 * lane);
        for (int i = 0; i < D / kWave; ++i) new_v[i] = vn[lane + kWave * i];
    };
    uint16_t* new_kdst = nullptr;
    uint16_t* new_vdst = nullptr;
    if (append_wave) {
        const int pos = L - 1;
        const size_t tile = ((size_t)rowc[pos / BS] * kv_heads + g) * tile_elems;
        load_new_row();
        new_kdst = const_cast<uint16_t*>(kc) + tile + ((size_t)lane * BS + pos % BS) * 8;
        new_vdst = const_cast<uint16_t*>(vc) + tile + pos % BS;
    }
    auto store_new_row = [&]() {
        if (lane < D / 8) st16(new_kdst, new_k);
        for (int i = 0; i < D / kWave; ++i) new_vdst[(size_t)(lane + kWave * i) * BS] = new_v[i];
    };
    if (store_first) {
        store_new_row();
        __builtin_amdgcn_s_waitcnt(0);                       // stored before any K/V load
    }

    // Page ids: scalar loads through the constant address space (the table
    // is read-only during the kernel), issued one chunk ahead of their use.
    // They bypass the vector memory queue that the K/V stream keeps full,
    // and need no LDS staging or barrier.  Ids outside the pool read page 0.
    const int blk_first = start / BS;
    const int blk_last = (end - 1) / BS;                     // last page the partition uses
    // raw ids of chunk ci's pages; at block 16 the second one repeats the
    // first when the chunk does not reach it
    auto chunk_pages = [&](int ci, int& first, int& second) {
        const int blk = blk_first + ci * (kChunk / BS);
        first = rowc[blk];
        second = BS == 16 ? rowc[min(blk + 1, blk_last)] : first;
    };
    auto clamp_page = [&](int x) { return (uint32_t)x >= (uint64_t)p.num_blocks ? 0 : x; };
    int next0 = 0, next1 = 0;
    if (w < nchunks) chunk_pages(w, next0, next1);
    for (int ci = w; ci < nchunks; ci += kWaves) {
        const int cstart = start + ci * kChunk;
        const int valid = min(kChunk, end - cstart);

        // ---- pages of the chunk (wave-uniform); the next chunk's ids go in flight
        const int raw0 = __builtin_amdgcn_readfirstlane(next0);
        const int raw1 = __builtin_amdgcn_readfirstlane(next1);
        const int pg0 = clamp_page(raw0);
        const int pg1 = clamp_page(raw1);
        if (ci + kWaves < nchunks) chunk_pages(ci + kWaves, next0, next1);
        // shared-page path: the appended row is in this (last) chunk, and
        // this wave's own stores of it complete before the chunk's loads
        if (!SPLIT && append_wave && !store_first && ci == nchunks - 1) __builtin_amdgcn_s_waitcnt(0);

        // ---- loads: K of both row tiles, V of every 16-dim tile
        u32x4_t kraw[2][KSTEPS];
        u32x4_t vop[DC];                 // V^T operand, 8 bf16 per lane
        if constexpr (SPLIT) {
            // the appending wave's last chunk: its mask entry (a vector load,
            // so that no branch waits for it) and the new row go out with its
            // K/V loads; the page id of L - 1 is the chunk's own, loaded a chunk
            // ahead
            const bool last_cand = append_cand && ci == nchunks - 1;        // wave-uniform
            u32x2_t mask_v = u32x2_t{0u, 0u};
            if (last_cand) {
                if (p.append_mask != nullptr)
                    mask_v = __builtin_amdgcn_raw_buffer_load_b64(make_rsrc(p.append_mask + b, 8), 0, 0, 0);
                load_new_row();
            }
            if constexpr (IL) {
                // block 32: the chunk is one page; row tile t's K rows sit 4 t
                // tokens (64 bytes) in, each V operand is one 16-byte load (8
                // tokens of a dim).  Every load covers whole 64-byte blocks of
                // the page; tokens past the context are masked below.
                const size_t tile = ((size_t)pg0 * kv_heads + g) * tile_elems;
                const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + tile, kTileBytes);
                const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + tile, kTileBytes);
                for (int t = 0; t < 2; ++t)
                    for (int s = 0; s < KSTEPS; ++s) kraw[t][s] = bload16(krs, kofs, 64u * t + s * kStepBytes);
                for (int dc = 0; dc < DC; ++dc) vop[dc] = bload16(vrs, vofs, dc * kTileStep);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                __amdgpu_buffer_rsrc_t krs[2], vrs[2];
                for (int t = 0; t < 2; ++t) {
                    const size_t tile = ((size_t)(t ? pg1 : pg0) * kv_heads + g) * tile_elems;
                    // a half (page) with no valid token gets an empty range: loads return 0
                    const bool live = t == 0 || valid > kHalf;
                    krs[t] = make_rsrc(kc + tile, live ? kTileBytes : 0);
                    vrs[t] = make_rsrc(vc + tile, live ? kTileBytes : 0);
                }
                for (int t = 0; t < 2; ++t)
                    for (int s = 0; s < KSTEPS; ++s) kraw[t][s] = bload16(krs[t], kofs, s * kStepBytes);
                u32x2_t vh[2][DC];
                for (int t = 0; t < 2; ++t)
                    for (int dc = 0; dc < DC; ++dc) vh[t][dc] = bload8(vrs[t], vofs, dc * kTileStep);
                // every load of the chunk is in flight before the first MFMA waits on one
                __builtin_amdgcn_sched_barrier(0);
                for (int dc = 0; dc < DC; ++dc)
                    vop[dc] = u32x4_t{vh[0][dc][0], vh[0][dc][1], vh[1][dc][0], vh[1][dc][1]};
            }
            if (last_cand) {
                // The new row into this chunk's registers.  Position L - 1 is
                // chunk token p0: K row r0 of tile t0 (lane (r0, j) holds its
                // 16-byte column 4 s + j, held by lane 4 s + j of new_k); V
                // element e0 of the lanes with j = j0 (dword q0 = e0 / 2, half
                // e0 % 2; lane (r, j0) takes dim 16 dc + r, held by lane
                // (16 dc + r) % 64, element (16 dc + r) / 64).  Split halves:
                // p0 = 16 t0 + r0, r0 = 4 j0 + i0, e0 = 4 t0 + i0; interleaved:
                // p0 = 8 (r0 / 4) + 4 t0 + r0 % 4, e0 = p0 % 8, j0 = p0 / 8.
                const int p0 = L - 1 - cstart;
                const int t0 = IL ? (p0 / 4) % 2 : p0 / kHalf;
                const int r0 = IL ? 4 * (p0 / 8) + p0 % 4 : p0 % kHalf;
                const int j0 = IL ? p0 / 8 : (p0 % kHalf) / 4;
                const int e0 = IL ? p0 % 8 : 4 * t0 + p0 % 4;
                const int q0 = e0 / 2;
                const uint32_t sh = 16u * (uint32_t)(e0 % 2);
                // the same in every lane: the sequence appends (mask entry >= 0)
                // into a page inside the pool
                const bool app = (int32_t)mask_v[1] >= 0 &&
                                 (uint32_t)(t0 && !IL ? raw1 : raw0) < (uint64_t)p.num_blocks;
                for (int s = 0; s < KSTEPS; ++s) {
                    u32x4_t v;
                    for (int e = 0; e < 4; ++e)
                        v[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (4 * s + j), (int)new_k[e]);
                    for (int t = 0; t < 2; ++t)
                        if (t == t0) kraw[t][s] = app && r == r0 ? v : kraw[t][s];
                }
                for (int dc = 0; dc < DC; ++dc) {
                    const int d = 16 * dc + r;
                    const uint32_t nv = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (d % kWave), (int)new_v[(16 * dc) / kWave]);
                    for (int q = 0; q < 4; ++q)
                        if (q == q0) {
                            const uint32_t patched = (vop[dc][q] & ~(0xffffu << sh)) | ((nv & 0xffffu) << sh);
                            vop[dc][q] = app && j == j0 ? patched : vop[dc][q];
                        }
                }
                // The row goes to the cache inside whole 64-byte blocks: the
                // four tokens of its K columns (rows r with r / 4 = r0 / 4 of
                // tile t0), and every dim row of its page's V tile, the other
                // tokens' bytes as just loaded -- the same bits -- rather than
                // as 2-byte pieces of 128 V dim rows.
                const int pg_t0 = t0 && !IL ? pg1 : pg0;
                uint16_t* kw = const_cast<uint16_t*>(kc) + ((size_t)pg_t0 * kv_heads + g) * tile_elems;
                uint16_t* vw = const_cast<uint16_t*>(vc) + ((size_t)pg_t0 * kv_heads + g) * tile_elems;
                const int krow = IL ? tk + 4 * t0 : r;           // page token of this lane's tile-t0 row
                if (app && (r & ~3) == (r0 & ~3))
                    for (int s = 0; s < KSTEPS; ++s)
                        st16(kw + ((size_t)(4 * s + j) * BS + krow) * 8, t0 ? kraw[1][s] : kraw[0][s]);
                if (app) {
                    for (int dc = 0; dc < DC; ++dc) {
                        if constexpr (IL) {
                            st16(vw + (size_t)(16 * dc + r) * BS + tv, vop[dc]);
                        } else {
                            *reinterpret_cast<u32x2_t*>(vw + (size_t)(16 * dc + r) * BS + 4 * j) =
                                u32x2_t{vop[dc][2 * t0], vop[dc][2 * t0 + 1]};
                        }
                    }
                }
            }
        } else {
            const int kpage = (BS == 16 && tk >= kHalf) ? pg1 : pg0;
            const uint16_t* kb = kc + ((size_t)kpage * kv_heads + g) * tile_elems +
                                 (size_t)(tk % BS) * 8 + (size_t)j * BS * 8;
            const int vpage = (BS == 16 && tv >= kHalf) ? pg1 : pg0;
            const uint16_t* vb = vc + ((size_t)vpage * kv_heads + g) * tile_elems + (tv % BS) +
                                 (size_t)r * BS;
            for (int t = 0; t < 2; ++t)
                for (int s = 0; s < KSTEPS; ++s) kraw[t][s] = ld16(kb + 32 * t + (size_t)s * 4 * BS * 8);
            for (int dc = 0; dc < DC; ++dc) vop[dc] = ld16(vb + (size_t)dc * 16 * BS);
            __builtin_amdgcn_sched_barrier(0);
        }
        // shared-page path: the appending wave stores the new row behind its
        // first chunk's loads
        if (!SPLIT && append_wave && !store_first && ci == w) store_new_row();

        // ---- S = K . Q^T
        f32x4_t st[2];
        for (int t = 0; t < 2; ++t) {
            st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < KSTEPS; ++s)
                st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kraw[t][s]), qf[s], st[t], 0, 0, 0);
        }

        // ---- online softmax; slot 4 t + i of lane (hl, j) is token slot_token(t, i, j)
        float sc[8];
        for (int t = 0; t < 2; ++t)
            for (int i = 0; i < 4; ++i) sc[4 * t + i] = st[t][i] * p.scale_log2;
        if (valid < kChunk) {
            for (int t = 0; t < 2; ++t)
                for (int i = 0; i < 4; ++i)
                    sc[4 * t + i] = (slot_token<IL>(t, i, j) < valid) ? sc[4 * t + i] : neg_inf();
        }
        float mx = sc[0];
        for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sc[k]);
        mx = max_xor16(mx);
        mx = max_xor32(mx);
        // Lazy rescaling: the reference max moves only when a score exceeds it
        // by more than kRescaleSlack (always on the first chunk, m_run = -inf).
        // Between moves the weights are 2^(s - m_run) <= 2^kRescaleSlack; acc
        // and l share the reference, so the result is the same.
        const bool grow = mx > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {       // wave-uniform branch
            const float mn = grow ? mx : m_run;
            const float alpha = fast_exp2(m_run - mn);      // 0 on the first chunk
            for (int dc = 0; dc < DC; ++dc) acc[dc] = acc[dc] * alpha;
            l_run *= alpha;
            m_run = mn;
        }
        bf16x8_t pf;
        float psum = 0.f;
        for (int k = 0; k < 8; ++k) {
            const bf16_t pb = (bf16_t)fast_exp2(sc[k] - m_run);
            pf[k] = pb;
            psum += (float)pb;           // normalise with the weights actually used
        }
        l_run += psum;

        // ---- O^T += V^T . P^T
        if (valid < kChunk) {
            // zero the value slots past the context: dword q holds slots 2 q, 2 q + 1
            for (int q = 0; q < 4; ++q) {
                const int tok = slot_token<IL>(q / 2, 2 * (q % 2), j);
                const uint32_t lo = (tok < valid) ? 0x0000ffffu : 0u;
                const uint32_t hi = (tok + 1 < valid) ? 0xffff0000u : 0u;
                for (int dc = 0; dc < DC; ++dc) vop[dc][q] &= (lo | hi);
            }
        }
        for (int dc = 0; dc < DC; ++dc)
            acc[dc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vop[dc]), pf, acc[dc], 0, 0, 0);
    }

    // ---- merge the waves; lane (hl, j) holds dims 16 dc + 4 j + i of head hl
    l_run = sum_xor16(l_run);
    l_run = sum_xor32(l_run);
    if (lane < 16) {
        sm_m[w * 16 + hl] = m_run;
        sm_l[w * 16 + hl] = l_run;
    }
    if (hl < G) {
        float* dst = sacc + (size_t)(w * G + hl) * D + 4 * j;
        for (int dc = 0; dc < DC; ++dc)
            for (int i = 0; i < 4; ++i) dst[16 * dc + i] = acc[dc][i];
    }
    __syncthreads();

    const int wsp = p.ws_parts > 0 ? p.ws_parts : p.max_parts;      // workspace row length
    const size_t rows = ws_rows(p.num_seqs, p.num_heads, wsp);
    for (int e = tid; e < G * D; e += kThreads) {
        const int h = e / D;
        const int d = e % D;
        float M = neg_inf();
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww * 16 + h]);
        float num = 0.f, den = 0.f;
        if (M != neg_inf()) {
            for (int ww = 0; ww < kWaves; ++ww) {
                const float f = fast_exp2(sm_m[ww * 16 + h] - M);
                num = fmaf(f, sacc[(size_t)(ww * G + h) * D + d], num);
                den = fmaf(f, sm_l[ww * 16 + h], den);
            }
        }
        if (p.split) {
            const size_t rr = (head0 + h) * wsp + part + shift;
            p.ws[rr * D + d] = num;
            if (d == 0) {
                p.ws[rows * D + rr] = M;
                p.ws[rows * D + rows + rr] = den;
            }
        } else {
            out[(head0 + h) * D + d] = f32_to_bf16(den > 0.f ? num / den : 0.f);
        }
    }
}

}  // namespace mfma_detail

}  // namespace pa_impl
