#pragma once
// Multi-query paged attention on the MFMA matrix cores (bf16 caches, gfx950).
//
// Sequence b brings n new tokens whose K/V rows are already in its pages (at
// positions L - n .. L - 1); the query of new token j attends over positions
// 0 .. L - n + j through the block table.  This is what verifying draft
// tokens of speculative decoding over paged memory needs [PagedAttention
// Internals, "The Mathematical Cause of KV Cache Fragmentation", closing
// link], with the paging and attention of "How PagedAttention Works" items
// 1-3; a chunk of a prompt is the same computation.
//
// Same structure as the decode kernel, with the B operand of both products
// widened from "the G query heads of a kv head" to (new token, head) pairs:
// column c of a kv head's group is query token c / G, head c % G.  All
// columns share every K and V row they see, so one K/V read serves up to
// 16 * NT columns (NT = 1 or 2 tiles of 16): with G = 4, eight draft tokens
// fill two tiles, where a decode step pads 4 heads to 16.  Column groups
// beyond 16 * NT columns are separate workgroups.
//
// Work unit, loads, lazy rescaling and the wave merge are those of the
// decode kernel's streaming path (split halves, raw buffer loads); only the
// score mask differs: column c keeps token positions <= L - n + c / G, so
// only the chunks that reach into the new tokens are masked per column.  A
// column that has seen no visible position yet keeps a running max of -inf;
// its weights are taken relative to 0 instead, which makes them 0, and its
// rescale factor is 0 when a neighbouring column moves the tile's maxima.
//
// Partitions end at the last position any column of the group sees, so no
// workgroup reads K/V that none of its queries attends to.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {


namespace multi_detail {

constexpr int kChunk = 32;            // tokens per MFMA step (k of the P.V product)
constexpr int kHalf = 16;             // tokens per row tile
constexpr float kRescaleSlack = 8.f;  // log2 units: weights stay <= 256 between rescales

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}

template <int POLICY>
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, POLICY);
}
template <int POLICY>
__device__ __forceinline__ u32x2_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, POLICY);
}

// Chunk-relative token of score slot 4 t + i held by lane group j: row tile
// t is the 16-token half t of the chunk (block 16: page t), or, at block 32
// (one page per chunk), the interleaved order in which lane group j holds
// tokens 8 j .. 8 j + 7.
template <bool IL>
__device__ __forceinline__ int slot_token(int t, int i, int j) {
    return IL ? 8 * j + 4 * t + i : kHalf * t + 4 * j + i;
}

// One workgroup's work: `bid` is its index in the launch's grid of
// (sequence, kv head, column group, partition) units, `smem` the launch's
// dynamic LDS (the wave-merge area below).
template <int D, int BS, int NT, int POLICY, int WAVES>
__device__ __forceinline__ void decode_multi_body(const DecodeParams& p, uint32_t bid, float* smem) {
    constexpr int kWaves = WAVES;
    constexpr int kThreads = kWaves * kWave;
    constexpr int KSTEPS = D / 32;   // Q.K^T k-steps
    constexpr int DC = D / 16;       // 16-dim output tiles of P.V
    constexpr int COLS = 16 * NT;    // (query token, head) columns per workgroup
    constexpr uint32_t kTileBytes = (uint32_t)D * BS * 2;
    static_assert(BS == 16 || BS == 32, "block size");
    constexpr bool IL = BS == 32;    // interleaved token order (one page per chunk)

    float* sm_m = smem;                          // [kWaves][16]
    float* sm_l = sm_m + kWaves * 16;            // [kWaves][16]
    float* sacc = sm_l + kWaves * 16;            // [kWaves][16][D]

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int hl = lane % 16;        // column of this lane inside a tile
    const int j = lane / 16;         // lane group
    const int r = lane % 16;         // A-operand row of this lane

    const WorkItem wi = decode_work_item(bid, (uint32_t)p.num_seqs,
                                         (uint32_t)(p.num_kv_heads * p.col_groups * p.max_parts));
    __shared__ __align__(16) int s_lens[kSortMax];
    __shared__ int s_pick;
    const int b = p.order_by_length ? seq_by_length<kThreads>(p.context_lens, p.num_seqs, wi.b, s_lens, &s_pick)
                                    : wi.b;                  // launch-uniform choice
    const int g = wi.q % p.num_kv_heads;
    const int cg = (wi.q / p.num_kv_heads) % p.col_groups;
    const int slot = wi.q / (p.num_kv_heads * p.col_groups);
    const int G = p.group;

    int L = p.uniform_len > 0 ? p.uniform_len : p.context_lens[b];
    const int cap = min(p.max_context_len, p.max_blocks_per_seq * BS);
    L = L < 0 ? 0 : (L > cap ? cap : L);
    // rows that all see the whole context are not bounded by its length
    const QueryRows qr = query_rows(p.query_start, b, p.all_visible ? INT_MAX : L, p.num_tokens, p.max_query_len);
    const int n = qr.n;
    const int col0 = cg * COLS;
    if (col0 >= G * n) return;                               // no query in this column group
    const int first_jq = col0 / G;
    const int last_jq = min(n - 1, (col0 + COLS - 1) / G);
    // causal rows: query token jq sees positions <= L - n + jq; with
    // all_visible (the queries of sequences that share these L positions as
    // their prefix) every row sees all of them
    const int vis = p.all_visible ? L - 1 : L - n;           // + jq when causal
    const int lo_lim = p.all_visible ? vis : vis + first_jq; // smallest last visible position
    const int hi_lim = p.all_visible ? vis : vis + last_jq;  // largest
    const int part = partition_of(slot, p.max_parts, L, p.partition, p.stream_kv != 0);
    if (part < 0) return;
    const int start = part * p.partition;
    if (start > hi_lim) return;                              // nothing here is visible to the group
    const int end = min(start + p.partition, hi_lim + 1);

    // Per tile: this lane's column, its query row and head, and the last
    // position it sees (-1: a padding column past the sequence's queries).
    int lim[NT];
    bf16x8_t qf[NT][KSTEPS];
    for (int nt = 0; nt < NT; ++nt) {
        const int c = col0 + 16 * nt + hl;
        const int jq = c / G;
        const bool live = jq < n;
        lim[nt] = live ? (p.all_visible ? vis : vis + jq) : -1;
        const size_t qrow = ((size_t)(qr.row0 + (live ? jq : 0)) * p.num_heads + (size_t)g * G + c % G) * D;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + qrow;
        // a padding column repeats token 0's query of its head and is masked
        // out entirely; no select on the loaded values, so the first wait on
        // them is the first MFMA
        for (int s = 0; s < KSTEPS; ++s) qf[nt][s] = as_bf16x8(ld16(qp + 32 * s + 8 * j));
    }

    // this lane's K row (token of tile 0) and V token group in the chunk
    const int tk = IL ? 8 * (r / 4) + (r % 4) : r;
    const int tv = IL ? 8 * j : 4 * j;
    const uint32_t kofs = (uint32_t)((j * BS + tk) * 16);
    const uint32_t vofs = (uint32_t)((r * BS + tv) * 2);
    constexpr uint32_t kStepBytes = 4u * BS * 16;
    constexpr uint32_t kTileStep = 16u * BS * 2;

    // a group of sequences sharing a prefix reads it through its first
    // member's table row
    const int* row = p.block_tables + (size_t)(p.table_rows_from_queries ? qr.row0 : b) * p.max_blocks_per_seq;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(p.k_cache);
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(p.v_cache);
    const size_t tile_elems = (size_t)D * BS;
    const size_t kv_heads = (size_t)p.num_kv_heads;

    float m_run[NT], l_run[NT];
    f32x4_t acc[NT][DC];
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = neg_inf();
        l_run[nt] = 0.f;
        for (int dc = 0; dc < DC; ++dc) acc[nt][dc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Fused append (pa_decode_multi_append): new token j's K and V rows (row
    // row0 + j of k_new / v_new, aligned with q) belong at position
    // L - n + j.  A workgroup handles the new rows that fall inside the
    // positions it reads.  Up to kPatchRows of them (the usual case): it
    // copies them into LDS, its waves patch them into the registers of the
    // chunk that holds them (whose loads read the slots before the append),
    // and the rows go to the cache after the loop, when this workgroup reads
    // nothing more -- nothing waits on the stores.  More rows: they are
    // stored first and a barrier publishes them to every wave.  Column
    // groups of one (sequence, kv head) store the same bytes, which cannot
    // change what either reads.  A page id outside the pool writes nothing.
    constexpr int kPatchRows = 32;                           // LDS: 32 x 2 x D bf16 fits in sacc
    const int first_new = p.k_new != nullptr ? max(start, L - n) : end;
    const int count = end - first_new;                       // new rows read here (<= 0: none)
    const bool patch = count > 0 && count <= kPatchRows;     // workgroup-uniform
    uint16_t* s_new = reinterpret_cast<uint16_t*>(sacc);     // [count][K row | V row]
    const uint16_t* kn = reinterpret_cast<const uint16_t*>(p.k_new);
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(p.v_new);
    auto new_src = [&](int pos) { return ((size_t)(qr.row0 + pos - (L - n)) * kv_heads + g) * D; };
    auto store_new_rows = [&]() {                            // rows [first_new, end) to the cache
        uint16_t* kw = const_cast<uint16_t*>(kc);
        uint16_t* vw = const_cast<uint16_t*>(vc);
        for (int e = tid; e < count * (D / 8); e += kThreads) {          // K: 16-byte chunks
            const int pos = first_new + e / (D / 8);
            const int c = e % (D / 8);
            const int pg = row[pos / BS];
            if ((uint32_t)pg >= (uint64_t)p.num_blocks) continue;
            const size_t tile = ((size_t)pg * kv_heads + g) * tile_elems;
            const u32x4_t v = patch ? *reinterpret_cast<const u32x4_t*>(s_new + (size_t)(pos - first_new) * 2 * D + 8 * c)
                                    : ld16(kn + new_src(pos) + 8 * c);
            st16(kw + tile + ((size_t)c * BS + pos % BS) * 8, v);
        }
        for (int e = tid; e < count * D; e += kThreads) {                // V: one element per dim
            const int pos = first_new + e / D;
            const int d = e % D;
            const int pg = row[pos / BS];
            if ((uint32_t)pg >= (uint64_t)p.num_blocks) continue;
            const size_t tile = ((size_t)pg * kv_heads + g) * tile_elems;
            vw[tile + (size_t)d * BS + pos % BS] = patch ? s_new[(size_t)(pos - first_new) * 2 * D + D + d]
                                                         : vn[new_src(pos) + d];
        }
    };
    if (patch) {
        for (int e = tid; e < count * (D / 4); e += kThreads) {          // K and V rows, 16 bytes at a time
            const int rr = e / (D / 4);
            const int c = e % (D / 4);                       // chunks 0 .. D/8-1: K, then V
            const uint16_t* src = (c < D / 8 ? kn : vn) + new_src(first_new + rr) + 8 * (c % (D / 8));
            *reinterpret_cast<u32x4_t*>(s_new + (size_t)rr * 2 * D + 8 * c) = ld16(src);
        }
        __syncthreads();
    } else if (count > 0) {
        store_new_rows();
        __syncthreads();
    }

    // Page ids: scalar loads through the constant address space (the table
    // is read-only during the kernel), one chunk ahead of their use; ids
    // outside the pool read page 0.
    typedef const __attribute__((address_space(4))) int* const_row_t;
    const const_row_t rowc = (const_row_t)row;
    const int nchunks = (end - start + kChunk - 1) / kChunk;
    const int blk_first = start / BS;
    const int blk_last = (end - 1) / BS;                     // last page the partition uses
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

        const int pg0 = clamp_page(__builtin_amdgcn_readfirstlane(next0));
        const int pg1 = clamp_page(__builtin_amdgcn_readfirstlane(next1));
        if (ci + kWaves < nchunks) chunk_pages(ci + kWaves, next0, next1);

        u32x4_t kraw[2][KSTEPS];
        u32x4_t vop[DC];
        if constexpr (IL) {
            // block 32: row tile t's K rows sit 4 t tokens (64 bytes) into the
            // page, each V operand is one 16-byte load; every load covers whole
            // 64-byte blocks, and tokens past the partition are masked below
            const size_t tile = ((size_t)pg0 * kv_heads + g) * tile_elems;
            const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + tile, kTileBytes);
            const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + tile, kTileBytes);
            for (int t = 0; t < 2; ++t)
                for (int s = 0; s < KSTEPS; ++s) kraw[t][s] = bload16<POLICY>(krs, kofs, 64u * t + s * kStepBytes);
            for (int dc = 0; dc < DC; ++dc) vop[dc] = bload16<POLICY>(vrs, vofs, dc * kTileStep);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            __amdgpu_buffer_rsrc_t krs[2], vrs[2];
            for (int t = 0; t < 2; ++t) {
                const size_t tile = ((size_t)(t ? pg1 : pg0) * kv_heads + g) * tile_elems;
                const bool half_live = t == 0 || valid > kHalf;
                krs[t] = make_rsrc(kc + tile, half_live ? kTileBytes : 0);
                vrs[t] = make_rsrc(vc + tile, half_live ? kTileBytes : 0);
            }
            for (int t = 0; t < 2; ++t)
                for (int s = 0; s < KSTEPS; ++s) kraw[t][s] = bload16<POLICY>(krs[t], kofs, s * kStepBytes);
            u32x2_t vh[2][DC];
            for (int t = 0; t < 2; ++t)
                for (int dc = 0; dc < DC; ++dc) vh[t][dc] = bload8<POLICY>(vrs[t], vofs, dc * kTileStep);
            __builtin_amdgcn_sched_barrier(0);
            for (int dc = 0; dc < DC; ++dc)
                vop[dc] = u32x4_t{vh[0][dc][0], vh[0][dc][1], vh[1][dc][0], vh[1][dc][1]};
        }
        if (patch && cstart + kChunk > first_new) {          // wave-uniform: new rows in this chunk
            // One small group at a time (scheduling barriers between them), so the
            // patch never holds more than a few LDS values in registers.
            // K: lane (r, j) holds token tk + (block 32: 4 t; block 16: 16 t),
            // 16-byte columns 4 s + j
            for (int t = 0; t < 2; ++t) {
                const int pos = cstart + tk + (IL ? 4 : kHalf) * t;
                const bool is_new = pos >= first_new && pos < end;
                const uint16_t* src = s_new + (size_t)(is_new ? pos - first_new : 0) * 2 * D;
                for (int s = 0; s < KSTEPS; ++s) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + 8 * (4 * s + j));
                    kraw[t][s] = is_new ? v : kraw[t][s];
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // V: dword q of vop[dc] holds tokens slot_token<IL>(q / 2, 2 (q % 2), j) and the next, dim 16 dc + r
            for (int q = 0; q < 4; ++q) {
                for (int hh = 0; hh < 2; ++hh) {
                    const int pos = cstart + slot_token<IL>(q / 2, 2 * (q % 2) + hh, j);
                    const bool is_new = pos >= first_new && pos < end;
                    const uint16_t* src = s_new + (size_t)(is_new ? pos - first_new : 0) * 2 * D + D;
                    const uint32_t sh = 16u * (uint32_t)hh;
                    for (int dc = 0; dc < DC; ++dc) {
                        const uint32_t nv = ((uint32_t)src[16 * dc + r] << sh) | (vop[dc][q] & ~(0xffffu << sh));
                        vop[dc][q] = is_new ? nv : vop[dc][q];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // wave-uniform: does any score of this chunk need masking?
        const bool masked = valid < kChunk || cstart + kChunk - 1 > lo_lim;
        bf16x8_t pf[NT];
        for (int nt = 0; nt < NT; ++nt) {
            f32x4_t st[2];
            for (int t = 0; t < 2; ++t) {
                st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                for (int s = 0; s < KSTEPS; ++s)
                    st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kraw[t][s]), qf[nt][s], st[t], 0, 0, 0);
            }
            float sc[8];
            for (int t = 0; t < 2; ++t)
                for (int i = 0; i < 4; ++i) sc[4 * t + i] = st[t][i] * p.scale_log2;
            if (masked) {
                // keep chunk tokens < cut: inside the partition and visible to this column
                const int cut = min(valid, lim[nt] - cstart + 1);
                for (int t = 0; t < 2; ++t)
                    for (int i = 0; i < 4; ++i)
                        sc[4 * t + i] = slot_token<IL>(t, i, j) < cut ? sc[4 * t + i] : neg_inf();
            }
            float mx = sc[0];
            for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sc[k]);
            mx = max_xor16(mx);
            mx = max_xor32(mx);
            const bool grow = mx > m_run[nt] + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float mn = grow ? mx : m_run[nt];
                // A column with nothing accumulated yet (running max -inf)
                // takes factor 0, not 2^(-inf - -inf) = NaN: another column
                // of the tile may be what took the branch.
                const float alpha = m_run[nt] == neg_inf() ? 0.f : fast_exp2(m_run[nt] - mn);
                for (int dc = 0; dc < DC; ++dc) acc[nt][dc] = acc[nt][dc] * alpha;
                l_run[nt] *= alpha;
                m_run[nt] = mn;
            }
            // -inf running max: nothing visible yet, every score here is -inf too
            const float mref = m_run[nt] == neg_inf() ? 0.f : m_run[nt];
            float psum = 0.f;
            for (int k = 0; k < 8; ++k) {
                const bf16_t pb = (bf16_t)fast_exp2(sc[k] - mref);
                pf[nt][k] = pb;
                psum += (float)pb;
            }
            l_run[nt] += psum;
        }

        if (valid < kChunk) {
            for (int q = 0; q < 4; ++q) {
                const int tok = slot_token<IL>(q / 2, 2 * (q % 2), j);
                const uint32_t lo = (tok < valid) ? 0x0000ffffu : 0u;
                const uint32_t hi = (tok + 1 < valid) ? 0xffff0000u : 0u;
                for (int dc = 0; dc < DC; ++dc) vop[dc][q] &= (lo | hi);
            }
        }
        for (int nt = 0; nt < NT; ++nt)
            for (int dc = 0; dc < DC; ++dc)
                acc[nt][dc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vop[dc]), pf[nt], acc[nt][dc], 0, 0, 0);
    }

    if (patch) {
        store_new_rows();                                    // from LDS; nothing here reads them
        __syncthreads();                                     // before the merge reuses that LDS
    }

    // ---- merge the four waves, one tile at a time through the same LDS
    const int wsp = p.ws_parts > 0 ? p.ws_parts : p.max_parts;      // workspace row length
    const size_t rows = ws_rows(p.num_tokens, p.num_heads, wsp);
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
    for (int nt = 0; nt < NT; ++nt) {
        float l = l_run[nt];
        l = sum_xor16(l);
        l = sum_xor32(l);
        if (nt > 0) __syncthreads();              // the previous tile's reads are done
        if (lane < 16) {
            sm_m[w * 16 + hl] = m_run[nt];
            sm_l[w * 16 + hl] = l;
        }
        {
            float* dst = sacc + (size_t)(w * 16 + hl) * D + 4 * j;
            for (int dc = 0; dc < DC; ++dc)
                for (int i = 0; i < 4; ++i) dst[16 * dc + i] = acc[nt][dc][i];
        }
        __syncthreads();
        for (int e = tid; e < 16 * D; e += kThreads) {
            const int h = e / D;
            const int d = e % D;
            const int c = col0 + 16 * nt + h;
            const int jq = c / G;
            if (jq >= n) continue;
            float M = neg_inf();
            for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww * 16 + h]);
            float num = 0.f, den = 0.f;
            if (M != neg_inf()) {
                for (int ww = 0; ww < kWaves; ++ww) {
                    const float f = fast_exp2(sm_m[ww * 16 + h] - M);
                    num = fmaf(f, sacc[(size_t)(ww * 16 + h) * D + d], num);
                    den = fmaf(f, sm_l[ww * 16 + h], den);
                }
            }
            const size_t orow = (size_t)(qr.row0 + jq) * p.num_heads + (size_t)g * G + c % G;
            if (p.split) {
                const size_t rr = orow * wsp + part;
                p.ws[rr * D + d] = num;
                if (d == 0) {
                    p.ws[rows * D + rr] = M;
                    p.ws[rows * D + rows + rr] = den;
                }
            } else {
                out[orow * D + d] = f32_to_bf16(den > 0.f ? num / den : 0.f);
            }
        }
    }
}

}  // namespace multi_detail

}  // namespace pa_impl
