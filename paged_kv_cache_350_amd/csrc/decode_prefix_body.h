#pragma once
// Shared-prefix attention for many queries at once (bf16 caches, gfx950).
//
// When many sequences hold their first S tokens in the same pages -- a
// prompt forked to many requests [PagedAttention Internals, "Copy-on-Write
// and Prefix Sharing"; What is PagedAttention?, "Copy-on-Write Memory
// Forking"] -- the attention of every decode query over those S positions
// is one dense product per kv head: the queries of all the group's
// sequences against the same K/V rows.  With 100 sequences and 4 query heads
// per kv head that is 400 query columns over one run of pages, a real dense
// contraction for the matrix cores.
//
// A workgroup takes one kv head, one partition of the shared positions and
// 32 * WAVES query columns (128 in the launches made: WAVES = 4); each wave
// owns 32 of the columns (two 16-column MFMA tiles) for the whole partition.
// The partition's K/V rows go through LDS in chunks of 64 tokens,
// double-buffered: all the workgroup's threads load chunk i + 1 from the
// pages (16-byte loads, contiguous inside each page tile) while the waves
// compute chunk i from LDS, so each page is read from memory once per 128
// columns instead of once per 32 (the per-wave-loads kernel) or once per
// sequence (the per-sequence path).
//
//   S = K.Q^T   v_mfma_f32_16x16x32_bf16, A = K rows (16 tokens), B = Q^T
//   P.V         v_mfma_f32_16x16x32_bf16, A = V^T (16 dims), B = P^T
// with the operand layouts of the decode kernel: score tile lane (c, j)
// holds tokens 4 j .. 4 j + 3 of a 16-token row tile for column c, and the
// P.V contraction runs over the tokens of a 32-token step in the order
// k = 8 j + 4 t + i <-> token 16 t + 4 j + i.  V is laid out in LDS in that
// order, one 128-byte row per dim whose 16-byte slots are XOR-swizzled by
// the dim (one 16-byte LDS read per lane and 16-dim tile, the 16 lanes of a
// read spread over the banks); K keeps the page's [16-byte chunk][token]
// order over 64 tokens.  Two chunk buffers take 64 KiB of LDS.
//
// The same body serves multi-query calls with many query columns per
// (sequence, kv head) -- a chunk of a prompt, whose n new tokens attend
// causally [PagedAttention Internals, "The Mathematical Cause of KV Cache
// Fragmentation", closing link; paging and attention as in "How
// PagedAttention Works" items 1-3]: with CAUSAL, column c (new token c / G
// of the sequence's n) sees positions <= L - n + c / G.  A workgroup's
// partition ends at the last position any of its columns sees, a wave skips
// the chunks none of its columns sees, and scores past a column's last
// position are masked.  The context's last page may hold stale values past
// L, so in a chunk that ends early the V slots past it are zeroed as well
// (a shared prefix always ends on a page boundary).  A single pass (no
// split) writes the normalised output rows directly: each wave owns its
// columns for the whole partition, so no merge across waves is needed.
//
// Online softmax in log2 units with the lazy rescale of the decode kernel
// (the running max moves only when a score exceeds it by more than 8).
// Each wave writes its columns' split-path partials (running max, running
// sum, unnormalised accumulator) to workspace slot `partition` of each
// (query row, head) row; the merge kernel combines them with the rest of
// each sequence's context.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {


namespace prefix_detail {

constexpr int kTok = 64;              // tokens per LDS chunk
constexpr float kRescaleSlack = 8.f;  // log2 units: weights stay <= 256 between rescales

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// One workgroup's work: `bid` is its index in the grid of (unit, column
// group) workgroups that launch_shape sizes, `lds` two chunk buffers.
template <int D, int BS, int WAVES, bool CAUSAL = false>
__device__ __forceinline__ void decode_prefix_body(const DecodeParams& p, uint32_t bid, unsigned char* lds) {
    constexpr int kWaves = WAVES;
    constexpr int kThreads = kWaves * kWave;
    constexpr int kCols = 32 * kWaves;        // query columns per workgroup
    constexpr int KSTEPS = D / 32;            // Q.K^T k-steps
    constexpr int DC = D / 16;                // 16-dim output tiles of P.V
    constexpr int KCH = D / 8;                // 16-byte chunks of a K row
    constexpr int VROW = kTok * 2;            // bytes per V dim row in LDS (8 swizzled 16-byte slots)
    constexpr int KBUF = KCH * kTok * 16;     // bytes of one K buffer
    constexpr int VBUF = D * VROW;            // bytes of one V buffer
    constexpr int KUNITS = KCH * kTok;        // 16-byte K units per chunk
    constexpr int VUNITS = D * kTok / 8;      // 16-byte V units per chunk
    constexpr int KPER = KUNITS / kThreads;   // per thread
    constexpr int VPER = VUNITS / kThreads;
    static_assert(KUNITS % kThreads == 0 && VUNITS % kThreads == 0, "staging split");
    static_assert(BS == 16 || BS == 32, "block size");

    // lds: [2][K buffer | V buffer]

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int hl = lane % 16;
    const int j = lane / 16;
    const int r = lane % 16;

    // Work item.  Units (group, kv head, partition) are spread over the XCDs
    // (workgroup i runs on XCD i % 8) with every column group of one unit on
    // the same XCD, so the groups that read the same pages share its L2.
    const uint32_t units = (uint32_t)p.num_seqs * (uint32_t)p.num_kv_heads * (uint32_t)p.max_parts;
    const uint32_t k8 = bid / kXcds;
    const uint32_t cg = k8 % (uint32_t)p.col_groups;
    const uint32_t u = (k8 / (uint32_t)p.col_groups) * kXcds + bid % kXcds;
    if (u >= units) return;
    const int gi = (int)(u % (uint32_t)p.num_seqs);
    const int g = (int)((u / (uint32_t)p.num_seqs) % (uint32_t)p.num_kv_heads);
    const int part = (int)(u / ((uint32_t)p.num_seqs * (uint32_t)p.num_kv_heads));
    const int G = p.group;

    int L = p.uniform_len > 0 ? p.uniform_len : p.context_lens[gi];
    const int cap = min(p.max_context_len, p.max_blocks_per_seq * BS);
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const QueryRows qr = query_rows(p.query_start, gi, CAUSAL ? L : INT_MAX, p.num_tokens, p.max_query_len);
    const int ncols = G * qr.n;
    const int col0 = (int)cg * kCols;
    if (col0 >= ncols) return;
    const int start = part * p.partition;
    // last position any column of the workgroup sees
    const int hi_lim = CAUSAL ? L - qr.n + min(qr.n - 1, (col0 + kCols - 1) / G) : L - 1;
    if (start > hi_lim) return;
    const int end = min(start + p.partition, hi_lim + 1);
    const int nch = (end - start + kTok - 1) / kTok;

    // this wave's 32 columns (none when past the group's queries: the wave
    // still stages chunks for the others)
    const int wc0 = col0 + 32 * w;
    const bool has_cols = wc0 < ncols;                       // wave-uniform
    // causal: the last position this lane's column sees (-1: a padding
    // column), and the smallest and largest over the wave's live columns
    int lim[2];
    for (int nt = 0; nt < 2; ++nt) {
        const int c = wc0 + 16 * nt + hl;
        lim[nt] = c < ncols ? L - qr.n + c / G : -1;
    }
    const int wave_lo = L - qr.n + wc0 / G;
    const int wave_hi = L - qr.n + min(qr.n - 1, (wc0 + 31) / G);
    bf16x8_t qf[2][KSTEPS];
    for (int nt = 0; nt < 2; ++nt) {
        const int c = wc0 + 16 * nt + hl;
        const int jq = c < ncols ? c / G : 0;                // a padding column repeats row 0's query
        const size_t qrow = ((size_t)(qr.row0 + jq) * p.num_heads + (size_t)g * G + c % G) * D;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + qrow;
        // a negative scale is folded into the query's sign (exact in bf16), so
        // the kernel scales by |scale| >= 0 and a column's max score is
        // |scale| times its max dot product
        const uint32_t flip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
        for (int s = 0; s < KSTEPS; ++s) {
            u32x4_t v = ld16(qp + 32 * s + 8 * j);
            for (int e = 0; e < 4; ++e) v[e] ^= flip;
            qf[nt][s] = as_bf16x8(v);
        }
    }
    // (a zero scale is raised to 1e-30: every weight is then exactly 1, as
    // for scale 0, while a masked score of -inf still gets weight 0)
    const float sabs = fmaxf(fabsf(p.scale_log2), 1e-30f);

    const int* row = p.block_tables + (size_t)(p.table_rows_from_queries ? qr.row0 : gi) * p.max_blocks_per_seq;
    typedef const __attribute__((address_space(4))) int* const_row_t;
    const const_row_t rowc = (const_row_t)row;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(p.k_cache);
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(p.v_cache);
    const size_t tile_elems = (size_t)D * BS;
    const size_t kv_heads = (size_t)p.num_kv_heads;

    // ---- staging: this thread's K and V units of a chunk.  Unit k lies in
    // page unit_page(k) of the chunk (wave-uniform) at 16-byte unit
    // unit_rem(k) of its tile.  The chunk's page ids are scalar loads issued
    // together (an index past the partition's end reads the last live
    // entry), then every unit is one buffer load whose range is empty for a
    // page past the end, so it returns zeros: no branch and no wait between
    // the loads.
    constexpr int KUPP = KCH * BS;            // 16-byte K units per page tile
    constexpr int VUPP = D * BS / 8;          // 16-byte V units per page tile
    constexpr uint32_t kTileBytes = (uint32_t)D * BS * 2;
    auto unit_page = [&](int k, int upp) {
        return __builtin_amdgcn_readfirstlane((kThreads * k + tid) / upp);
    };
    auto unit_rem = [&](int k, int upp) { return (kThreads * k + tid) % upp; };
    auto page_rsrc = [&](const uint16_t* cache, int pg, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(cache + ((size_t)pg * kv_heads + g) * tile_elems), 0,
            live ? (int)kTileBytes : 0, kBufferFlags);
    };
    u32x4_t sk[KPER], sv[VPER];
    auto load_chunk = [&](int ci) {
        const int cstart = start + ci * kTok;
        const int live_pages = (min(kTok, end - cstart) + BS - 1) / BS;
        int kpg[KPER], vpg[VPER];
        for (int k = 0; k < KPER; ++k) {
            const int pg = rowc[cstart / BS + min(unit_page(k, KUPP), live_pages - 1)];
            kpg[k] = (uint32_t)pg >= (uint64_t)p.num_blocks ? 0 : pg;
        }
        for (int k = 0; k < VPER; ++k) {
            const int pg = rowc[cstart / BS + min(unit_page(k, VUPP), live_pages - 1)];
            vpg[k] = (uint32_t)pg >= (uint64_t)p.num_blocks ? 0 : pg;
        }
        for (int k = 0; k < KPER; ++k)
            sk[k] = __builtin_amdgcn_raw_buffer_load_b128(page_rsrc(kc, kpg[k], unit_page(k, KUPP) < live_pages),
                                                          unit_rem(k, KUPP) * 16, 0, kPolicyReuse);
        for (int k = 0; k < VPER; ++k)
            sv[k] = __builtin_amdgcn_raw_buffer_load_b128(page_rsrc(vc, vpg[k], unit_page(k, VUPP) < live_pages),
                                                          unit_rem(k, VUPP) * 16, 0, kPolicyReuse);
    };
    auto store_chunk = [&](int buf) {
        unsigned char* kb = lds + buf * (KBUF + VBUF);
        unsigned char* vb = kb + KBUF;
        for (int k = 0; k < KPER; ++k) {
            const int uu = tid + kThreads * k;
            const int pi = uu / (KCH * BS);
            const int rem = uu % (KCH * BS);
            const int c = rem / BS;                          // 16-byte chunk of the row
            const int tok = pi * BS + rem % BS;              // chunk-local token
            *reinterpret_cast<u32x4_t*>(kb + (c * kTok + tok) * 16) = sk[k];
        }
        for (int k = 0; k < VPER; ++k) {
            const int uu = tid + kThreads * k;
            const int pi = uu / (D * BS / 8);
            const int rem = uu % (D * BS / 8);
            const int d = rem / (BS / 8);
            const int t0 = pi * BS + (rem % (BS / 8)) * 8;  // 8 tokens t0 .. t0 + 7 of dim d
            // token 32 s + 16 t + 4 jj + i goes to position 32 s + 8 jj + 4 t + i,
            // i.e. to byte 8 t + 2 i of logical slot 4 s + jj: the 4-token groups
            // t0 and t0 + 4 (same t, jj and jj + 1) land in neighbouring slots
            const int s32 = t0 / 32;
            const int tt = (t0 % 32) / 16;
            const int jj = (t0 % 16) / 4;
            const int slot = 4 * s32 + jj;
            unsigned char* row_d = vb + d * VROW + 8 * tt;
            typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
            *reinterpret_cast<u32x2_t*>(row_d + ((slot ^ (d & 7)) * 16)) = u32x2_t{sv[k][0], sv[k][1]};
            *reinterpret_cast<u32x2_t*>(row_d + (((slot + 1) ^ (d & 7)) * 16)) = u32x2_t{sv[k][2], sv[k][3]};
        }
    };

    float m_run[2] = {neg_inf(), neg_inf()};
    float l_run[2] = {0.f, 0.f};
    f32x4_t acc[2][DC];
    for (int nt = 0; nt < 2; ++nt)
        for (int dc = 0; dc < DC; ++dc) acc[nt][dc] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int ci = 0; ci < nch; ++ci) {
        const int buf = ci & 1;
        if (ci + 1 < nch) load_chunk(ci + 1);                // in flight during the compute below
        if (has_cols && (!CAUSAL || start + ci * kTok <= wave_hi)) {
            const unsigned char* kb = lds + buf * (KBUF + VBUF);
            const unsigned char* vb = kb + KBUF;
            const int valid = min(kTok, end - (start + ci * kTok));

            // ---- scores (unscaled) of the 64 tokens for both column tiles
            f32x4_t st[2][kTok / 16];
            for (int rt = 0; rt < kTok / 16; ++rt) {
                u32x4_t kf[KSTEPS];
                for (int s = 0; s < KSTEPS; ++s)
                    kf[s] = *reinterpret_cast<const u32x4_t*>(kb + ((4 * s + j) * kTok + 16 * rt + r) * 16);
                for (int nt = 0; nt < 2; ++nt) {
                    st[nt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    for (int s = 0; s < KSTEPS; ++s)
                        st[nt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[s]), qf[nt][s],
                                                                             st[nt][rt], 0, 0, 0);
                }
            }

            // ---- online softmax per column tile, P in bf16 in the k order above.
            // |scale| is applied to the column max and inside the exponent's
            // fma, not to each score; only a chunk that ends early masks (its
            // missing tokens' scores are 0 against zeroed K rows: out of the
            // max, and weight 0); the row sums add the bf16 weights the P.V
            // product uses, two per dot2.
            const bool partial = valid < kTok;                       // wave-uniform
            // causal: some column of the wave stops inside this chunk
            const bool cut_cols = CAUSAL && start + ci * kTok + kTok - 1 > wave_lo;
            bf16x8_t pf[2][kTok / 32];
            if (partial || cut_cols) {
                // drop the missing (or, causal, unseen) tokens' scores from the
                // max (-inf) and their weights (0) once, here, so the common
                // path below has no selects
                for (int nt = 0; nt < 2; ++nt) {
                    const int cut = CAUSAL ? min(valid, lim[nt] - (start + ci * kTok) + 1) : valid;
                    for (int rt = 0; rt < kTok / 16; ++rt)
                        for (int i = 0; i < 4; ++i)
                            st[nt][rt][i] = 16 * rt + 4 * j + i < cut ? st[nt][rt][i] : neg_inf();
                }
            }
            for (int nt = 0; nt < 2; ++nt) {
                float mx = st[nt][0][0];
                for (int rt = 0; rt < kTok / 16; ++rt)
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[nt][rt][i]);
                mx = max_xor16(mx);
                mx = max_xor32(mx);
                mx *= sabs;                                          // -inf stays -inf
                const bool grow = mx > m_run[nt] + kRescaleSlack;
                if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                    const float mn = grow ? mx : m_run[nt];
                    const float alpha = m_run[nt] == neg_inf() ? 0.f : fast_exp2(m_run[nt] - mn);
                    for (int dc = 0; dc < DC; ++dc) acc[nt][dc] = acc[nt][dc] * alpha;
                    l_run[nt] *= alpha;
                    m_run[nt] = mn;
                }
                const float neg_m = m_run[nt] == neg_inf() ? 0.f : -m_run[nt];
                float psum = l_run[nt];
                for (int s2 = 0; s2 < kTok / 32; ++s2) {
                    // weights of k slots 2 q, 2 q + 1 (slot 4 t + i <-> score i of row tile 2 s2 + t);
                    // a masked score (-inf) gives exp2(-inf) = 0
                    uint32_t pk[4];
                    for (int q = 0; q < 4; ++q) {
                        const int t = q / 2;
                        const int i = 2 * (q % 2);
                        const float e0 = fast_exp2(fmaf(st[nt][2 * s2 + t][i], sabs, neg_m));
                        const float e1 = fast_exp2(fmaf(st[nt][2 * s2 + t][i + 1], sabs, neg_m));
                        const bf16x2_t pair = __builtin_convertvector(f32x2_t{e0, e1}, bf16x2_t);
                        psum = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, psum, false);
                        pk[q] = __builtin_bit_cast(uint32_t, pair);
                    }
                    pf[nt][s2] = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
                }
                l_run[nt] = psum;
            }

            // ---- P.V: V^T operands from LDS, one 16-byte read per lane and tile
            for (int s2 = 0; s2 < kTok / 32; ++s2)
                for (int dc = 0; dc < DC; ++dc) {
                    u32x4_t vf = *reinterpret_cast<const u32x4_t*>(
                        vb + (16 * dc + r) * VROW + (((4 * s2 + j) ^ (r & 7)) * 16));
                    if (CAUSAL && partial) {
                        // dword q holds tokens 32 s2 + 16 (q / 2) + 4 j + 2 (q % 2) and the
                        // next; past the context they may hold anything: zeroed, never
                        // multiplied by a zero weight
                        for (int q = 0; q < 4; ++q) {
                            const int tok = 32 * s2 + 16 * (q / 2) + 4 * j + 2 * (q % 2);
                            vf[q] &= (tok < valid ? 0x0000ffffu : 0u) | (tok + 1 < valid ? 0xffff0000u : 0u);
                        }
                    }
                    for (int nt = 0; nt < 2; ++nt)
                        acc[nt][dc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), pf[nt][s2],
                                                                              acc[nt][dc], 0, 0, 0);
                }
        }
        if (ci + 1 < nch) store_chunk(buf ^ 1);
        __syncthreads();
    }
    if (!has_cols) return;

    if (CAUSAL && !p.split) {
        // ---- one pass: the output rows of this wave's columns, normalised;
        // lane (c, j) holds dims 16 dc + 4 j + i
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
        for (int nt = 0; nt < 2; ++nt) {
            float l = l_run[nt];
            l = sum_xor16(l);
            l = sum_xor32(l);
            const int c = wc0 + 16 * nt + hl;
            if (c >= ncols) continue;
            const size_t orow = (size_t)(qr.row0 + c / G) * p.num_heads + (size_t)g * G + c % G;
            for (int dc = 0; dc < DC; ++dc) {
                uint32_t h2[2];
                for (int k = 0; k < 2; ++k) {
                    const uint32_t lo = f32_to_bf16(l > 0.f ? acc[nt][dc][2 * k] / l : 0.f);
                    const uint32_t hi = f32_to_bf16(l > 0.f ? acc[nt][dc][2 * k + 1] / l : 0.f);
                    h2[k] = lo | (hi << 16);
                }
                typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
                *reinterpret_cast<u32x2_t*>(out + orow * D + 16 * dc + 4 * j) = u32x2_t{h2[0], h2[1]};
            }
        }
        return;
    }

    // ---- partials of this wave's columns: lane (c, j) holds dims 16 dc + 4 j + i
    const int wsp = p.ws_parts > 0 ? p.ws_parts : p.max_parts;
    const size_t rows = ws_rows(p.num_tokens, p.num_heads, wsp);
    for (int nt = 0; nt < 2; ++nt) {
        float l = l_run[nt];
        l = sum_xor16(l);
        l = sum_xor32(l);
        const int c = wc0 + 16 * nt + hl;
        if (c >= ncols) continue;
        const size_t orow = (size_t)(qr.row0 + c / G) * p.num_heads + (size_t)g * G + c % G;
        const size_t rr = orow * wsp + part;
        for (int dc = 0; dc < DC; ++dc)
            *reinterpret_cast<f32x4_t*>(p.ws + rr * D + 16 * dc + 4 * j) = acc[nt][dc];
        if (j == 0) {
            p.ws[rows * D + rr] = m_run[nt];
            p.ws[rows * D + rows + rr] = l;
        }
    }
}

}  // namespace prefix_detail

}  // namespace pa_impl
