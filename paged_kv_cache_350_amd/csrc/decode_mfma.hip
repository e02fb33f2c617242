// Paged decode attention on the MFMA matrix cores (bf16 caches, gfx950).
//
// Same contract as the vector-ALU kernel: one workgroup per (sequence, kv
// head, partition), all G <= 16 query heads of the kv head at once, K/V read
// in place through the block table.  [PagedAttention Internals, "How
// PagedAttention Works" item 3; What is PagedAttention?, "On-the-Fly CUDA
// Block Fetching"]
//
// Why matrix cores: with grouped-query attention the G query heads of one kv
// head share every K and V row, so Q.K^T over a tile of tokens is a genuine
// [tokens x D] . [D x G] product and P.V a [D x tokens] . [tokens x G] one.
// On the vector ALU they cost ~2G FMAs per cached element plus lane
// reductions, which approaches the VALU rate at G = 8; one 16x16x32 bf16
// MFMA retires 8192 of them.  G is padded to 16 (zero query rows).
//
// Work unit: a chunk of 32 tokens (two 16-token pages or one 32-token page).
// Inside a chunk, token slot tau = 0..31 is the tau-th token of the chunk.
//
//   Q.K^T  v_mfma_f32_16x16x32_bf16, A = K (rows = tokens), B = Q^T
//          (columns = heads), D/32 k-steps, two row tiles t = 0, 1.
//          Row r of tile t holds tau = 8 (r / 4) + 4 t + r % 4.  The result
//          layout (lane: column lane % 16, rows 4 (lane / 16) + i) then gives
//          lane (h, j) the scores of head h for tau = 8 j .. 8 j + 7.
//          K pages are [D/8 chunks][BS][8]: lane (r, j) of k-step s loads the
//          16 bytes of chunk 4 s + j of its token, four 64-byte runs per
//          quarter-wave.
//   softmax per head: chunk max over the lane's 8 scores, then across the
//          four lane groups; running max / sum rescaled by 2^(m_old - m_new).
//   P.V    v_mfma_f32_16x16x32_bf16, A = V^T (rows = 16 dims), B = P^T
//          (columns = heads).  Lane (h, j) already holds P for tau = 8 j ..
//          8 j + 7 -- exactly its B operand -- and V pages are dim-major
//          [D][BS], so the A operand is one 16-byte load of 8 consecutive
//          tokens of dim 16 dc + lane % 16.  No data is exchanged between
//          lanes and nothing goes through LDS inside the loop.
// Masking of the last, partly valid chunk selects -inf scores and zero V
// values (never multiplies a possibly-NaN slot by zero).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunk = 32;          // tokens per MFMA step (k of the P.V product)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int D, int BS>
__global__ __launch_bounds__(kThreads)
void decode_mfma_kernel(DecodeParams p) {
    constexpr int KSTEPS = D / 32;   // Q.K^T k-steps
    constexpr int DC = D / 16;       // 16-dim output tiles of P.V
    static_assert(BS == 16 || BS == 32, "block size");

    extern __shared__ float smem[];
    float* sm_m = smem;                          // [kWaves][16]
    float* sm_l = sm_m + kWaves * 16;            // [kWaves][16]
    float* sacc = sm_l + kWaves * 16;            // [kWaves][G][D]

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int hl = lane % 16;        // head (column) of this lane
    const int j = lane / 16;         // lane group

    const WorkItem wi = decode_work_item(blockIdx.x, (uint32_t)p.num_seqs,
                                         (uint32_t)(p.num_kv_heads * p.max_parts));
    const int b = wi.b;
    const int g = wi.q % p.num_kv_heads;
    const int part = wi.q / p.num_kv_heads;
    const int G = p.group;

    int L = p.context_lens[b];
    const int cap = min(p.max_context_len, p.max_blocks_per_seq * BS);
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int start = part * p.partition;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
    const size_t head0 = (size_t)b * p.num_heads + (size_t)g * G;
    if (start >= L) {
        if (!p.split && part == 0) {
            for (int e = tid; e < G * D; e += kThreads) out[head0 * D + e] = 0;
        }
        return;
    }
    const int end = min(start + p.partition, L);

    // Q^T as the B operand: lane (hl, j) holds head hl, dims 32 s + 8 j .. + 8.
    bf16x8_t qf[KSTEPS];
    {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                               (head0 + (hl < G ? hl : 0)) * D;
        for (int s = 0; s < KSTEPS; ++s) {
            u32x4_t raw = ld16(qrow + 32 * s + 8 * j);
            if (hl >= G) raw = u32x4_t{0u, 0u, 0u, 0u};
            qf[s] = as_bf16x8(raw);
        }
    }

    const int* row = p.block_tables + (size_t)b * p.max_blocks_per_seq;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(p.k_cache);
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(p.v_cache);
    const size_t tile_elems = (size_t)D * BS;
    const size_t kv_heads = (size_t)p.num_kv_heads;

    const int r = lane % 16;
    const int tau_k0 = 8 * (r / 4) + (r % 4);    // Q.K^T row r of tile 0; tile 1 adds 4
    const int tau_v0 = 8 * j;                    // P.V k-slots of this lane: tau_v0 .. + 7

    float m_run = neg_inf();
    float l_run = 0.f;
    f32x4_t acc[DC];
    for (int dc = 0; dc < DC; ++dc) acc[dc] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (end - start + kChunk - 1) / kChunk;
    for (int ci = w; ci < nchunks; ci += kWaves) {
        const int cstart = start + ci * kChunk;
        const int valid = min(kChunk, end - cstart);
        const int blk0 = cstart / BS;
        int pg0 = row[blk0];
        if ((uint32_t)pg0 >= (uint64_t)p.num_blocks) pg0 = 0;
        int pg1 = pg0;
        if (BS == 16 && valid > 16) {
            pg1 = row[blk0 + 1];
            if ((uint32_t)pg1 >= (uint64_t)p.num_blocks) pg1 = 0;
        }

        // ---- loads: K for both row tiles, V for every 16-dim tile
        u32x4_t kraw[2][KSTEPS];
        for (int t = 0; t < 2; ++t) {
            const int tau = tau_k0 + 4 * t;
            const int page = (BS == 16 && tau >= 16) ? pg1 : pg0;
            const uint16_t* base = kc + ((size_t)page * kv_heads + g) * tile_elems + (tau % BS) * 8;
            for (int s = 0; s < KSTEPS; ++s) kraw[t][s] = ld16(base + (size_t)(4 * s + j) * BS * 8);
        }
        u32x4_t vraw[DC];
        {
            const int page = (BS == 16 && tau_v0 >= 16) ? pg1 : pg0;
            const uint16_t* base = vc + ((size_t)page * kv_heads + g) * tile_elems + (tau_v0 % BS);
            for (int dc = 0; dc < DC; ++dc) vraw[dc] = ld16(base + (size_t)(16 * dc + r) * BS);
        }

        // ---- S = K . Q^T
        f32x4_t st[2];
        for (int t = 0; t < 2; ++t) {
            st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < KSTEPS; ++s)
                st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kraw[t][s]), qf[s], st[t], 0, 0, 0);
        }

        // ---- online softmax; lane holds head hl at tau = tau_v0 + k
        float sc[8];
        for (int t = 0; t < 2; ++t)
            for (int i = 0; i < 4; ++i) sc[4 * t + i] = st[t][i] * p.scale_log2;
        if (valid < kChunk) {
            for (int k = 0; k < 8; ++k) sc[k] = (tau_v0 + k < valid) ? sc[k] : neg_inf();
        }
        float mx = sc[0];
        for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sc[k]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - mn);
        m_run = mn;
        bf16x8_t pf;
        float psum = 0.f;
        for (int k = 0; k < 8; ++k) {
            const bf16_t pb = (bf16_t)fast_exp2(sc[k] - mn);
            pf[k] = pb;
            psum += (float)pb;           // normalise with the weights actually used
        }
        l_run = l_run * alpha + psum;

        // ---- O^T += V^T . P^T
        if (valid < kChunk) {
            // zero the value slots past the context (lane's k-slots tau_v0 + 0..7)
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = (tau_v0 + 2 * q < valid) ? 0x0000ffffu : 0u;
                const uint32_t hi = (tau_v0 + 2 * q + 1 < valid) ? 0xffff0000u : 0u;
                for (int dc = 0; dc < DC; ++dc) vraw[dc][q] &= (lo | hi);
            }
        }
        for (int dc = 0; dc < DC; ++dc) {
            acc[dc] = acc[dc] * alpha;
            acc[dc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vraw[dc]), pf, acc[dc], 0, 0, 0);
        }
    }

    // ---- merge the four waves; lane (hl, j) holds dims 16 dc + 4 j + i of head hl
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
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

    const size_t rows = ws_rows(p.num_seqs, p.num_heads, p.max_parts);
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
            const size_t rr = (head0 + h) * p.max_parts + part;
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

template <int D, int BS>
hipError_t launch_shape(const DecodeParams& p, hipStream_t stream) {
    const size_t smem = sizeof(float) * (2 * kWaves * 16 + (size_t)kWaves * p.group * D);
    const uint64_t nwg = (uint64_t)p.num_seqs * p.num_kv_heads * p.max_parts;
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS>), dim3((unsigned)nwg), dim3(kThreads), smem,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
    if (p.head_dim == 64)
        return p.block_size == 16 ? launch_shape<64, 16>(p, stream) : launch_shape<64, 32>(p, stream);
    return p.block_size == 16 ? launch_shape<128, 16>(p, stream) : launch_shape<128, 32>(p, stream);
}

}  // namespace pa_impl
