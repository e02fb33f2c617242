// Paged decode attention on the vector ALU (fp32 and bf16 caches).
//
// Each workgroup owns one (sequence, kv head, partition) and computes all G
// query heads of that kv head, so every K/V byte of the partition is read
// once.  The block table is read in place and K/V pages are loaded straight
// from their physical addresses -- no gathered copy is ever written.
// [PagedAttention Internals, "How PagedAttention Works" item 3; What is
// PagedAttention?, "On-the-Fly CUDA Block Fetching"]
//
// Wave-level scheme, one page (block_size tokens) at a time, pages of the
// partition dealt round-robin to the four wavefronts:
//   Q.K^T  lane = (token o = lane % BS, chunk group j = lane / BS).  A K page
//          tile is [D/X chunks][BS tokens][X], so for each chunk the BS token
//          rows sit side by side: lane (o, j) loads 16 bytes of token o for
//          chunks j, j + NJ, ... (coalesced per chunk), multiplies by q from
//          LDS, and the NJ partial dots are summed with lane shuffles.
//   softmax running max / sum per head (online form, scores in log2 units);
//          masked slots of a partly filled page become -inf by selection.
//   P.V    lane = value dims (lane, lane + 64).  A V page tile is
//          [D dims][BS tokens], so a lane reads its dims' BS values as 16-byte
//          vectors; the probabilities come from LDS (one write per token).
// At the end the four waves' (m, l, acc) are merged in LDS, and the result is
// either the normalised output (single pass) or the partition's partials.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

template <typename E>
__device__ __forceinline__ float load_elem(const E* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// Unpack one 16-byte vector into X floats.
template <typename E, int X>
__device__ __forceinline__ void unpack16(u32x4_t raw, float (&f)[X]) {
    if constexpr (sizeof(E) == 4) {
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = raw[i];
            f[i] = u32_as_f32(u);
        }
    } else {
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = raw[i];
            f[2 * i] = u32_as_f32(u << 16);
            f[2 * i + 1] = u32_as_f32(u & 0xffff0000u);
        }
    }
}

template <typename E>
__device__ __forceinline__ void store_out(E* out, size_t idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* out, size_t idx, float v) { out[idx] = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* out, size_t idx, float v) {
    out[idx] = f32_to_bf16(v);
}

template <typename E, int D, int BS, int GMAX, bool STREAM>
__global__ __launch_bounds__(kThreads)
void decode_valu_kernel(DecodeParams p) {
    constexpr int X = 16 / (int)sizeof(E);     // elements per 16-byte chunk
    constexpr int NC = D / X;                  // chunks per K row
    constexpr int NJ = kWave / BS;             // lane groups per page
    constexpr int CPL = NC / NJ;               // K chunks per lane
    constexpr int DPL = D / kWave;             // value dims per lane
    constexpr int VV = BS * (int)sizeof(E) / 16;   // 16-byte vectors per V dim row
    static_assert(NC % NJ == 0 && D % kWave == 0 && VV >= 1, "shape");

    extern __shared__ float smem[];
    float* sq = smem;                          // [GMAX][D]     query (fp32)
    float* sp = sq + GMAX * D;                 // [kWaves][BS][GMAX] probabilities
    float* sm_m = sp + kWaves * BS * GMAX;     // [kWaves][GMAX]
    float* sm_l = sm_m + kWaves * GMAX;        // [kWaves][GMAX]
    float* sacc = sm_l + kWaves * GMAX;        // [kWaves][GMAX][D]

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform

    const WorkItem wi = decode_work_item(blockIdx.x, (uint32_t)p.num_seqs,
                                         (uint32_t)(p.num_kv_heads * p.max_parts));
    const int b = wi.b;
    const int g = wi.q % p.num_kv_heads;
    const int slot = wi.q / p.num_kv_heads;
    const int G = p.group;

    int L = p.context_lens[b];
    const int cap = min(p.max_context_len, p.max_blocks_per_seq * BS);
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int part = partition_of(slot, p.max_parts, L, p.partition, STREAM);
    E* out = reinterpret_cast<E*>(p.out);
    const size_t head0 = (size_t)b * p.num_heads + (size_t)g * G;
    if (part < 0) {
        if (!p.split && slot == 0) {                  // single pass, empty context: zeros
            for (int e = tid; e < G * D; e += kThreads) store_out<E>(out, head0 * D + e, 0.f);
        }
        return;
    }
    const int start = part * p.partition;
    const int end = min(start + p.partition, L);

    // Fused append (pa_decode_append): the workgroup that reads position
    // L - 1 first stores kv head g's new K and V rows into that slot; the
    // barrier after the query staging below makes the stores visible to the
    // whole workgroup, which then reads the new token like any other.  No
    // other workgroup reads that page (see the matrix-core kernel).  A page
    // id outside the pool writes nothing.
    const int* trow = p.block_tables + (size_t)b * p.max_blocks_per_seq;
    const bool appends = p.k_new != nullptr && end == L &&    // workgroup-uniform
                         (p.append_mask == nullptr || p.append_mask[b] >= 0) &&
                         (uint32_t)trow[(L - 1) / BS] < (uint64_t)p.num_blocks;
    if (appends) {
        constexpr int NCH = D * (int)sizeof(E) / 16;        // 16-byte chunks per K row
        const int pos = L - 1;
        const int pg = trow[pos / BS];
        const int off = pos % BS;
        const size_t tile = ((size_t)pg * p.num_kv_heads + g) * (size_t)D * BS;
        const size_t src = ((size_t)b * p.num_kv_heads + g) * D;
        const E* kn = reinterpret_cast<const E*>(p.k_new) + src;
        const E* vn = reinterpret_cast<const E*>(p.v_new) + src;
        E* kw = const_cast<E*>(reinterpret_cast<const E*>(p.k_cache)) + tile;
        E* vw = const_cast<E*>(reinterpret_cast<const E*>(p.v_cache)) + tile;
        for (int c = tid; c < NCH; c += kThreads) st16(kw + ((size_t)c * BS + off) * X, ld16(kn + c * X));
        for (int d = tid; d < D; d += kThreads) vw[(size_t)d * BS + off] = vn[d];
    }

    const E* qb = reinterpret_cast<const E*>(p.q) + head0 * D;
    for (int e = tid; e < GMAX * D; e += kThreads) {
        sq[e] = (e / D) < G ? load_elem<E>(qb + e) : 0.f;
    }
    __syncthreads();

    const int* row = p.block_tables + (size_t)b * p.max_blocks_per_seq;
    const int first_blk = start / BS;
    const int last_blk = (end - 1) / BS;
    const E* kc = reinterpret_cast<const E*>(p.k_cache);
    const E* vc = reinterpret_cast<const E*>(p.v_cache);
    const size_t tile_elems = (size_t)D * BS;

    const int o = lane % BS;
    const int j = lane / BS;
    float m[GMAX], l[GMAX], acc[GMAX][DPL];
    for (int h = 0; h < GMAX; ++h) {
        m[h] = neg_inf();
        l[h] = 0.f;
        for (int i = 0; i < DPL; ++i) acc[h][i] = 0.f;
    }

    for (int blk = first_blk + w; blk <= last_blk; blk += kWaves) {
        int page = row[blk];
        if ((uint32_t)page >= (uint64_t)p.num_blocks) page = 0;     // guard a bad entry
        const int valid = min(BS, end - blk * BS);
        const size_t tile = ((size_t)page * p.num_kv_heads + g) * tile_elems;
        const E* kt = kc + tile;
        const E* vt = vc + tile;

        // ---- Q.K^T: partial dots over this lane's chunks, then across groups
        float ps[GMAX];
        for (int h = 0; h < GMAX; ++h) ps[h] = 0.f;
        u32x4_t kraw[CPL];
        for (int cc = 0; cc < CPL; ++cc) kraw[cc] = ld16_kv<STREAM>(kt + ((cc * NJ + j) * BS + o) * X);
        for (int cc = 0; cc < CPL; ++cc) {
            const int c = cc * NJ + j;
            float kf[X];
            unpack16<E, X>(kraw[cc], kf);
            for (int h = 0; h < GMAX; ++h) {
                const float* qh = sq + h * D + c * X;
                for (int x = 0; x < X; ++x) ps[h] = fmaf(kf[x], qh[x], ps[h]);
            }
        }
        for (int sh = BS; sh < kWave; sh *= 2)
            for (int h = 0; h < GMAX; ++h) ps[h] += __shfl_xor(ps[h], sh);

        // ---- online softmax (log2 units)
        float s[GMAX], mx[GMAX];
        for (int h = 0; h < GMAX; ++h) {
            s[h] = o < valid ? ps[h] * p.scale_log2 : neg_inf();
            mx[h] = s[h];
        }
        for (int sh = 1; sh < BS; sh *= 2)
            for (int h = 0; h < GMAX; ++h) mx[h] = fmaxf(mx[h], __shfl_xor(mx[h], sh));
        float alpha[GMAX];
        for (int h = 0; h < GMAX; ++h) {
            const float mn = fmaxf(m[h], mx[h]);
            alpha[h] = fast_exp2(m[h] - mn);
            const float pr = fast_exp2(s[h] - mn);
            l[h] = l[h] * alpha[h] + pr;
            m[h] = mn;
            if (j == 0) sp[(w * BS + o) * GMAX + h] = pr;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- P.V
        for (int i = 0; i < DPL; ++i) {
            const int d = lane + kWave * i;
            float vals[BS];
            for (int vv = 0; vv < VV; ++vv) {
                float f[X];
                unpack16<E, X>(ld16_kv<STREAM>(vt + (size_t)d * BS + vv * X), f);
                for (int x = 0; x < X; ++x) vals[vv * X + x] = f[x];
            }
            if (valid < BS)
                for (int t = 0; t < BS; ++t) vals[t] = t < valid ? vals[t] : 0.f;
            for (int h = 0; h < GMAX; ++h) acc[h][i] *= alpha[h];
            for (int t = 0; t < BS; ++t) {
                const float* pt = sp + (w * BS + t) * GMAX;
                for (int h = 0; h < GMAX; ++h) acc[h][i] = fmaf(pt[h], vals[t], acc[h][i]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- merge the four waves
    for (int sh = 1; sh < BS; sh *= 2)
        for (int h = 0; h < GMAX; ++h) l[h] += __shfl_xor(l[h], sh);
    if (lane == 0) {
        for (int h = 0; h < GMAX; ++h) {
            sm_m[w * GMAX + h] = m[h];
            sm_l[w * GMAX + h] = l[h];
        }
    }
    for (int h = 0; h < GMAX; ++h)
        for (int i = 0; i < DPL; ++i) sacc[(w * GMAX + h) * D + lane + kWave * i] = acc[h][i];
    __syncthreads();

    const size_t rows = ws_rows(p.num_seqs, p.num_heads, p.max_parts);
    for (int e = tid; e < G * D; e += kThreads) {
        const int h = e / D;
        const int d = e % D;
        float M = neg_inf();
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww * GMAX + h]);
        float num = 0.f, den = 0.f;
        if (M != neg_inf()) {
            for (int ww = 0; ww < kWaves; ++ww) {
                const float f = fast_exp2(sm_m[ww * GMAX + h] - M);
                num = fmaf(f, sacc[(ww * GMAX + h) * D + d], num);
                den = fmaf(f, sm_l[ww * GMAX + h], den);
            }
        }
        if (p.split) {
            const size_t r = (head0 + h) * p.max_parts + part;
            p.ws[r * D + d] = num;
            if (d == 0) {
                p.ws[rows * D + r] = M;
                p.ws[rows * D + rows + r] = den;
            }
        } else {
            store_out<E>(out, (head0 + h) * D + d, den > 0.f ? num / den : 0.f);
        }
    }
}

template <typename E, int D, int BS, int GMAX, bool STREAM>
hipError_t launch_shape(const DecodeParams& p, hipStream_t stream) {
    const size_t smem = sizeof(float) *
        (GMAX * D + kWaves * BS * GMAX + 2 * kWaves * GMAX + kWaves * GMAX * D);
    const uint64_t nwg = (uint64_t)p.num_seqs * p.num_kv_heads * p.max_parts;
    hipLaunchKernelGGL((decode_valu_kernel<E, D, BS, GMAX, STREAM>), dim3((unsigned)nwg), dim3(kThreads),
                       smem, stream, p);
    return hipGetLastError();
}

template <typename E, int D, int BS, bool STREAM>
hipError_t launch_group(const DecodeParams& p, hipStream_t stream) {
    if (p.group <= 1) return launch_shape<E, D, BS, 1, STREAM>(p, stream);
    if (p.group <= 2) return launch_shape<E, D, BS, 2, STREAM>(p, stream);
    if (p.group <= 4) return launch_shape<E, D, BS, 4, STREAM>(p, stream);
    if (p.group <= 8) return launch_shape<E, D, BS, 8, STREAM>(p, stream);
    return launch_shape<E, D, BS, 16, STREAM>(p, stream);
}

template <typename E, int D, int BS>
hipError_t launch_policy(const DecodeParams& p, hipStream_t stream) {
    return p.stream_kv ? launch_group<E, D, BS, true>(p, stream)
                       : launch_group<E, D, BS, false>(p, stream);
}

template <typename E>
hipError_t launch_dtype(const DecodeParams& p, hipStream_t stream) {
    if (p.head_dim == 64)
        return p.block_size == 16 ? launch_policy<E, 64, 16>(p, stream)
                                  : launch_policy<E, 64, 32>(p, stream);
    return p.block_size == 16 ? launch_policy<E, 128, 16>(p, stream)
                              : launch_policy<E, 128, 32>(p, stream);
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, pa_dtype dtype, hipStream_t stream) {
    return dtype == PA_BF16 ? launch_dtype<uint16_t>(p, stream) : launch_dtype<float>(p, stream);
}

}  // namespace pa_impl
