// Merge pass of the split-context path: partition p of (sequence, head) left
// its running max m_p (log2 units), running sum l_p and unnormalised
// accumulator acc_p; with M = max_p m_p the attention output is
//     out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// (the common factor 2^-M cancels).
//
// One wavefront per (sequence, head), four per workgroup.  Lane q holds the
// max, sum and weight 2^(m_q - M) of partition q (blocks of 64 partitions);
// M and the denominator are wave reductions.  Each lane then owns D / 64
// consecutive dims and walks the partitions, taking partition k's weight from
// lane k with a scalar read-lane and its accumulator slice with one 4- or
// 8-byte load (the wave reads a whole row, coalesced).  The first eight rows
// are loaded together with the maxima and sums, later ones four at a time.
// The output is rounded once to its dtype.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * kWave;
constexpr int kUnroll = 8;
constexpr int kPre = 16;         // partitions whose rows are loaded up front

template <int N>
struct FloatN;
template <>
struct FloatN<1> { typedef float T; };
template <>
struct FloatN<2> { typedef __attribute__((__vector_size__(2 * sizeof(float)))) float T; };

__device__ __forceinline__ float wave_max(float v) {
    for (int s = 32; s >= 1; s /= 2) v = fmaxf(v, __shfl_xor(v, s));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int s = 32; s >= 1; s /= 2) v += __shfl_xor(v, s);
    return v;
}

__device__ __forceinline__ float lane_value(float v, int k) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), k));
}

__device__ __forceinline__ int clamp_len(int L, int max_context_len) {
    return L < 0 ? 0 : (L > max_context_len ? max_context_len : L);
}

// Multi-query merge: positions query token t sees (0 if no sequence covers
// row t).  Its sequence is the last s with query_start[s] <= t (binary
// search over the wave-uniform t, so scalar loads); the rows that sequence
// covers come from query_rows, as in the partition kernel.
__device__ __forceinline__ int token_context(const ReduceParams& p, int t) {
    int lo = 0, hi = p.num_groups - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (p.query_start[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    const int L = clamp_len(p.context_lens[lo], p.max_context_len);
    const QueryRows qr = query_rows(p.query_start, lo, L, p.num_seqs, p.max_query_len);
    if (t < qr.row0 || t >= qr.row0 + qr.n) return 0;
    return L - qr.n + (t - qr.row0) + 1;
}

template <typename E>
__device__ __forceinline__ void store_out(E* out, size_t i, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* out, size_t i, float v) { out[i] = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* out, size_t i, float v) {
    out[i] = f32_to_bf16(v);
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads)
void decode_reduce_kernel(ReduceParams p) {
    constexpr int DPL = D / kWave;                 // dims per lane
    typedef typename FloatN<DPL>::T vec_t;
    static_assert(D % kWave == 0 && (DPL == 1 || DPL == 2), "head_dim");

    const int lane = threadIdx.x % kWave;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t bh = (size_t)blockIdx.x * kWavesPerBlock + w;
    const size_t pairs = (size_t)p.num_seqs * p.num_heads;
    if (bh >= pairs) return;
    const int b = (int)(bh / (size_t)p.num_heads);
    const size_t rows = ws_rows(p.num_seqs, p.num_heads, p.max_parts);
    const float* acc = p.ws + bh * p.max_parts * D;
    const float* wm = p.ws + rows * D + bh * p.max_parts;
    const float* wl = p.ws + rows * D + rows + bh * p.max_parts;
    E* out = reinterpret_cast<E*>(p.out) + bh * D;

    // Loads that do not depend on the context length go out before it is
    // known: the first kPre partitions' accumulator slices and this lane's
    // max and sum among the first kWave partitions.  Every slot below
    // max_parts lies inside the workspace row; slots past the sequence's
    // own partitions hold stale values and are masked once n is known.
    vec_t pre[kPre];
    {
        const float* row = acc + DPL * lane;
        for (int u = 0; u < kPre; ++u)
            pre[u] = u < p.max_parts ? *reinterpret_cast<const vec_t*>(row + (size_t)u * D) : vec_t{};
    }
    const float m0 = lane < p.max_parts ? wm[lane] : neg_inf();
    const float l0 = lane < p.max_parts ? wl[lane] : 0.f;

    const int L = p.query_start ? token_context(p, b) : clamp_len(p.context_lens[b], p.max_context_len);
    int n = (L + p.partition - 1) / p.partition;
    n += p.seq_first ? seq_slot_shift(p.seq_first[b], p.partition, p.prefix_partition) : p.slot_shift;
    n = n < 0 ? 0 : (n > p.max_parts ? p.max_parts : n);

    float M = lane < n ? m0 : neg_inf();
    for (int q = lane + kWave; q < n; q += kWave) M = fmaxf(M, wm[q]);
    M = wave_max(M);

    float a[DPL];
    for (int i = 0; i < DPL; ++i) a[i] = 0.f;
    float den = 0.f;
    for (int base = 0; base < n; base += kWave) {
        const int q = base + lane;
        const float mq = q < n ? (base == 0 ? m0 : wm[q]) : 0.f;
        const float wq = q < n ? fast_exp2(mq - M) : 0.f;
        den = fmaf(wq, q < n ? (base == 0 ? l0 : wl[q]) : 0.f, den);
        const int cnt = min(kWave, n - base);
        const float* row = acc + (size_t)base * D + DPL * lane;
        int k = 0;
        if (base == 0) {
            for (int u = 0; u < kPre; ++u) {
                if (u < cnt) {
                    const float wk = lane_value(wq, u);
                    if constexpr (DPL == 1) {
                        a[0] = fmaf(wk, pre[u], a[0]);
                    } else {
                        a[0] = fmaf(wk, pre[u][0], a[0]);
                        a[1] = fmaf(wk, pre[u][1], a[1]);
                    }
                }
            }
            k = min(kPre, cnt);
        }
        for (; k + kUnroll <= cnt; k += kUnroll) {
            vec_t v[kUnroll];
            for (int u = 0; u < kUnroll; ++u) v[u] = *reinterpret_cast<const vec_t*>(row + (size_t)(k + u) * D);
            for (int u = 0; u < kUnroll; ++u) {
                const float wk = lane_value(wq, k + u);
                if constexpr (DPL == 1) {
                    a[0] = fmaf(wk, v[u], a[0]);
                } else {
                    a[0] = fmaf(wk, v[u][0], a[0]);
                    a[1] = fmaf(wk, v[u][1], a[1]);
                }
            }
        }
        for (; k < cnt; ++k) {
            const vec_t v = *reinterpret_cast<const vec_t*>(row + (size_t)k * D);
            const float wk = lane_value(wq, k);
            if constexpr (DPL == 1) {
                a[0] = fmaf(wk, v, a[0]);
            } else {
                a[0] = fmaf(wk, v[0], a[0]);
                a[1] = fmaf(wk, v[1], a[1]);
            }
        }
    }
    den = wave_sum(den);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int i = 0; i < DPL; ++i) store_out<E>(out, (size_t)DPL * lane + i, den > 0.f ? a[i] * inv : 0.f);
}

template <typename E>
hipError_t launch_dtype(const ReduceParams& p, hipStream_t stream) {
    const uint64_t pairs = (uint64_t)p.num_seqs * p.num_heads;
    const dim3 grid((unsigned)((pairs + kWavesPerBlock - 1) / kWavesPerBlock));
    if (p.head_dim == 64)
        hipLaunchKernelGGL((decode_reduce_kernel<E, 64>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_reduce_kernel<E, 128>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(const ReduceParams& p, pa_dtype dtype, hipStream_t stream) {
    return dtype == PA_BF16 ? launch_dtype<uint16_t>(p, stream) : launch_dtype<float>(p, stream);
}

}  // namespace pa_impl
