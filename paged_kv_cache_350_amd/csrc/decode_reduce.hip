// Merge pass of the split-context path: partition p of (sequence, head) left
// its running max m_p (log2 units), running sum l_p and unnormalised
// accumulator acc_p; with M = max_p m_p the attention output is
//     out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// (the common factor 2^-M cancels).
//
// One workgroup of 256 threads per (sequence, head).  Pass 1: threads load the
// partition maxima and reduce M across the workgroup; each partition's weight
// 2^(m_p - M) goes to LDS.  Pass 2: thread t owns 4 consecutive dims
// (t % (D/4)) and every (256 / (D/4))-th partition, accumulating weighted
// 16-byte rows; the partial sums meet in LDS and the first D/4 threads round
// and store.  The output is rounded once to its dtype.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxStaged = 1024;          // partition weights held in LDS per pass

template <typename E>
__device__ __forceinline__ void put4(E* out, size_t i, const float (&v)[4]);
template <>
__device__ __forceinline__ void put4<float>(float* out, size_t i, const float (&v)[4]) {
    for (int k = 0; k < 4; ++k) out[i + k] = v[k];
}
template <>
__device__ __forceinline__ void put4<uint16_t>(uint16_t* out, size_t i, const float (&v)[4]) {
    for (int k = 0; k < 4; ++k) out[i + k] = f32_to_bf16(v[k]);
}

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int s = 32; s >= 1; s /= 2) v = fmaxf(v, __shfl_xor(v, s));
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads)
void decode_reduce_kernel(ReduceParams p) {
    constexpr int NQ = D / 4;                 // float4 groups per row
    constexpr int NP = kThreads / NQ;         // partitions summed in parallel
    __shared__ float s_w[kMaxStaged];         // 2^(m_p - M)
    __shared__ float s_red[kThreads / kWave];
    __shared__ float s_acc[NP][D];
    __shared__ float s_den[NP];

    const size_t bh = blockIdx.x;
    const int b = (int)(bh / (size_t)p.num_heads);
    int L = p.context_lens[b];
    L = L < 0 ? 0 : (L > p.max_context_len ? p.max_context_len : L);
    int n = (L + p.partition - 1) / p.partition;
    n = n > p.max_parts ? p.max_parts : n;

    const size_t rows = ws_rows(p.num_seqs, p.num_heads, p.max_parts);
    const float* acc = p.ws + bh * p.max_parts * D;
    const float* wm = p.ws + rows * D + bh * p.max_parts;
    const float* wl = p.ws + rows * D + rows + bh * p.max_parts;

    float M = neg_inf();
    for (int q = threadIdx.x; q < n; q += kThreads) M = fmaxf(M, wm[q]);
    M = block_max(M, s_red);

    const int t = threadIdx.x;
    const int dq = t % NQ;
    const int pl = t / NQ;
    float a4[4] = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int base = 0; base < n; base += kMaxStaged) {
        const int cnt = min(kMaxStaged, n - base);
        for (int q = t; q < cnt; q += kThreads) s_w[q] = fast_exp2(wm[base + q] - M);
        __syncthreads();
        for (int q = pl; q < cnt; q += NP) {
            const float w = s_w[q];
            const u32x4_t raw = ld16(acc + (size_t)(base + q) * D + 4 * dq);
            for (int k = 0; k < 4; ++k) a4[k] = fmaf(w, u32_as_f32(raw[k]), a4[k]);
            if (dq == 0) den = fmaf(w, wl[base + q], den);
        }
        __syncthreads();
    }
    for (int k = 0; k < 4; ++k) s_acc[pl][4 * dq + k] = a4[k];
    if (dq == 0) s_den[pl] = den;
    __syncthreads();
    if (t < NQ) {
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        float dsum = 0.f;
        for (int q = 0; q < NP; ++q) {
            dsum += s_den[q];
            for (int k = 0; k < 4; ++k) o[k] += s_acc[q][4 * t + k];
        }
        const float inv = dsum > 0.f ? 1.f / dsum : 0.f;
        for (int k = 0; k < 4; ++k) o[k] = dsum > 0.f ? o[k] * inv : 0.f;
        put4<E>(reinterpret_cast<E*>(p.out), bh * D + 4 * t, o);
    }
}

template <typename E>
hipError_t launch_dtype(const ReduceParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)((uint64_t)p.num_seqs * p.num_heads));
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
