// Merge pass of the split-context path: partition p of (sequence, head) left
// its running max m_p (log2 units), running sum l_p and unnormalised
// accumulator acc_p; with M = max_p m_p the attention output is
//     out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// (the common factor 2^-M cancels).  One workgroup per (sequence, head), one
// thread per output dim; the output is rounded once to its dtype.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {

namespace {

template <typename E>
__device__ __forceinline__ void put(E* out, size_t i, float v);
template <>
__device__ __forceinline__ void put<float>(float* out, size_t i, float v) { out[i] = v; }
template <>
__device__ __forceinline__ void put<uint16_t>(uint16_t* out, size_t i, float v) { out[i] = f32_to_bf16(v); }

template <typename E>
__global__ __launch_bounds__(128)
void decode_reduce_kernel(ReduceParams p) {
    const int D = p.head_dim;
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
    for (int q = 0; q < n; ++q) M = fmaxf(M, wm[q]);
    E* out = reinterpret_cast<E*>(p.out);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float num = 0.f, den = 0.f;
        for (int q = 0; q < n; ++q) {
            const float f = fast_exp2(wm[q] - M);
            num = fmaf(f, acc[(size_t)q * D + d], num);
            den = fmaf(f, wl[q], den);
        }
        put<E>(out, bh * D + d, den > 0.f ? num / den : 0.f);
    }
}

}  // namespace

hipError_t launch_decode_reduce(const ReduceParams& p, pa_dtype dtype, hipStream_t stream) {
    const dim3 grid((unsigned)((uint64_t)p.num_seqs * p.num_heads));
    const dim3 block((unsigned)(p.head_dim < 128 ? p.head_dim : 128));
    if (dtype == PA_BF16)
        hipLaunchKernelGGL(decode_reduce_kernel<uint16_t>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(decode_reduce_kernel<float>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa_impl
