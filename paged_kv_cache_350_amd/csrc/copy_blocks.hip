// Whole-page copy for copy-on-write forks: page dst becomes a bit-exact copy
// of page src, K and V, every kv head.
// [What is PagedAttention?, "Copy-on-Write Memory Forking"; PagedAttention
// Internals, "Copy-on-Write and Prefix Sharing"]
//
// A page (all kv heads) is one contiguous run of num_kv_heads * head_dim *
// block_size elements in each cache, so the copy is a flat 16-byte-vector
// stream.  Grid: x = pair, y = slice of the page; every workgroup moves
// kVecPerBlock 16-byte vectors of K and the same of V.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa_impl {

namespace {

constexpr int kThreads = 256;
constexpr int kVecPerBlock = 4 * kThreads;

__global__ __launch_bounds__(kThreads)
void copy_blocks_kernel(u32x4_t* __restrict__ k_cache, u32x4_t* __restrict__ v_cache,
                        const int64_t* __restrict__ block_mapping, int64_t page_vecs,
                        int64_t num_blocks) {
    const int64_t src = block_mapping[2 * (int64_t)blockIdx.x];
    const int64_t dst = block_mapping[2 * (int64_t)blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    const int64_t begin = (int64_t)blockIdx.y * kVecPerBlock;
    const int64_t end = begin + kVecPerBlock < page_vecs ? begin + kVecPerBlock : page_vecs;
    const u32x4_t* ks = k_cache + src * page_vecs;
    const u32x4_t* vs = v_cache + src * page_vecs;
    u32x4_t* kd = k_cache + dst * page_vecs;
    u32x4_t* vd = v_cache + dst * page_vecs;
    for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) {
        const u32x4_t a = ks[i];
        const u32x4_t b = vs[i];
        kd[i] = a;
        vd[i] = b;
    }
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                              int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                              hipStream_t stream) {
    const int64_t elem = dtype == PA_BF16 ? 2 : 4;
    const int64_t page_vecs = (int64_t)num_kv_heads * head_dim * block_size * elem / 16;
    const dim3 grid((unsigned)num_pairs, (unsigned)((page_vecs + kVecPerBlock - 1) / kVecPerBlock));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, stream,
                       (u32x4_t*)k_cache, (u32x4_t*)v_cache, block_mapping, page_vecs,
                       num_blocks);
    return hipGetLastError();
}

}  // namespace pa_impl
