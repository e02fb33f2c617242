// The shared-prefix step's launch: the LDS-staged prefix kernel (body and
// design in decode_prefix_body.h) together with the decode kernel's
// shared-page path (decode_mfma_body.h) over the rest of every context.
#include "decode_mfma_body.h"
#include "decode_multi_body.h"
#include "decode_prefix_body.h"

namespace pa_impl {

namespace {

using namespace prefix_detail;

// The shared-prefix stage and the rest of every context in one launch:
// workgroups 0 .. n_pre - 1 are the LDS-staged prefix kernel (4 waves, 128
// columns), the others the decode kernel's shared-page path over each
// sequence's own positions (4 waves).  The prefix stage is bound by its
// matrix and LDS work and the rest by memory, so they share the compute
// units: with about one prefix workgroup per unit (the host sizes the
// prefix partitions so) and two workgroups per unit (64 KiB of LDS each,
// two waves per SIMD), every unit streams sequences' pages in its second
// slot while its prefix workgroup computes, instead of the two stages
// following each other.  n_pre is a multiple of the XCD count, so a rest
// workgroup keeps its XCD-aware work mapping.
template <int D, int BS>
__global__ __launch_bounds__(4 * kWave, 2)
void decode_prefix_rest_kernel(DecodeParams pre, DecodeParams rest, uint32_t n_pre) {
    extern __shared__ __align__(16) unsigned char lds[];
    if (blockIdx.x < n_pre)
        decode_prefix_body<D, BS, 4>(pre, blockIdx.x, lds);
    else
        mfma_detail::decode_mfma_body<D, BS, false, 4>(rest, blockIdx.x - n_pre, reinterpret_cast<float*>(lds));
}

template <int D, int BS>
hipError_t launch_fused_shape(const DecodeParams& pre, const DecodeParams& rest, hipStream_t stream) {
    constexpr size_t kBuf = (size_t)(D / 8) * kTok * 16 + (size_t)D * kTok * 2;
    const uint64_t units = (uint64_t)pre.num_seqs * pre.num_kv_heads * pre.max_parts;
    const uint64_t n_pre = (units + kXcds - 1) / kXcds * kXcds * (uint64_t)pre.col_groups;
    const uint64_t n_rest = (uint64_t)rest.num_seqs * rest.num_kv_heads * (rest.max_parts - rest.first_part);
    const size_t rest_smem = sizeof(float) * (2 * 4 * 16 + (size_t)4 * rest.group * D);
    const size_t smem = 2 * kBuf > rest_smem ? 2 * kBuf : rest_smem;
    if (n_pre + n_rest == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_prefix_rest_kernel<D, BS>), dim3((unsigned)(n_pre + n_rest)), dim3(4 * kWave), smem,
                       stream, pre, rest, (uint32_t)n_pre);
    return hipGetLastError();
}

// The same for a prefix stage of fewer columns: the multi-query kernel (one
// or two 16-column tiles per workgroup, ordinary loads; each workgroup reads
// its partition's pages itself) with the rest of every context beside it on
// the compute units.  Workgroups n_pre .. n_pre_pad - 1 are idle padding to
// a multiple of the XCD count.  One tile holds the kernel to three waves
// per SIMD, so that two rest workgroups fit beside a prefix workgroup.
template <int D, int BS, int NT>
__global__ __launch_bounds__(4 * kWave, NT == 1 ? 3 : 2)
void decode_multi_rest_kernel(DecodeParams pre, DecodeParams rest, uint32_t n_pre, uint32_t n_pre_pad) {
    extern __shared__ float smem[];
    if (blockIdx.x < n_pre_pad) {
        if (blockIdx.x < n_pre)
            multi_detail::decode_multi_body<D, BS, NT, kPolicyReuse, 4>(pre, blockIdx.x, smem);
    } else {
        mfma_detail::decode_mfma_body<D, BS, false, 4>(rest, blockIdx.x - n_pre_pad, smem);
    }
}

template <int D, int BS, int NT>
hipError_t launch_multi_fused_shape(const DecodeParams& pre, const DecodeParams& rest, hipStream_t stream) {
    const uint64_t n_pre = (uint64_t)pre.num_seqs * pre.num_kv_heads * pre.col_groups * pre.max_parts;
    const uint64_t n_pre_pad = (n_pre + kXcds - 1) / kXcds * kXcds;
    const uint64_t n_rest = (uint64_t)rest.num_seqs * rest.num_kv_heads * (rest.max_parts - rest.first_part);
    const size_t pre_smem = sizeof(float) * (2 * 4 * 16 + (size_t)4 * 16 * D);
    const size_t rest_smem = sizeof(float) * (2 * 4 * 16 + (size_t)4 * rest.group * D);
    const size_t smem = pre_smem > rest_smem ? pre_smem : rest_smem;
    if (n_pre_pad + n_rest == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_multi_rest_kernel<D, BS, NT>), dim3((unsigned)(n_pre_pad + n_rest)), dim3(4 * kWave),
                       smem, stream, pre, rest, (uint32_t)n_pre, (uint32_t)n_pre_pad);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_multi_fused_tiles(const DecodeParams& pre, const DecodeParams& rest, hipStream_t stream) {
    if (pre.head_dim == 64)
        return pre.block_size == 16 ? launch_multi_fused_shape<64, 16, NT>(pre, rest, stream)
                                    : launch_multi_fused_shape<64, 32, NT>(pre, rest, stream);
    return pre.block_size == 16 ? launch_multi_fused_shape<128, 16, NT>(pre, rest, stream)
                                : launch_multi_fused_shape<128, 32, NT>(pre, rest, stream);
}

// The LDS-staged body on its own as the multi-query kernel of many columns
// (a prompt chunk): causal rows, one pass or partials for the merge.
// Workgroups take (sequence, kv head, partition) units spread over the XCDs
// with every column group of a unit on one XCD, so the groups that stage the
// same pages share its L2.
template <int D, int BS>
__global__ __launch_bounds__(4 * kWave, 2)
void decode_multi_wide_kernel(DecodeParams p) {
    extern __shared__ __align__(16) unsigned char lds[];
    decode_prefix_body<D, BS, 4, true>(p, blockIdx.x, lds);
}

template <int D, int BS>
hipError_t launch_wide_shape(const DecodeParams& p, hipStream_t stream) {
    constexpr size_t kBuf = (size_t)(D / 8) * kTok * 16 + (size_t)D * kTok * 2;
    const uint64_t units = (uint64_t)p.num_seqs * p.num_kv_heads * p.max_parts;
    const uint64_t n = (units + kXcds - 1) / kXcds * kXcds * (uint64_t)p.col_groups;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_multi_wide_kernel<D, BS>), dim3((unsigned)n), dim3(4 * kWave), 2 * kBuf, stream, p);
    return hipGetLastError();
}

}  // namespace

// Query columns per prefix workgroup (the host sizes col_groups with it),
// and the chunk its partition sizes are whole multiples of.
int decode_prefix_columns() { return 32 * 4; }
int decode_prefix_chunk() { return kTok; }

hipError_t launch_decode_prefix_rest(const DecodeParams& pre, const DecodeParams& rest, hipStream_t stream) {
    if (pre.head_dim == 64)
        return pre.block_size == 16 ? launch_fused_shape<64, 16>(pre, rest, stream)
                                    : launch_fused_shape<64, 32>(pre, rest, stream);
    return pre.block_size == 16 ? launch_fused_shape<128, 16>(pre, rest, stream)
                                : launch_fused_shape<128, 32>(pre, rest, stream);
}

hipError_t launch_decode_multi_wide(const DecodeParams& p, hipStream_t stream) {
    if (p.head_dim == 64)
        return p.block_size == 16 ? launch_wide_shape<64, 16>(p, stream) : launch_wide_shape<64, 32>(p, stream);
    return p.block_size == 16 ? launch_wide_shape<128, 16>(p, stream) : launch_wide_shape<128, 32>(p, stream);
}

hipError_t launch_decode_multi_rest(const DecodeParams& pre, int col_tiles, const DecodeParams& rest,
                                   hipStream_t stream) {
    return col_tiles == 1 ? launch_multi_fused_tiles<1>(pre, rest, stream)
                          : launch_multi_fused_tiles<2>(pre, rest, stream);
}

}  // namespace pa_impl
