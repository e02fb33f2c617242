// Launchers of the multi-query kernel (its body and design are in
// decode_multi_body.h).
#include "decode_multi_body.h"

namespace pa_impl {

namespace {

using namespace multi_detail;

template <int D, int BS, int NT, int POLICY, int WAVES>
__global__ __launch_bounds__(WAVES * kWave)
void decode_multi_kernel(DecodeParams p) {
    extern __shared__ float smem[];
    decode_multi_body<D, BS, NT, POLICY, WAVES>(p, blockIdx.x, smem);
}

template <int D, int BS, int NT, int POLICY, int WAVES>
hipError_t launch_shape(const DecodeParams& p, hipStream_t stream) {
    const size_t smem = sizeof(float) * (2 * WAVES * 16 + (size_t)WAVES * 16 * D);
    const uint64_t nwg = (uint64_t)p.num_seqs * p.num_kv_heads * p.col_groups * p.max_parts;
    hipLaunchKernelGGL((decode_multi_kernel<D, BS, NT, POLICY, WAVES>), dim3((unsigned)nwg), dim3(WAVES * kWave), smem,
                       stream, p);
    return hipGetLastError();
}

template <int NT, int POLICY, int WAVES>
hipError_t launch_tiles(const DecodeParams& p, hipStream_t stream) {
    if (p.head_dim == 64)
        return p.block_size == 16 ? launch_shape<64, 16, NT, POLICY, WAVES>(p, stream)
                                  : launch_shape<64, 32, NT, POLICY, WAVES>(p, stream);
    return p.block_size == 16 ? launch_shape<128, 16, NT, POLICY, WAVES>(p, stream)
                              : launch_shape<128, 32, NT, POLICY, WAVES>(p, stream);
}

}  // namespace

// Streaming loads come in two workgroup sizes (p.waves): 4 waves, or 8 (one
// workgroup fills a compute unit at this kernel's two waves per SIMD) for a
// single pass whose workgroups take the sequences longest first.  Shared-page
// loads always use 4.
hipError_t launch_decode_multi(const DecodeParams& p, int col_tiles, hipStream_t stream) {
    if (p.stream_kv) {
        if (p.waves == 8)
            return col_tiles == 1 ? launch_tiles<1, kPolicyStream, 8>(p, stream)
                                  : launch_tiles<2, kPolicyStream, 8>(p, stream);
        return col_tiles == 1 ? launch_tiles<1, kPolicyStream, 4>(p, stream)
                              : launch_tiles<2, kPolicyStream, 4>(p, stream);
    }
    return col_tiles == 1 ? launch_tiles<1, kPolicyReuse, 4>(p, stream) : launch_tiles<2, kPolicyReuse, 4>(p, stream);
}

}  // namespace pa_impl
