// Launchers of the paged decode kernel on the MFMA matrix cores (the
// kernel body and its design are in decode_mfma_body.h).
#include "decode_mfma_body.h"

namespace pa_impl {

namespace {

using namespace mfma_detail;

// (5-wave workgroups are held to three waves per SIMD, so two of them fit on
// one compute unit: 3 + 3 + 2 + 2 waves over its four SIMDs)
template <int D, int BS, bool SPLIT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave, WAVES == kPairWaves ? 3 : 1)
void decode_mfma_kernel(DecodeParams p) {
    extern __shared__ float smem[];
    decode_mfma_body<D, BS, SPLIT, WAVES>(p, blockIdx.x, smem);
}

template <int D, int BS, bool SPLIT, int WAVES>
hipError_t launch_shape(const DecodeParams& p, hipStream_t stream) {
    const size_t smem = sizeof(float) * (2 * WAVES * 16 + (size_t)WAVES * p.group * D);
    const uint64_t nwg = (uint64_t)p.num_seqs * p.num_kv_heads * (p.max_parts - (SPLIT ? 0 : p.first_part));
    if (nwg == 0) return hipSuccess;                          // every position lies in the prefix
    hipLaunchKernelGGL((decode_mfma_kernel<D, BS, SPLIT, WAVES>), dim3((unsigned)nwg), dim3(WAVES * kWave), smem,
                       stream, p);
    return hipGetLastError();
}

template <bool SPLIT, int WAVES>
hipError_t launch_path(const DecodeParams& p, hipStream_t stream) {
    if (p.head_dim == 64)
        return p.block_size == 16 ? launch_shape<64, 16, SPLIT, WAVES>(p, stream)
                                  : launch_shape<64, 32, SPLIT, WAVES>(p, stream);
    return p.block_size == 16 ? launch_shape<128, 16, SPLIT, WAVES>(p, stream)
                              : launch_shape<128, 32, SPLIT, WAVES>(p, stream);
}

}  // namespace

// Streaming loads come in three workgroup sizes: 4 waves (several
// workgroups share a compute unit, so one's set-up and merge overlap the
// others' streaming), 12 waves (one workgroup fills a compute unit, three
// times the bytes in flight for one (sequence, kv head, partition), which
// drains long and ragged work units faster) and 5 waves (for a
// longest-first single pass).  Shared-page loads always use 4.
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
    if (!p.stream_kv) return launch_path<false, 4>(p, stream);
    if (p.waves == kPairWaves) return launch_path<true, kPairWaves>(p, stream);
    return p.waves == kWideWaves ? launch_path<true, kWideWaves>(p, stream) : launch_path<true, 4>(p, stream);
}

}  // namespace pa_impl
