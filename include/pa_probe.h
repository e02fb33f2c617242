/*
 * pa_probe.h -- measurement helper shipped in libpa.so.  Not part of the
 * paged-attention path: it exists so that a benchmark can put the decode
 * kernel's achieved read bandwidth next to what a plain streaming read of
 * the same device reaches (the achievable HBM rate, as opposed to the
 * published peak).
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_probe_stream_read -- read `bytes` bytes at `buf` once with 16-byte
 * vector loads (grid-stride loop, `num_workgroups` workgroups of 256
 * threads; 0 picks 2048) and fold them into a checksum that is stored to
 * `sink` (device, 4 bytes) only when it equals an improbable constant, so
 * the loads cannot be dropped and the write traffic is nil.
 *
 *   buf            device, 16-byte aligned, read
 *   bytes          a multiple of 16
 *   nontemporal    1: loads carry the non-temporal (streaming) bit
 *   sink           device, 4 bytes, normally not written
 * Returns PA_OK (bytes == 0 is a no-op), PA_ERR_NULL, PA_ERR_ARG or
 * PA_ERR_HIP.  Asynchronous on `stream`.
 */
pa_status pa_probe_stream_read(const void* buf, size_t bytes, int32_t nontemporal,
                               int32_t num_workgroups, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
