/* Reference rates measured on the device for roofline fractions (not part of the attention path).
 *
 * The attention kernels' achieved rates are reported against the vendor peaks and against what
 * the same GPU reaches on the simplest kernel of each kind; these two entry points are those
 * kernels.  Both enqueue one launch on `stream` and return at once; time them with events on the
 * same stream.  Status codes and dca_last_error() as in dca.h.
 */
#ifndef DCA_CALIBRATE_H
#define DCA_CALIBRATE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "dca.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix cores only: n_workgroups workgroups of 4 waves; each wave issues iters x 32
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on four independent accumulators, with no memory
 * traffic.  FLOP = n_workgroups * 4 * iters * 32 * 32768.
 * sink: device fp32 [n_workgroups * 256], written (keeps the work alive).
 * 1 <= n_workgroups <= 65536, 1 <= iters <= 1 << 20; else DCA_ERR_INVALID_ARGUMENT. */
dca_status dca_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float* sink, hipStream_t stream);

/* Streaming read of `bytes` at src with 16-byte nontemporal loads (grid-stride, 8 loads in flight
 * per thread);
 * every byte is read once.  src is device memory, or pinned host memory read in place over the host
 * link (pageable host memory: DCA_ERR_INVALID_ARGUMENT).  bytes >= 0 and a multiple of 16, src 16-byte
 * aligned; sink: device fp32 [n_workgroups * 256], written.  1 <= n_workgroups <= 65536. */
dca_status dca_probe_hbm_read(const void* src, int64_t bytes, int32_t n_workgroups, float* sink,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DCA_CALIBRATE_H */
