/*
 * moe_probe.h -- achievable-peak probes of the GPU the MoE layer runs on.
 *
 * Not part of the layer's computation: the benchmark runs these beside the
 * layer and reports what they reach next to the nominal MI355X peaks, so the
 * layer's kernels can be read against both the published and the measured
 * ceilings (plain streaming bandwidth of HBM; the MFMA pipes fed from
 * registers only).  Same conventions as moe.h: device pointers, asynchronous
 * launches on `stream`, host validation first (nothing enqueued on error).
 */
#ifndef MOE_PROBE_H_
#define MOE_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_probe_stream -- one pass over `bytes` bytes (a multiple of 16) with
 * 16-byte accesses by `workgroups` workgroups of 256 threads, each taking
 * every workgroups-th contiguous block of 16 KB (kind 2) or 32 KB (kinds 0, 1)
 * in turn, loads non-temporal:
 *   kind 0: copy src -> dst (reads and writes `bytes` each);
 *   kind 1: read src (sink [workgroups * 256] uint32 receives one word per
 *           thread so the loads stay live; dst unused, may be NULL);
 *   kind 2: write a pattern to dst (src unused, may be NULL).
 * dst and src 16-byte aligned.  MOE_ERR_INVALID_ARGUMENT on a bad kind,
 * size or pointer; MOE_ERR_UNSUPPORTED if the grid reaches 2^32 work-items.
 */
moe_status_t moe_probe_stream(int32_t kind, void* dst, const void* src, size_t bytes,
                              uint32_t* sink, int32_t workgroups, moe_stream_t stream);

/*
 * moe_probe_mfma -- `workgroups` workgroups of 8 waves (two per SIMD), each
 * wave issuing `iters` rounds of 8 independent register-only MFMAs:
 *   kind 0: v_mfma_f32_32x32x16_bf16;
 *   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit scales).
 * out [workgroups * 512] fp32 receives one sum per lane.  The flops of the
 * launch are moe_probe_mfma_flops(kind, workgroups, iters).
 */
moe_status_t moe_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, float* out,
                            moe_stream_t stream);
double moe_probe_mfma_flops(int32_t kind, int32_t workgroups, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H_ */
