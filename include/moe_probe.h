/*
 * moe_probe.h -- C ABI of libmoe_probe.so: two calibration kernels that
 * measure, on the GPU at hand, the two roofs the MoE FFN kernels are priced
 * against (the per-stage measurement discipline of SharpInference #388,
 * "Measurement discipline": measure each phase against a warm, isolated
 * reference rather than a nominal figure).  They compute nothing of the
 * method; the benchmark times them with HIP events next to the layer.
 *
 * Both return 0 on success, -1 for an invalid argument (nothing enqueued) and
 * -5 when the launch fails.  Work is enqueued on `stream` without a host
 * synchronisation.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense int8 matrix-core issue rate: n_workgroups workgroups of 4
 * wavefronts, each wavefront issuing `iters` rounds of four independent
 * v_mfma_i32_32x32x32_i8 (65536 int8 ops each, operands in registers, no
 * memory traffic inside the loop).  Total ops = n_workgroups * 4 * iters * 4
 * * 65536.  sink: device int32 [n_workgroups * 256], receives a value derived
 * from every accumulator so that no MFMA is dead code.  1 <= iters <= 2^24,
 * 1 <= n_workgroups <= 2^20. */
int moe_probe_int8_mfma(int32_t iters, int32_t n_workgroups, int32_t* sink, hipStream_t stream);

/* HBM streaming rate: dst[i] = src[i] for `bytes` bytes (both device
 * pointers, 16-byte aligned, bytes a multiple of 16, not overlapping) with
 * 16-byte loads and stores in a grid-stride loop; moves 2 * bytes. */
int moe_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H */
