// probe.hip -- calibration kernels of libmoe_probe.so: the measured int8
// matrix-core rate and HBM streaming rate that the layer's kernels are priced
// against next to the datasheet peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Four independent accumulators per wavefront, so that consecutive MFMAs never
// wait for one another's results; the operands are registers that differ per
// lane (never constant-folded).
__global__ __launch_bounds__(256) void int8_mfma_loop(int iters, int32_t* __restrict__ sink) {
  const int t = threadIdx.x;
  const v4i a = {t, t * 3 + 1, t * 5 + 2, t * 7 + 3};
  const v4i b = {t * 11 + 4, t * 13 + 5, t ^ 0x5a5a5a5a, t + 0x01010101};
  v16i c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] ^ c1[v] ^ c2[v] ^ c3[v];
  sink[(size_t)blockIdx.x * 256 + t] = s;
}

// Four 16-byte loads in flight per thread before their stores.
__global__ __launch_bounds__(256) void copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int moe_probe_int8_mfma(int32_t iters, int32_t n_workgroups, int32_t* sink, hipStream_t stream) {
  if (iters < 1 || iters > (1 << 24) || n_workgroups < 1 || n_workgroups > (1 << 20) || !sink) return -1;
  int8_mfma_loop<<<n_workgroups, 256, 0, stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int moe_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst || (bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return -1;
  const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
  if (bytes && s < d + bytes && d < s + bytes) return -1;
  if (bytes == 0) return 0;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0) {
    (void)hipGetLastError();
    return -5;
  }
  copy16<<<n_cu * 16, 256, 0, stream>>>((const uint4*)src, (uint4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
