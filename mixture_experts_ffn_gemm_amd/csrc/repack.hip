// repack.hip -- load-time repacking of the layer weights (not on the timed path).
//
// Q8_0 rows arrive as 34-byte blocks {binary16 scale, int8 q[32]} (the format of
// the Q8_0 MMQ path in SharpInference #406 "References").  34-byte blocks are not
// 16-byte aligned, so the int8 codes are split out into 1 KiB chunks that are
// exactly one 32x32x32 MFMA operand in lane order, and the scales into their own
// binary16 plane.  The repack is lossless: the down planes store each scale
// times a power of two chosen per group so that the product stays a finite
// binary16 (an exact rescaling, undone in the down GEMM's epilogue).
#include <hip/hip_fp16.h>

#include "internal.h"

namespace moe {
namespace {

// One thread per 16-byte piece of a chunk (strip c, block kb, tile tt, lane);
// the half-0 lanes also move the block scale.  Destination per group:
// [strip][k-step][16 chunks of codes + the k-step's scales].  Gate/up form
// (dn_exp == NULL): 1 KiB of scales [tt][32 rows][4 blocks].  Down form: 2 KiB
// of pairs {W, W/2}, W = scale * 2^(23 - dn_exp[g]), [tt][half][32 rows][4].
__global__ __launch_bounds__(256) void repack_q8_kernel(
    const uint8_t* __restrict__ src0, const uint8_t* __restrict__ src1, size_t src_group_bytes,
    int src_rows, int src_blocks, int tiles_per_src, int n_strips, int kb_pad,
    uint8_t* __restrict__ dst, size_t dst_group_bytes, const int32_t* __restrict__ dn_exp) {
  const int g = blockIdx.y;
  const long piece = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long n_pieces = (long)n_strips * kb_pad * 4 * 64;
  if (piece >= n_pieces) return;
  const int lane = (int)(piece % 64);
  const int tt = (int)((piece / 64) % 4);
  const int kb = (int)((piece / 256) % kb_pad);
  const int c = (int)(piece / (256L * kb_pad));
  const int half = lane / 32, r = lane % 32;
  const int row = c * 32 * tiles_per_src + 32 * (tt % tiles_per_src) + r;
  const uint8_t* src = (tt / tiles_per_src) ? src1 : src0;
  const bool valid = row < src_rows && kb < src_blocks;
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  uint16_t scale = 0;
  if (valid) {
    const uint8_t* blk = src + (size_t)g * src_group_bytes + ((size_t)row * src_blocks + kb) * Q8_BYTES;
    const uint8_t* q = blk + 2 + half * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      words[i] = (uint32_t)q[4 * i] | ((uint32_t)q[4 * i + 1] << 8) | ((uint32_t)q[4 * i + 2] << 16) |
                 ((uint32_t)q[4 * i + 3] << 24);
    scale = (uint16_t)(blk[0] | (blk[1] << 8));
  }
  const int step_bytes = dn_exp ? DN_KSTEP_BYTES : KSTEP_BYTES;
  const int n_ks = kb_pad / KSTEP, ks = kb / KSTEP, kbi = kb % KSTEP;
  uint8_t* step = dst + (size_t)g * dst_group_bytes + ((size_t)c * n_ks + ks) * step_bytes;
  *reinterpret_cast<uint4*>(step + (size_t)(kbi * 4 + tt) * 1024 + lane * 16) =
      make_uint4(words[0], words[1], words[2], words[3]);
  if (half != 0) return;
  if (!dn_exp) {
    *reinterpret_cast<uint16_t*>(step + 16 * 1024 + ((tt * 32 + r) * KSTEP + kbi) * 2) = scale;
    return;
  }
  // Power-of-two rescaling of a binary16 value: exact (the exponent keeps W
  // finite; W/2 is exact unless W is subnormal, which needs e >= 13).
  const float wf = ldexpf(__half2float(__ushort_as_half(scale)), 23 - dn_exp[g]);
  const uint32_t pair = (uint32_t)__half_as_ushort(__float2half_rn(wf)) |
                        ((uint32_t)__half_as_ushort(__float2half_rn(0.5f * wf)) << 16);
  *reinterpret_cast<uint32_t*>(step + 16 * 1024 + tt * 512 + (kbi >> 1) * 256 + r * 8 + (kbi & 1) * 4) =
      pair;
}

// One workgroup per group: the largest |scale| of its Q8_0 blocks, then the
// smallest e >= 0 with largest * 2^(23 - e) <= 65504 (the largest binary16).
__global__ __launch_bounds__(256) void scale_exponent_kernel(const uint8_t* __restrict__ src,
                                                             size_t src_group_bytes, long n_blocks,
                                                             int32_t* __restrict__ e_out) {
  __shared__ uint32_t part[256];
  const int g = blockIdx.x;
  const uint8_t* base = src + (size_t)g * src_group_bytes;
  uint32_t m = 0;
  for (long i = threadIdx.x; i < n_blocks; i += blockDim.x) {
    const uint8_t* blk = base + (size_t)i * Q8_BYTES;
    m = max(m, (uint32_t)(blk[0] | (blk[1] << 8)) & 0x7fffu);
  }
  part[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] = max(part[threadIdx.x], part[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float mx = __half2float(__ushort_as_half((uint16_t)min(part[0], 0x7bffu)));
    int e = 0;
    while (e < 23 && ldexpf(mx, 23 - e) > 65504.0f) ++e;
    e_out[g] = e;
  }
}

__global__ __launch_bounds__(256) void transpose_router_kernel(const float* __restrict__ w, int E,
                                                               int d, int E64,
                                                               float* __restrict__ wt) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;  // over (j/4, e, j%4)
  if (i >= (long)d * E64) return;
  const int j4 = (int)(i % 4);
  const int e = (int)((i / 4) % E64);
  const int jq = (int)(i / (4L * E64));
  const int j = jq * 4 + j4;
  wt[i] = (e < E) ? w[(size_t)e * d + j] : 0.0f;
}

}  // namespace

hipError_t launch_repack_q8(const uint8_t* src0, const uint8_t* src1, int n_groups,
                            size_t src_group_bytes, int src_rows, int src_blocks,
                            int tiles_per_src, int n_strips, int kb_pad, uint8_t* dst,
                            size_t dst_group_bytes, const int32_t* dn_exp, hipStream_t s) {
  const long n_pieces = (long)n_strips * kb_pad * 4 * 64;
  dim3 grid((unsigned)((n_pieces + 255) / 256), (unsigned)n_groups);
  repack_q8_kernel<<<grid, 256, 0, s>>>(src0, src1, src_group_bytes, src_rows, src_blocks,
                                        tiles_per_src, n_strips, kb_pad, dst, dst_group_bytes,
                                        dn_exp);
  return hipGetLastError();
}

hipError_t launch_scale_exponent(const uint8_t* src, int n_groups, size_t src_group_bytes,
                                 long n_blocks, int32_t* e, hipStream_t s) {
  scale_exponent_kernel<<<n_groups, 256, 0, s>>>(src, src_group_bytes, n_blocks, e);
  return hipGetLastError();
}

hipError_t launch_transpose_router(const float* w, int E, int d, int E64, float* wt, hipStream_t s) {
  const long n = (long)d * E64;
  transpose_router_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w, E, d, E64, wt);
  return hipGetLastError();
}

}  // namespace moe
