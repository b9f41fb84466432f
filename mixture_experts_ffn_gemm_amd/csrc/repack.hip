// repack.hip -- load-time repacking of the layer weights (not on the timed path).
// Q8_0, Q4_K and Q3_K expert rows; the router matrix transposed.
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

// Q4_K (the k-quant format beside Q8_0 in SharpInference #406 "References"):
// a row is a run of 144-byte super-blocks of 256 weights {binary16 d,
// binary16 dmin, 12 bytes of packed 6-bit sub-block scales and mins, 128
// bytes of 4-bit codes}; weight i of sub-block j (32 weights) is
// d * sc_j * q_i - dmin * m_j.  Sub-blocks 0-3 keep their scale and min in
// the low 6 bits of bytes j and j + 4 of the 12; sub-blocks 4-7 take the low
// (scale) or high (min) nibble of byte j + 4 as their low 4 bits and the top
// 2 bits of byte j - 4 (scale) or byte j (min) as their high 2 bits.  Code i
// of sub-block j is the low (j even) or high (j odd) nibble of code byte
// 32 * (j / 2) + i.
__device__ inline void q4k_scale_min(const uint8_t* s12, int j, int& sc, int& m) {
  if (j < 4) {
    sc = s12[j] & 63;
    m = s12[j + 4] & 63;
  } else {
    sc = (s12[j + 4] & 15) | ((s12[j - 4] >> 6) << 4);
    m = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
  }
}

// v as the binary16 pair {hi, lo}: hi = v rounded to binary16, lo = the
// remainder v - hi (exact in fp32) rounded to binary16.  A product d * sc or
// dmin * m has at most 17 significant bits, so hi + lo == v exactly unless
// the remainder lies below the binary16 normal range, where its error stays
// below 2^-25.  Sets bad when a finite v overflows binary16.
__device__ inline void split_half(float v, uint16_t& hi, uint16_t& lo, bool& bad) {
  const __half h = __float2half_rn(v);
  const float hf = __half2float(h);
  if (isfinite(v) && !isfinite(hf)) bad = true;
  hi = __half_as_ushort(h);
  lo = __half_as_ushort(__float2half_rn(v - hf));
}

// One thread per (strip c, k-step ks, tile tt, lane) of group blockIdx.y: its
// 8-byte code piece of each of the k-step's 4 blocks, and its 8 bytes of the
// D and M pair planes (layout in gemm_q4k.hip).
__global__ __launch_bounds__(256) void repack_q4k_kernel(
    const uint8_t* __restrict__ src0, const uint8_t* __restrict__ src1, size_t src_group_bytes,
    int src_rows, int src_supers, int tiles_per_src, int n_strips, int n_ks, uint8_t* __restrict__ dst,
    size_t dst_group_bytes, int32_t* __restrict__ overflow) {
  const int g = blockIdx.y;
  const long piece = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long n_pieces = (long)n_strips * n_ks * 4 * 64;
  if (piece >= n_pieces) return;
  const int lane = (int)(piece % 64);
  const int tt = (int)((piece / 64) % 4);
  const int ks = (int)((piece / 256) % n_ks);
  const int c = (int)(piece / (256L * n_ks));
  const int half = lane / 32, r = lane % 32;
  const int row = c * 32 * tiles_per_src + 32 * (tt % tiles_per_src) + r;
  const uint8_t* src = (tt / tiles_per_src) ? src1 : src0;
  const int sb = ks / 2, j0 = 4 * (ks % 2);  // super-block and its first sub-block in this k-step
  const bool valid = row < src_rows && sb < src_supers;
  uint8_t* step = dst + (size_t)g * dst_group_bytes + ((size_t)c * n_ks + ks) * Q4K_KSTEP_BYTES;
  uint16_t dpl[4] = {0, 0, 0, 0}, mpl[4] = {0, 0, 0, 0};
  bool bad = false;
  const uint8_t* blk = valid ? src + (size_t)g * src_group_bytes + ((size_t)row * src_supers + sb) * Q4K_BYTES
                             : nullptr;
  const float d = valid ? __half2float(__ushort_as_half((uint16_t)(blk[0] | (blk[1] << 8)))) : 0.0f;
  const float dmin = valid ? __half2float(__ushort_as_half((uint16_t)(blk[2] | (blk[3] << 8)))) : 0.0f;
#pragma unroll
  for (int kbi = 0; kbi < 4; ++kbi) {
    uint32_t X = 0u, Y = 0u;
    if (valid) {
      const int j = j0 + kbi;
      const uint8_t* qb = blk + 16 + 32 * (j / 2) + 16 * half;
      const int sh = (j & 1) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q0 = (qb[i] >> sh) & 15u, q4 = (qb[i + 4] >> sh) & 15u;
        const uint32_t q8 = (qb[i + 8] >> sh) & 15u, q12 = (qb[i + 12] >> sh) & 15u;
        X |= (q0 | (q4 << 4)) << (8 * i);
        Y |= (q8 | (q12 << 4)) << (8 * i);
      }
      int sc, m;
      q4k_scale_min(blk + 4, j, sc, m);
      uint16_t hi, lo;
      split_half(d * (float)sc, hi, lo, bad);  // exact in fp32: 11 + 6 significant bits
      dpl[kbi] = half ? lo : hi;
      split_half(dmin * (float)m, hi, lo, bad);
      if ((kbi >> 1) == half) {
        mpl[2 * (kbi & 1)] = hi;
        mpl[2 * (kbi & 1) + 1] = lo;
      }
    }
    *reinterpret_cast<uint2*>(step + (kbi * 4 + tt) * 512 + lane * 8) = make_uint2(X, Y);
  }
  *reinterpret_cast<uint2*>(step + 8 * 1024 + tt * 512 + lane * 8) =
      make_uint2(dpl[0] | ((uint32_t)dpl[1] << 16), dpl[2] | ((uint32_t)dpl[3] << 16));
  *reinterpret_cast<uint2*>(step + 10 * 1024 + tt * 512 + lane * 8) =
      make_uint2(mpl[0] | ((uint32_t)mpl[1] << 16), mpl[2] | ((uint32_t)mpl[3] << 16));
  if (bad) *overflow = 1;
}

// Q3_K (the format of the Q3_K expert GEMM of SharpInference #388 "Key
// references"): a row is a run of 110-byte super-blocks of 256 weights {32
// bytes of high bits, 64 bytes of 2-bit codes, 12 bytes of 6-bit sub-block
// scales, binary16 d}.  Weight 128h + 32g + l takes its 2-bit code from bits
// 2g of code byte 32h + l and its high bit from bit 4h + g of high-bit byte
// l; q = code, minus 4 when the high bit is clear (q in -4..3).  It lies in
// 16-weight sub-block s = 8h + 2g + l/16, whose scale sc_s has nibble s/8
// (low first) of scale byte s%8 as its low 4 bits and bits 2(s/4), 2(s/4)+1
// of scale byte 8 + s%4 as its high 2; the weight is d * (sc_s - 32) * q.
//
// The products (sc_s - 32) * q lie in [-124, 128], so their negations fit
// int8, and a Q3_K 32-block is exactly the Q8_0 block {scale -d, codes
// -(sc_s - 32) * q}: one thread per output block writes that 34-byte block.
// The Q8_0 planes built from these rows then give every GEMM and matvec the
// exact Q3_K products.  (|code sum| <= 32 * 127 * 128 < 2^19, the bound the
// down pipeline's exact form needs.)
__global__ __launch_bounds__(256) void q3k_to_q8_kernel(const uint8_t* __restrict__ src, size_t src_group_bytes,
                                                        int rows, int supers, uint8_t* __restrict__ dst,
                                                        size_t dst_group_bytes) {
  const int g = blockIdx.y;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long n = (long)rows * supers * 8;
  if (idx >= n) return;
  const long row = idx / (supers * 8);
  const int b = (int)(idx % (supers * 8));
  const uint8_t* blk = src + (size_t)g * src_group_bytes + ((size_t)row * supers + b / 8) * Q3K_BYTES;
  uint8_t* out = dst + (size_t)g * dst_group_bytes + (size_t)idx * Q8_BYTES;
  const int h = (b % 8) / 4, gq = (b % 8) % 4;
  int mult[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int s = 8 * h + 2 * gq + u;
    const int lo4 = (blk[96 + s % 8] >> (4 * (s / 8))) & 15;
    const int hi2 = (blk[104 + s % 4] >> (2 * (s / 4))) & 3;
    mult[u] = (lo4 | (hi2 << 4)) - 32;
  }
  const uint16_t dbits = (uint16_t)(blk[108] | (blk[109] << 8)) ^ 0x8000u;  // -d
  out[0] = (uint8_t)(dbits & 0xff);
  out[1] = (uint8_t)(dbits >> 8);
#pragma unroll 4
  for (int t = 0; t < 32; ++t) {
    const int code = (blk[32 + 32 * h + t] >> (2 * gq)) & 3;
    const int high = (blk[t] >> (4 * h + gq)) & 1;
    const int q = high ? code : code - 4;
    out[2 + t] = (uint8_t)(int8_t)(-mult[t / 16] * q);
  }
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

hipError_t launch_repack_q4k(const uint8_t* src0, const uint8_t* src1, int n_groups, size_t src_group_bytes,
                             int src_rows, int src_supers, int tiles_per_src, int n_strips, int n_ksteps,
                             uint8_t* dst, size_t dst_group_bytes, int32_t* overflow, hipStream_t s) {
  const long n_pieces = (long)n_strips * n_ksteps * 4 * 64;
  dim3 grid((unsigned)((n_pieces + 255) / 256), (unsigned)n_groups);
  repack_q4k_kernel<<<grid, 256, 0, s>>>(src0, src1, src_group_bytes, src_rows, src_supers, tiles_per_src,
                                         n_strips, n_ksteps, dst, dst_group_bytes, overflow);
  return hipGetLastError();
}

hipError_t launch_q3k_to_q8(const uint8_t* src, int n_groups, size_t src_group_bytes, int rows, int supers,
                            uint8_t* dst, size_t dst_group_bytes, hipStream_t s) {
  const long n = (long)rows * supers * 8;
  dim3 grid((unsigned)((n + 255) / 256), (unsigned)n_groups);
  q3k_to_q8_kernel<<<grid, 256, 0, s>>>(src, src_group_bytes, rows, supers, dst, dst_group_bytes);
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
