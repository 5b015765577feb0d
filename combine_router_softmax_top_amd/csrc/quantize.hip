// MX-FP8 block quantization of the rows of a matrix.
//
// Operation ("Efficient and portable mixture-of-experts communication",
// Dispatch: the token payload travels with block scaling factors; the page
// fixes no format).  Format: OCP MX-FP8, the one gfx950's scaled MFMA reads --
// every 32 consecutive elements of a row share a power-of-two scale 2^s,
// stored as the byte s + 127, with s = floor(log2 max|x|) - 8 kept within
// [-127, 127] (so the block's largest element lands in [256, 512)); each
// element is x / 2^s clamped to +-448 and rounded to the nearest E4M3 value,
// ties to even.
//
// Scale layouts: MOE_MX_ROWS keeps row r's scales at r * cols/32 + block;
// MOE_MX_MFMA arranges them for the scaled-MFMA grouped GEMM, which reads, per
// lane, one dword for two 128-deep k-tiles: block 16g + m of row r (m = 8d +
// 4j + 2s + h) is byte 2j + s of dword ((2g + d) R + r) 2 + h, R = rows.
//
// One lane per 8 consecutive elements, four lanes per block: the block maximum
// is shared with two xor shuffles; floor(log2 max) is the maximum's exponent
// field (a zero or subnormal maximum gives the clamped -127); x * 2^-s is exact
// in fp32 wherever the rounding to E4M3 can see the difference; the hardware
// conversion rounds to nearest even and does not saturate, hence the clamp.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}


template <typename T>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const T* __restrict__ in,
                                                             long long ld, int rows, int cols,
                                                             int layout,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int per_row = cols / 8;  // pieces of 8 elements
  const long long n = (long long)rows * per_row;
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  // Whole blocks of four lanes stay together (per_row is a multiple of 4), so
  // a piece past the end belongs to a block that is past the end entirely.
  const bool live = p < n;
  const long long pc = live ? p : n - 1;
  const int r = (int)(pc / per_row), c8 = (int)(pc % per_row);
  float v[8];
  load8<T>(in + (long long)r * ld + (long long)c8 * 8, v);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  const int ef = (int)((__float_as_uint(m) >> 23) & 0xff);  // 0 for zero and subnormals
  const int s = min(127, max(-127, ef - 127 - 8));
  const float inv = __uint_as_float((uint32_t)(127 - s) << 23);  // 2^-s, s <= 120 here
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = fminf(448.f, fmaxf(-448.f, v[i] * inv));
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  if (!live) return;
  *reinterpret_cast<u32x2*>(codes + (long long)r * cols + (long long)c8 * 8) =
      u32x2{(uint32_t)lo, (uint32_t)hi};
  if ((c8 & 3) == 0) {
    const int q = c8 / 4;
    long long at;
    if (layout == MOE_MX_ROWS) {
      at = (long long)r * (cols / 32) + q;
    } else {
      const int g = q >> 4, m = q & 15;
      const int d = m >> 3, b = ((m >> 2) & 1) * 2 + ((m >> 1) & 1), hh = m & 1;
      at = (((long long)(2 * g + d) * rows + r) * 2 + hh) * 4 + b;
    }
    scales[at] = (uint8_t)(s + 127);
  }
}

}  // namespace

hipError_t launch_mxfp8_quantize(int rows, int cols, int dtype, const void* in, long long ld,
                                 int layout, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const long long pieces = (long long)rows * (cols / 8);
  const dim3 grid((unsigned)((pieces + 255) / 256));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(mxfp8_quantize_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), ld, rows, cols, layout, codes, scales);
  else
    hipLaunchKernelGGL(mxfp8_quantize_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(in), ld, rows, cols, layout, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
