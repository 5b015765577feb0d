// Combine: weighted sum of each token's expert outputs, back in token order.
//
// Operation ("Efficient and portable mixture-of-experts communication",
// Introduction: the layer output is the router-weighted sum of the selected
// experts' outputs; Sharding and Parallelism: the accumulation is folded into
// the gather; Combine: the receiving side applies the routing weights and
// writes an externally allocated tensor).
//
// One wave per token, four tokens per workgroup.  The row maps and weights of
// the token are read into lanes 0..K-1 and broadcast with readlane (scalar
// registers).  Each lane owns 16-byte pieces of the output row; for each piece
// it issues the K gathers, accumulates w_k * y in fp32 in ascending k, adds
// the shared-expert rows, and rounds once.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // bf16: 8 per 16 bytes
  static constexpr int N = 8;
  __device__ static void load(const u32x4& v, float (&f)[8]) {
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static u32x4 store(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_bits(f[2 * i]) | ((uint32_t)f32_to_bf16_bits(f[2 * i + 1]) << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
  }
};
template <>
struct Vec<float> {  // fp32: 4 per 16 bytes
  static constexpr int N = 4;
  __device__ static void load(const u32x4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v[0]); f[1] = __uint_as_float(v[1]);
    f[2] = __uint_as_float(v[2]); f[3] = __uint_as_float(v[3]);
  }
  __device__ static u32x4 store(const float (&f)[4]) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};

constexpr int kPieces = 2;  // 16-byte pieces per lane per iteration

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(
    const u32x4* __restrict__ y_sorted, const int32_t* __restrict__ row_of,
    const float* __restrict__ weights, const u32x4* __restrict__ y_shared, int num_tokens, int K,
    int n_shared, int row_vecs, u32x4* __restrict__ out) {
  constexpr int N = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  int myrow = -1;
  float myw = 0.f;
  if (lane < K) {
    myrow = row_of[(size_t)t * K + lane];
    myw = weights[(size_t)t * K + lane];
  }
  for (int v0 = 0; v0 < row_vecs; v0 += kWave * kPieces) {
    float acc[kPieces][N];
#pragma unroll
    for (int p = 0; p < kPieces; ++p)
#pragma unroll
      for (int i = 0; i < N; ++i) acc[p][i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int rk = __builtin_amdgcn_readlane(myrow, k);
      if (rk < 0) continue;
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myw), k));
      const u32x4* src = y_sorted + (size_t)rk * row_vecs;
#pragma unroll
      for (int p = 0; p < kPieces; ++p) {
        const int v = v0 + p * kWave + lane;
        if (v < row_vecs) {
          float f[N];
          Vec<T>::load(src[v], f);
#pragma unroll
          for (int i = 0; i < N; ++i) acc[p][i] = fmaf(wk, f[i], acc[p][i]);
        }
      }
    }
    for (int s = 0; s < n_shared; ++s) {
      const u32x4* src = y_shared + ((size_t)s * num_tokens + t) * row_vecs;
#pragma unroll
      for (int p = 0; p < kPieces; ++p) {
        const int v = v0 + p * kWave + lane;
        if (v < row_vecs) {
          float f[N];
          Vec<T>::load(src[v], f);
#pragma unroll
          for (int i = 0; i < N; ++i) acc[p][i] += f[i];
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int v = v0 + p * kWave + lane;
      if (v < row_vecs) out[(size_t)t * row_vecs + v] = Vec<T>::store(acc[p]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const moe_config_t& c, const void* y_sorted, const int32_t* row_of,
                          const float* weights, const void* y_shared, void* out, hipStream_t s) {
  const int elem = c.dtype == MOE_BF16 ? 2 : 4;
  const int row_vecs = c.hidden * elem / 16;
  const dim3 grid(ceil_div(c.num_tokens, 4)), block(256);
  const int n_sh = y_shared ? c.num_shared : 0;
  if (c.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const u32x4*>(y_sorted), row_of, weights,
                       static_cast<const u32x4*>(y_shared), c.num_tokens, c.top_k, n_sh, row_vecs,
                       static_cast<u32x4*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s,
                       static_cast<const u32x4*>(y_sorted), row_of, weights,
                       static_cast<const u32x4*>(y_shared), c.num_tokens, c.top_k, n_sh, row_vecs,
                       static_cast<u32x4*>(out));
  return hipGetLastError();
}

}  // namespace moe
