// Router: projection to per-expert logits, score function and top-K selection.
//
// Operation ("Efficient and portable mixture-of-experts communication",
// Introduction): a small linear layer gives each token a distribution over
// the experts; the K best-scoring experts are kept, weighted by values
// derived from that distribution.  Softmax and sigmoid are both increasing in
// the logit, so the K experts are chosen on the logits directly; equal logits
// go to the lower expert id; slots come out in descending order.
//
// bf16: one workgroup = 16 tokens x all experts.  The four waves split the
// reduction dimension (wave w takes 32-wide slices w, w+4, ...), each running
// 16x16x32 bf16 MFMAs into fp32 accumulators held for all expert tiles; the
// four partial sums are then added in LDS in fixed wave order (deterministic).
// fp32: each wave takes 4 tokens and reduces every dot product across its 64
// lanes with a butterfly.
// Selection: one wave per token, E/64 candidates per lane in registers, K
// rounds of a butterfly arg-max ordered by (logit desc, expert id asc).
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokTile = 16;

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Butterfly sum: every lane ends with the same bits (fp addition is commutative).
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// v[i] holds the logit of expert lane + 64*i (bias included), -inf past E.
template <int NV>
__device__ __forceinline__ void select_topk(float (&v)[NV], int E, int K, int score, int renorm,
                                            int t, int32_t* __restrict__ ids,
                                            float* __restrict__ weights,
                                            float* __restrict__ logits, int lane) {
  if (logits) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + kWave * i;
      if (e < E) logits[(size_t)t * E + e] = v[i];
    }
  }
  float m = 0.f, denom = 1.f;
  if (score == MOE_SCORE_SOFTMAX) {
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) lm = fmaxf(lm, v[i]);
    m = wave_max(lm);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + kWave * i < E) s += __expf(v[i] - m);
    denom = wave_sum(s);
  }
  int my_e = 0;
  float my_s = 0.f, sum_sel = 0.f;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (v[i] > bv) { bv = v[i]; be = lane + kWave * i; }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if ((be & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i == (be >> 6)) v[i] = -INFINITY;
    }
    const float sc = score == MOE_SCORE_SIGMOID ? 1.f / (1.f + __expf(-bv)) : __expf(bv - m);
    sum_sel += sc;
    if (lane == k) { my_e = be; my_s = sc; }
  }
  if (lane < K) {
    float w;
    if (renorm) w = my_s / sum_sel;
    else if (score == MOE_SCORE_SOFTMAX) w = my_s / denom;
    else w = my_s;
    ids[(size_t)t * K + lane] = my_e;
    weights[(size_t)t * K + lane] = w;
  }
}

template <int NT>
__global__ __launch_bounds__(256) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, int K, int score, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ weights, float* __restrict__ logits) {
  constexpr int EP = NT * 16;
  constexpr int NV = EP >= kWave ? EP / kWave : 1;
  __shared__ float zs[kTokTile][EP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kTokTile;
  const int arow = min(t0 + (lane & 15), T - 1);
  const int koff = (lane >> 4) * 8;
  const uint16_t* ap = x + (size_t)arow * d + koff;

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* bp[NT];
  bool bok[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int e = j * 16 + (lane & 15);
    bok[j] = e < E;
    bp[j] = wr + (size_t)(bok[j] ? e : 0) * d + koff;
  }
  const int n_kc = d / 32;
  for (int kc = wave; kc < n_kc; kc += 4) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + kc * 32);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      bf16x8 b = *reinterpret_cast<const bf16x8*>(bp[j] + kc * 32);
      if (!bok[j]) b = bf16x8{};
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
  }
  // Fixed-order sum of the four waves' partial logits: ((w0 + w1) + w2) + w3.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = (lane >> 4) * 4 + i, e = j * 16 + (lane & 15);
          zs[tok][e] = (w == 0) ? acc[j][i] : zs[tok][e] + acc[j][i];
        }
    }
    __syncthreads();
  }
  for (int tt = wave * 4; tt < wave * 4 + 4; ++tt) {
    const int t = t0 + tt;
    if (t >= T) break;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + kWave * i;
      v[i] = e < E ? zs[tt][e] + (bias ? bias[e] : 0.f) : -INFINITY;
    }
    select_topk<NV>(v, E, K, score, renorm, t, ids, weights, logits, lane);
  }
}

template <int NV>
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int K, int score, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ weights, float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int tt = wave * 4; tt < wave * 4 + 4; ++tt) {
    const int t = blockIdx.x * kTokTile + tt;
    if (t >= T) break;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = -INFINITY;
    const float* xr = x + (size_t)t * d;
    for (int e = 0; e < E; ++e) {
      const float* wrow = wr + (size_t)e * d;
      float p = 0.f;
      for (int i = lane; i < d; i += kWave) p = fmaf(xr[i], wrow[i], p);
      p = wave_sum(p);
      if (bias) p += bias[e];
      if ((e & (kWave - 1)) == lane) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (i == (e >> 6)) v[i] = p;
      }
    }
    select_topk<NV>(v, E, K, score, renorm, t, ids, weights, logits, lane);
  }
}

template <int NT>
hipError_t launch_bf16(const moe_config_t& c, const void* x, const void* wr, const float* bias,
                       int32_t* ids, float* w, float* logits, hipStream_t s) {
  const dim3 grid(ceil_div(c.num_tokens, kTokTile)), block(256);
  hipLaunchKernelGGL(route_bf16_kernel<NT>, grid, block, 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr), bias,
                     c.num_tokens, c.hidden, c.num_experts, c.top_k, c.score, c.renormalize, ids,
                     w, logits);
  return hipGetLastError();
}

template <int NV>
hipError_t launch_f32(const moe_config_t& c, const void* x, const void* wr, const float* bias,
                      int32_t* ids, float* w, float* logits, hipStream_t s) {
  const dim3 grid(ceil_div(c.num_tokens, kTokTile)), block(256);
  hipLaunchKernelGGL(route_f32_kernel<NV>, grid, block, 0, s, static_cast<const float*>(x),
                     static_cast<const float*>(wr), bias, c.num_tokens, c.hidden, c.num_experts,
                     c.top_k, c.score, c.renormalize, ids, w, logits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_config_t& c, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* weights, float* logits,
                        hipStream_t s) {
  if (c.dtype == MOE_BF16) {
    const int nt = ceil_div(c.num_experts, 16);
    if (nt <= 1) return launch_bf16<1>(c, x, w_router, bias, ids, weights, logits, s);
    if (nt <= 2) return launch_bf16<2>(c, x, w_router, bias, ids, weights, logits, s);
    if (nt <= 4) return launch_bf16<4>(c, x, w_router, bias, ids, weights, logits, s);
    if (nt <= 8) return launch_bf16<8>(c, x, w_router, bias, ids, weights, logits, s);
    if (nt <= 16) return launch_bf16<16>(c, x, w_router, bias, ids, weights, logits, s);
    return launch_bf16<32>(c, x, w_router, bias, ids, weights, logits, s);
  }
  const int nv = ceil_div(c.num_experts, kWave);
  if (nv <= 1) return launch_f32<1>(c, x, w_router, bias, ids, weights, logits, s);
  if (nv <= 2) return launch_f32<2>(c, x, w_router, bias, ids, weights, logits, s);
  if (nv <= 4) return launch_f32<4>(c, x, w_router, bias, ids, weights, logits, s);
  return launch_f32<8>(c, x, w_router, bias, ids, weights, logits, s);
}

}  // namespace moe
