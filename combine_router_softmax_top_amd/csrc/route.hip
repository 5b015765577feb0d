// Router: projection to per-expert logits, score function and top-K selection.
//
// Operation ("Efficient and portable mixture-of-experts communication",
// Introduction): a small linear layer gives each token a distribution over
// the experts; the K best-scoring experts are kept, weighted by values
// derived from that distribution.  Softmax and sigmoid are both increasing in
// the logit, so the K experts are chosen on the logits directly; equal logits
// go to the lower expert id; slots come out in descending order.
//
// bf16: a logits GEMM (16x16x32 bf16 MFMA, fp32 accumulation) over tiles of
// 64 tokens x up to 256 experts x one slice of the reduction dimension, then
// a selection kernel that adds the slices in a fixed order (deterministic).
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

// ---- bf16: logits GEMM with a fixed k-split, then selection ----
//
// route_logits_kernel<NT>: workgroup = 64 tokens x NT*16 experts x one slice
// of the reduction dimension.  Each of its 4 waves owns 16 tokens and all
// NT*16 experts (NT blocks of 16x16x32 MFMA).  Router rows are staged in
// 64-wide k-chunks through LDS (double-buffered, shared by the 4 waves);
// token fragments come straight from global memory.  Partial logits of slice
// s go to part[s][t][e] (fp32) and the select kernel adds the slices in
// ascending s.  The number of slices depends only on d and E, never on the
// token count, so a token's logits do not depend on how the batch is split.
constexpr int kRtTok = 64, kRtKc = 64;

// LDS rows of 128 B (64 bf16): logical 16-byte chunk c of row r sits in slot
// c ^ rsw(r); 16 lanes reading rows r..r+15 at one logical chunk then touch
// distinct slots in every 256-byte window (no bank conflicts).
__device__ __forceinline__ int rsw(int r) { return (r ^ (r >> 3)) & 7; }

template <int NT>
__global__ __launch_bounds__(256) void route_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    int e_pad, int k_slice, float* __restrict__ part) {
  constexpr int NE = NT * 16;
  constexpr int kStage = NE * 128;
  constexpr int kPer = (NE * 8 + 255) / 256;  // 16-byte staging chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t wt[2 * kStage];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kRtTok + wave * 16;
  const int e0 = blockIdx.y * NE;
  const int k0 = blockIdx.z * k_slice;
  const int kgrp = lane >> 4;
  const uint16_t* ap = x + (size_t)min(t0 + (lane & 15), T - 1) * d + k0 + kgrp * 8;

  // staging chunk q = tid + 256 i: router row q/8, 16-byte chunk q%8.  When
  // the stage has fewer than 256 chunks, the surplus threads copy an existing
  // chunk again (same bytes to the same place), which keeps the body free of
  // branches.
  const uint16_t* src[kPer];
  int dst[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = (tid + 256 * i) % (NE * 8);
    const int row = q >> 3, c = q & 7;
    const int e = min(e0 + row, E - 1);
    src[i] = wr + (size_t)e * d + k0 + c * 8;
    dst[i] = row * 128 + ((c ^ rsw(row)) << 4);
  }
  u32x4 stg[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) stg[i] = *reinterpret_cast<const u32x4*>(src[i]);
#pragma unroll
  for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4*>(wt + dst[i]) = stg[i];
  __syncthreads();

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int boff[NT][2];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int row = j * 16 + (lane & 15);
#pragma unroll
    for (int s = 0; s < 2; ++s) boff[j][s] = row * 128 + (((s * 4 + kgrp) ^ rsw(row)) << 4);
  }
  // Token fragments come straight from global memory (HBM) two chunks ahead,
  // issued after the next chunk's router-row loads: loads complete in issue
  // order, so the wait for those rows (before they are written to LDS) leaves
  // the newest token loads in flight.  The barrier waits for LDS only (a
  // __syncthreads would also drain the prefetches).
  const int nkc = k_slice / kRtKc;
  // One chunk: stage the next chunk's router rows, prefetch the token
  // fragments of chunk kc+2 into `aload`, multiply chunk kc (`ause`).  The
  // loop below rotates three fragment buffers by renaming (unrolled by 3), so
  // no copy ever waits on an in-flight prefetch.
  auto chunk = [&](int kc, const bf16x8(&ause)[2], bf16x8(&aload)[2]) {
    const uint8_t* cur = wt + (kc & 1) * kStage;
    uint8_t* nxt = wt + ((kc + 1) & 1) * kStage;
    // past the last chunk the last rows are staged again into the free slot
    const int kn = min(kc + 1, nkc - 1) * kRtKc;
#pragma unroll
    for (int i = 0; i < kPer; ++i) stg[i] = *reinterpret_cast<const u32x4*>(src[i] + kn);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      aload[s] = *reinterpret_cast<const bf16x8*>(ap + min(kc + 2, nkc - 1) * kRtKc + s * 32);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(cur + boff[j][s]);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ause[s], b, acc[j], 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4*>(nxt + dst[i]) = stg[i];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  bf16x8 a0[2], a1[2], a2[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    a0[s] = *reinterpret_cast<const bf16x8*>(ap + s * 32);
    a1[s] = *reinterpret_cast<const bf16x8*>(ap + min(1, nkc - 1) * kRtKc + s * 32);
  }
  for (int kc = 0; kc < nkc; kc += 3) {
    chunk(kc, a0, a2);
    if (kc + 1 < nkc) chunk(kc + 1, a1, a0);
    if (kc + 2 < nkc) chunk(kc + 2, a2, a1);
  }
  // lane holds tokens (lane/16)*4 + i, expert lane%16 of each 16-wide block;
  // experts past E hold partial sums of a clamped row and are never read.
  float* out = part + (size_t)blockIdx.z * T * e_pad;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + (lane >> 4) * 4 + i;
      if (t < T) out[(size_t)t * e_pad + e0 + j * 16 + (lane & 15)] = acc[j][i];
    }
}

// One wave per token: logits = sum of the k-slice partials (ascending) + bias.
template <int NV>
__global__ __launch_bounds__(256) void route_select_kernel(
    const float* __restrict__ part, int n_slices, int e_pad, const float* __restrict__ bias,
    int T, int E, int K, int score, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ weights, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      float z = part[(size_t)t * e_pad + e];
      for (int s = 1; s < n_slices; ++s) z += part[((size_t)s * T + t) * e_pad + e];
      v[i] = z + (bias ? bias[e] : 0.f);
    } else {
      v[i] = -INFINITY;
    }
  }
  select_topk<NV>(v, E, K, score, renorm, t, ids, weights, logits, lane);
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

// Router tile width: NT blocks of 16 experts, NT a power of two <= 16.
int route_nt(const moe_config_t& c) {
  int nt = 1;
  while (nt < 16 && nt * 16 < c.num_experts) nt *= 2;
  return nt;
}

int route_e_pad(const moe_config_t& c) {
  const int ne = route_nt(c) * 16;
  return ceil_div(c.num_experts, ne) * ne;
}

// Slices of the reduction dimension: a function of d and E only (never of
// the token count, so splitting a batch does not change any token's sum
// order).  At most d / (4 E_pad) slices, so the fp32 partials stay a small
// fraction of the token traffic, and at most 8; slices are 64-multiples.
int route_k_slices(const moe_config_t& c) {
  const int e_pad = route_e_pad(c);
  int ks = 1;
  while (ks < 8 && 2 * ks <= c.hidden / (4 * e_pad) && c.hidden % (2 * ks * kRtKc) == 0) ks *= 2;
  return ks;
}

size_t route_partial_floats(const moe_config_t& c) {
  return (size_t)route_k_slices(c) * c.num_tokens * route_e_pad(c);
}

template <int NV>
hipError_t launch_select(const moe_config_t& c, const float* part, int ks, int e_pad,
                         const float* bias, int32_t* ids, float* w, float* logits, hipStream_t s) {
  hipLaunchKernelGGL(route_select_kernel<NV>, dim3(ceil_div(c.num_tokens, 4)), dim3(256), 0, s,
                     part, ks, e_pad, bias, c.num_tokens, c.num_experts, c.top_k, c.score,
                     c.renormalize, ids, w, logits);
  return hipGetLastError();
}

template <int NT>
void launch_logits(const moe_config_t& c, const void* x, const void* wr, int e_pad, int ks,
                   float* part, hipStream_t s) {
  const dim3 grid(ceil_div(c.num_tokens, kRtTok), e_pad / (NT * 16), ks);
  hipLaunchKernelGGL(route_logits_kernel<NT>, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr),
                     c.num_tokens, c.hidden, c.num_experts, e_pad, c.hidden / ks, part);
}

hipError_t launch_bf16(const moe_config_t& c, const void* x, const void* wr, const float* bias,
                       int32_t* ids, float* w, float* logits, float* part, hipStream_t s) {
  const int ks = route_k_slices(c);
  const int e_pad = route_e_pad(c);
  switch (route_nt(c)) {
    case 1: launch_logits<1>(c, x, wr, e_pad, ks, part, s); break;
    case 2: launch_logits<2>(c, x, wr, e_pad, ks, part, s); break;
    case 4: launch_logits<4>(c, x, wr, e_pad, ks, part, s); break;
    case 8: launch_logits<8>(c, x, wr, e_pad, ks, part, s); break;
    default: launch_logits<16>(c, x, wr, e_pad, ks, part, s); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nv = ceil_div(c.num_experts, kWave);
  if (nv <= 1) return launch_select<1>(c, part, ks, e_pad, bias, ids, w, logits, s);
  if (nv <= 2) return launch_select<2>(c, part, ks, e_pad, bias, ids, w, logits, s);
  if (nv <= 4) return launch_select<4>(c, part, ks, e_pad, bias, ids, w, logits, s);
  return launch_select<8>(c, part, ks, e_pad, bias, ids, w, logits, s);
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

size_t route_workspace_bytes(const moe_config_t& c) {
  return c.dtype == MOE_BF16 ? align_up(route_partial_floats(c) * sizeof(float), 256) : 0;
}

hipError_t launch_route(const moe_config_t& c, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* weights, float* logits,
                        void* workspace, hipStream_t s) {
  if (c.dtype == MOE_BF16)
    return launch_bf16(c, x, w_router, bias, ids, weights, logits,
                       static_cast<float*>(workspace), s);
  const int nv = ceil_div(c.num_experts, kWave);
  if (nv <= 1) return launch_f32<1>(c, x, w_router, bias, ids, weights, logits, s);
  if (nv <= 2) return launch_f32<2>(c, x, w_router, bias, ids, weights, logits, s);
  if (nv <= 4) return launch_f32<4>(c, x, w_router, bias, ids, weights, logits, s);
  return launch_f32<8>(c, x, w_router, bias, ids, weights, logits, s);
}

}  // namespace moe
