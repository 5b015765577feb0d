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
// registers).  Each lane owns 16-byte pieces of the output row; it issues the
// gathers of up to 8 expert rows at once (for top-2 and top-4, of 4 or 2
// pieces each, so 8 rows' worth are in flight per lane), accumulates w_k * y
// in fp32 in ascending k, adds the shared-expert rows, and rounds once.
// Routed rows too many for the Infinity Cache are read with streaming loads.
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

// Issues the loads of one batch: y[rows[j]] piece v for the NB slots.
// rows[j] < 0 marks an empty slot: its load reads the valid row `dummy` and
// the value is discarded by consume_batch's select (never multiplied by 0,
// which could turn a non-finite dummy into NaN).  NT: streaming loads, which
// do not allocate in the caches.
template <int NB, bool NT>
__device__ __forceinline__ void issue_batch(const u32x4* __restrict__ base, long long row_stride,
                                            int v, const int (&rows)[NB], int dummy,
                                            u32x4 (&buf)[NB]) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const u32x4* p = base + (long long)(rows[j] >= 0 ? rows[j] : dummy) * row_stride + v;
    buf[j] = NT ? __builtin_nontemporal_load(p) : *p;
  }
}

// Accumulates w_j * y_j of the NB slots of a loaded batch, in slot order,
// into acc.
template <typename T, int NB>
__device__ __forceinline__ void consume_batch(const u32x4 (&buf)[NB], const int (&rows)[NB],
                                              const float (&w)[NB], float (&acc)[Vec<T>::N]) {
  constexpr int N = Vec<T>::N;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    float f[N];
    Vec<T>::load(buf[j], f);
    const bool ok = rows[j] >= 0;
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = ok ? fmaf(w[j], f[i], acc[i]) : acc[i];
  }
}

// Both, for one batch: every load issued before the first use.
template <typename T, int NB, bool NT>
__device__ __forceinline__ void gather_batch(const u32x4* __restrict__ base, long long row_stride,
                                             int v, const int (&rows)[NB], const float (&w)[NB],
                                             int dummy, float (&acc)[Vec<T>::N]) {
  u32x4 buf[NB];
  issue_batch<NB, NT>(base, row_stride, v, rows, dummy, buf);
  consume_batch<T, NB>(buf, rows, w, acc);
}

// KB = routed rows gathered per batch (2, 4 or 8: the smallest that holds
// min(K, 8); K <= 16, so at most two batches); the shared-expert rows (at most
// 4) form one batch of their own.  NT: stream the routed rows (see
// launch_combine).
// SUMS: no shared rows and no rounding; the fp32 sums go to `out` as floats
// ([T, d] fp32, N floats per 16-byte input piece).
template <typename T, int KB, bool NT, bool SUMS = false>
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
  // A valid row for the loads of empty slots: the token's first local row,
  // or (no local row at all) row 0 of the buffer, whose values are unused.
  const unsigned long long has = __ballot(myrow >= 0);
  const int dummy = has ? __shfl(myrow, __builtin_ctzll(has), 64) : 0;
  // Row numbers and weights of both batches, read into scalar registers once:
  // a readlane inside the column loop makes every iteration wait for the
  // previous iteration's output store.
  int rows0[KB], rows1[KB];
  float w0[KB], w1[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) {  // lanes >= K hold row -1
    rows0[j] = __builtin_amdgcn_readlane(myrow, j);
    rows1[j] = __builtin_amdgcn_readlane(myrow, KB + j);
    w0[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myw), j));
    w1[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myw), KB + j));
  }
  const bool second = K > KB;
  // The rest of piece v (lanes with v0 + lane >= row_vecs re-read the row's
  // end and store nothing): fp32 sums out (SUMS), or the shared rows added and
  // the rounded row written.
  auto finish = [&](int v0, int v, float (&acc)[N]) {
    if (SUMS) {
      if (v0 + lane < row_vecs) {
        u32x4* o = out + ((size_t)t * row_vecs + v) * (N / 4);
#pragma unroll
        for (int q = 0; q < N / 4; ++q)
          o[q] = u32x4{__float_as_uint(acc[4 * q]), __float_as_uint(acc[4 * q + 1]),
                       __float_as_uint(acc[4 * q + 2]), __float_as_uint(acc[4 * q + 3])};
      }
      return;
    }
    if (n_shared > 0) {
      constexpr int SB = MOE_MAX_SHARED;
      int rows[SB];
      float w[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        rows[j] = j < n_shared ? j * num_tokens + t : -1;
        w[j] = 1.f;
      }
      // Unit weights: fmaf(1, y, acc) == acc + y exactly.
      gather_batch<T, SB, false>(y_shared, row_vecs, v, rows, w, t, acc);
    }
    if (v0 + lane < row_vecs) out[(size_t)t * row_vecs + v] = Vec<T>::store(acc);
  };
  // With few routed rows per token (KB = 2 or 4, so a single batch) the loads
  // of CH column pieces are issued together, 8 rows' worth per lane in flight
  // as with KB = 8; each piece is then finished in turn.
  constexpr int CH = KB == 2 ? 4 : KB == 4 ? 2 : 1;
  if constexpr (CH == 1) {
    for (int v0 = 0; v0 < row_vecs; v0 += kWave) {
      const int v = min(v0 + lane, row_vecs - 1);
      float acc[N];
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] = 0.f;
      if (has) {
        gather_batch<T, KB, NT>(y_sorted, row_vecs, v, rows0, w0, dummy, acc);
        if (second) gather_batch<T, KB, NT>(y_sorted, row_vecs, v, rows1, w1, dummy, acc);
      }
      finish(v0, v, acc);
    }
  } else {
    for (int v0 = 0; v0 < row_vecs; v0 += CH * kWave) {
      u32x4 buf[CH][KB];
      if (has) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
          issue_batch<KB, NT>(y_sorted, row_vecs, min(v0 + c * kWave + lane, row_vecs - 1),
                              rows0, dummy, buf[c]);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int vc = v0 + c * kWave;
        if (vc >= row_vecs) break;
        float acc[N];
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = 0.f;
        if (has) consume_batch<T, KB>(buf[c], rows0, w0, acc);
        finish(vc, min(vc + lane, row_vecs - 1), acc);
      }
    }
  }
}

// out = round(sums + y_shared[0] + ... ): one thread per 16-byte piece of the
// output rows; the shared rows are added in ascending s as fmaf(1, y, acc),
// the very operations of combine_kernel's shared-row batch, so the result is
// bit for bit the fused combine's.
template <typename T>
__global__ __launch_bounds__(256) void combine_finish_kernel(const float* __restrict__ sums,
                                                             const u32x4* __restrict__ y_shared,
                                                             int n_shared, long long pieces,
                                                             long long shared_stride,
                                                             u32x4* __restrict__ out) {
  constexpr int N = Vec<T>::N;
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  if (p >= pieces) return;
  float acc[N];
  const f32x4* sp = reinterpret_cast<const f32x4*>(sums) + p * (N / 4);
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const f32x4 a = sp[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[4 * q + i] = a[i];
  }
  for (int sh = 0; sh < n_shared; ++sh) {
    float f[N];
    Vec<T>::load(y_shared[sh * shared_stride + p], f);
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = fmaf(1.f, f[i], acc[i]);
  }
  out[p] = Vec<T>::store(acc);
}

}  // namespace

// Routed rows that cannot stay in the 256 MB Infinity Cache are gathered with
// streaming loads: allocating them there only evicts lines the gather never
// reads again (measured: 443 MB of rows 94 us streamed vs 105 us cached, 268 MB
// 76 vs 98 us; at 221 MB and below cached loads are faster).
constexpr double kStreamBytes = 256.0 * 1024 * 1024;

template <typename T, int KB>
static void launch_kb(const moe_config_t& c, const void* y_sorted, const int32_t* row_of,
                      const float* weights, const void* y_shared, int n_sh, int row_vecs,
                      void* out, hipStream_t s) {
  const int n_loc = c.expert_end - c.expert_begin;
  const double routed_bytes = (double)c.num_tokens * (c.top_k < n_loc ? c.top_k : n_loc) *
                              row_vecs * 16.0;
  auto kern = routed_bytes > kStreamBytes ? combine_kernel<T, KB, true> : combine_kernel<T, KB, false>;
  hipLaunchKernelGGL(kern, dim3(ceil_div(c.num_tokens, 4)), dim3(256), 0, s,
                     static_cast<const u32x4*>(y_sorted), row_of, weights,
                     static_cast<const u32x4*>(y_shared), c.num_tokens, c.top_k, n_sh, row_vecs,
                     static_cast<u32x4*>(out));
}

template <typename T>
static void launch_t(const moe_config_t& c, const void* y_sorted, const int32_t* row_of,
                     const float* weights, const void* y_shared, int n_sh, int row_vecs, void* out,
                     hipStream_t s) {
  if (c.top_k <= 2)
    launch_kb<T, 2>(c, y_sorted, row_of, weights, y_shared, n_sh, row_vecs, out, s);
  else if (c.top_k <= 4)
    launch_kb<T, 4>(c, y_sorted, row_of, weights, y_shared, n_sh, row_vecs, out, s);
  else
    launch_kb<T, 8>(c, y_sorted, row_of, weights, y_shared, n_sh, row_vecs, out, s);
}

template <typename T>
static hipError_t launch_sums_t(const moe_config_t& c, const void* y_sorted,
                                const int32_t* row_of, const float* weights, float* sums,
                                int row_vecs, hipStream_t s) {
  const int n_loc = c.expert_end - c.expert_begin;
  const double routed_bytes = (double)c.num_tokens * (c.top_k < n_loc ? c.top_k : n_loc) *
                              row_vecs * 16.0;
  const bool nt = routed_bytes > kStreamBytes;
  void (*kern)(const u32x4*, const int32_t*, const float*, const u32x4*, int, int, int, int,
               u32x4*);
  if (c.top_k <= 2)
    kern = nt ? combine_kernel<T, 2, true, true> : combine_kernel<T, 2, false, true>;
  else if (c.top_k <= 4)
    kern = nt ? combine_kernel<T, 4, true, true> : combine_kernel<T, 4, false, true>;
  else
    kern = nt ? combine_kernel<T, 8, true, true> : combine_kernel<T, 8, false, true>;
  hipLaunchKernelGGL(kern, dim3(ceil_div(c.num_tokens, 4)), dim3(256), 0, s,
                     static_cast<const u32x4*>(y_sorted), row_of, weights, nullptr, c.num_tokens,
                     c.top_k, 0, row_vecs, reinterpret_cast<u32x4*>(sums));
  return hipGetLastError();
}

hipError_t launch_combine_sums(const moe_config_t& c, const void* y_sorted, const int32_t* row_of,
                               const float* weights, float* sums, hipStream_t s) {
  const int elem = c.dtype == MOE_BF16 ? 2 : 4;
  const int row_vecs = c.hidden * elem / 16;
  if (c.dtype == MOE_BF16)
    return launch_sums_t<uint16_t>(c, y_sorted, row_of, weights, sums, row_vecs, s);
  return launch_sums_t<float>(c, y_sorted, row_of, weights, sums, row_vecs, s);
}

hipError_t launch_combine_finish(const moe_config_t& c, const float* sums, const void* y_shared,
                                 void* out, hipStream_t s) {
  const int elem = c.dtype == MOE_BF16 ? 2 : 4;
  const long long row_vecs = (long long)c.hidden * elem / 16;
  const long long pieces = (long long)c.num_tokens * row_vecs;
  const dim3 grid((unsigned)((pieces + 255) / 256));
  const int n_sh = y_shared ? c.num_shared : 0;
  if (c.dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_finish_kernel<uint16_t>, grid, dim3(256), 0, s, sums,
                       static_cast<const u32x4*>(y_shared), n_sh, pieces, pieces,
                       static_cast<u32x4*>(out));
  else
    hipLaunchKernelGGL(combine_finish_kernel<float>, grid, dim3(256), 0, s, sums,
                       static_cast<const u32x4*>(y_shared), n_sh, pieces, pieces,
                       static_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_combine(const moe_config_t& c, const void* y_sorted, const int32_t* row_of,
                          const float* weights, const void* y_shared, void* out, hipStream_t s) {
  const int elem = c.dtype == MOE_BF16 ? 2 : 4;
  const int row_vecs = c.hidden * elem / 16;
  const int n_sh = y_shared ? c.num_shared : 0;
  if (c.dtype == MOE_BF16)
    launch_t<uint16_t>(c, y_sorted, row_of, weights, y_shared, n_sh, row_vecs, out, s);
  else
    launch_t<float>(c, y_sorted, row_of, weights, y_shared, n_sh, row_vecs, out, s);
  return hipGetLastError();
}

}  // namespace moe
