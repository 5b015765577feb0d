// Achievable-peak probes of one MI355X: plain streaming copy / read / write
// kernels (16-byte accesses in contiguous per-workgroup blocks) and register-
// only MFMA loops (bf16 v_mfma_f32_32x32x16_bf16 and the block-scaled fp8
// v_mfma_scale_f32_32x32x64_f8f6f4).  The benchmark reports what they reach
// beside the nominal peaks (8 TB/s HBM, 2.5 PFLOP/s bf16, 5.0 PFLOP/s fp8),
// as the practical ceilings of the memory-bound and MFMA-bound kernels.
#include "moe_internal.h"
#include "moe_probe.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;

// Each workgroup walks the buffer in blocks of UNR * 4 KB (one 16-byte
// access per lane per KB, all UNR of a block issued before any is used),
// block b, b + gridDim.x, ...: a workgroup's accesses stay contiguous, which
// measured 15-20 % faster than a grid-wide stride of 16-byte accesses.  Reads
// are non-temporal (they are used once).  kind 0: dst = src (8 in flight,
// non-temporal stores too); 1: read src (8 in flight; an xor of every word,
// one dword per thread written so the loads stay live); 2: dst = a pattern
// (4 per block).  A tail shorter than a block is covered 16 bytes per lane.
template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void probe_stream_kernel(u32x4* __restrict__ dst,
                                                                      const u32x4* __restrict__ src,
                                                                      long long n,
                                                                      uint32_t* __restrict__ sink) {
  constexpr int UNR = KIND == 2 ? 4 : 8;
  constexpr long long kPer = (long long)kProbeThreads * UNR;  // 16-byte elements per block
  const long long step = (long long)gridDim.x * kPer;
  u32x4 acc = {0u, 0u, 0u, 0u};
  long long b = (long long)blockIdx.x * kPer;
  for (; b + kPer <= n; b += step) {
    u32x4 v[UNR];
    if constexpr (KIND != 2) {
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        v[u] = __builtin_nontemporal_load(src + b + u * kProbeThreads + threadIdx.x);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const long long i = b + u * kProbeThreads + threadIdx.x;
      if constexpr (KIND == 0) __builtin_nontemporal_store(v[u], dst + i);
      if constexpr (KIND == 1) acc ^= v[u];
      if constexpr (KIND == 2) dst[i] = u32x4{(uint32_t)u, 1u, 2u, 3u};
    }
  }
  // The tail (fewer than kPer elements, past the last whole block), read by
  // the workgroup whose next block would have started there.
  if (b < n) {
    for (long long i = b + threadIdx.x; i < n; i += kProbeThreads) {
      if constexpr (KIND == 0) dst[i] = src[i];
      if constexpr (KIND == 1) acc ^= src[i];
      if constexpr (KIND == 2) dst[i] = u32x4{0u, 1u, 2u, 3u};
    }
  }
  if constexpr (KIND == 1)
    sink[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

constexpr int kMfmaWaves = 8;  // two per SIMD
constexpr int kMfmaChains = 8; // independent accumulators per wave

typedef int i32x8 __attribute__((ext_vector_type(8)));

// kind 0: bf16 32x32x16 (32768 flop each); kind 1: fp8 E4M3 32x32x64 with
// unit E8M0 scales (131072 flop each).  Operands come from registers only;
// every lane writes the sum of its accumulators, so no MFMA is dead.
template <int KIND>
__global__ __launch_bounds__(64 * kMfmaWaves) void probe_mfma_kernel(int iters,
                                                                     float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.0078125f * (float)((lane + e) & 7));
      b[e] = (__bf16)(0.0078125f * (float)((lane * 3 + e) & 7));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  } else {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // E4M3 bytes of small magnitudes (exponent field 1..3)
      a[e] = 0x18181818 + ((lane + e) & 3);
      b[e] = 0x10101010 + ((lane * 3 + e) & 3);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0,
                                                                 127);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(long long)blockIdx.x * 64 * kMfmaWaves + threadIdx.x] = s;
}

}  // namespace
}  // namespace moe

extern "C" {

moe_status_t moe_probe_stream(int32_t kind, void* dst, const void* src, size_t bytes,
                              uint32_t* sink, int32_t workgroups, moe_stream_t stream) {
  if (kind < 0 || kind > 2 || workgroups < 1 || bytes % 16 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (kind != 1 && (!dst || reinterpret_cast<uintptr_t>(dst) % 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (kind != 2 && (!src || reinterpret_cast<uintptr_t>(src) % 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (kind == 1 && !sink) return MOE_ERR_INVALID_ARGUMENT;
  if ((long long)workgroups * moe::kProbeThreads >= moe::kMaxWorkItems) return MOE_ERR_UNSUPPORTED;
  const long long n = (long long)(bytes / 16);
  if (n == 0) return MOE_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  auto* d = static_cast<moe::u32x4*>(dst);
  const auto* r = static_cast<const moe::u32x4*>(src);
  if (kind == 0)
    hipLaunchKernelGGL(moe::probe_stream_kernel<0>, dim3(workgroups), dim3(moe::kProbeThreads), 0,
                       s, d, r, n, sink);
  else if (kind == 1)
    hipLaunchKernelGGL(moe::probe_stream_kernel<1>, dim3(workgroups), dim3(moe::kProbeThreads), 0,
                       s, d, r, n, sink);
  else
    hipLaunchKernelGGL(moe::probe_stream_kernel<2>, dim3(workgroups), dim3(moe::kProbeThreads), 0,
                       s, d, r, n, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, float* out,
                            moe_stream_t stream) {
  if (kind < 0 || kind > 1 || workgroups < 1 || iters < 1 || !out) return MOE_ERR_INVALID_ARGUMENT;
  if ((long long)workgroups * 64 * moe::kMfmaWaves >= moe::kMaxWorkItems) return MOE_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(moe::probe_mfma_kernel<0>, dim3(workgroups), dim3(64 * moe::kMfmaWaves), 0,
                       s, iters, out);
  else
    hipLaunchKernelGGL(moe::probe_mfma_kernel<1>, dim3(workgroups), dim3(64 * moe::kMfmaWaves), 0,
                       s, iters, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

double moe_probe_mfma_flops(int32_t kind, int32_t workgroups, int32_t iters) {
  const double per = kind == 0 ? 32.0 * 32 * 16 * 2 : 32.0 * 32 * 64 * 2;
  return per * moe::kMfmaChains * moe::kMfmaWaves * (double)workgroups * iters;
}

}  // extern "C"
