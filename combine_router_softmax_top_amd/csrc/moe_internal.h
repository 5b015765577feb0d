// Internal declarations shared by the HIP kernels and the C-ABI layer.
// Written for CDNA4 (gfx950): 64-lane wavefronts, bf16 MFMA, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
// Assignments (t*K + k) per dispatch chunk: one workgroup counts and ranks one chunk.
constexpr int kDispatchChunk = 1024;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline long long ceil_div_ll(long long a, long long b) { return (a + b - 1) / b; }

// HIP launches hold fewer work-items than this in each grid dimension.
constexpr long long kMaxWorkItems = 0xffffffffLL;
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- launchers (each returns the launch status) ----
size_t route_workspace_bytes(const moe_config_t& c);
hipError_t launch_route(const moe_config_t& c, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* weights, float* logits,
                        void* workspace, hipStream_t s);

size_t dispatch_workspace_bytes(const moe_config_t& c);
// xq != nullptr: the bf16 rows are encoded as MX-FP8 into codes xq [T*K, d]
// and scale words xs (MFMA layout, T*K rows); x_sorted is not written.
// n_invalid_out: where the invalid-id count goes (default: the first int32 of
// the workspace).
hipError_t launch_dispatch(const moe_config_t& c, const void* x, const int32_t* ids,
                           int32_t* counts, int32_t* offsets, void* x_sorted, int32_t* src_index,
                           int32_t* row_of, void* workspace, hipStream_t s,
                           uint8_t* xq = nullptr, uint32_t* xs = nullptr,
                           int32_t* n_invalid_out = nullptr);

// The library's own dispatch scratch on the current device (a file-scope
// device array of kNoallocScratchBytes): its device address, looked up once per
// device.
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(void** ptr);

size_t mlp_workspace_bytes(const moe_config_t& c);
// Work-items of the largest grouped-GEMM launch of a layer with this shape
// (bf16 or fp32; the block-scaled launches use the same tile grids with fewer
// threads per workgroup).
long long expert_mlp_max_workitems(const moe_config_t& c);
// parts: which groups the two launches hold -- the routed experts (rows from
// the offsets), the shared experts (T rows each), or both (the default).
enum { kMlpRouted = 1, kMlpShared = 2, kMlpBoth = 3 };
hipError_t launch_expert_mlp(const moe_config_t& c, const void* x_sorted, const int32_t* offsets,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* y_sorted, const void* x, const void* ws_gate,
                             const void* ws_up, const void* ws_down, void* y_shared,
                             void* workspace, hipStream_t s, int parts = kMlpBoth);

// moe_pack_weights: [n, rows, cols] bf16 -> [n, rows/128, cols/64, 128, 64].
hipError_t launch_pack_weights(int n, int rows, int cols, const void* in, void* out,
                               hipStream_t s);

hipError_t launch_mxfp8_quantize(int rows, int cols, int dtype, const void* in, long long ld,
                                 int layout, uint8_t* codes, uint8_t* scales, hipStream_t s);

// Shared experts of the block-scaled MLP: the tokens encoded (T rows, MFMA
// layout), their encoded gate / up stacks, down weights in the form of the
// routed ones (bf16 w_down, or wq_down + scales), and y_shared [S, T, d].
struct MxfpShared {
  const uint8_t* xq;
  const uint8_t* xq_scales;
  const uint8_t* wq_gate;
  const uint8_t* wq_gate_scales;
  const uint8_t* wq_up;
  const uint8_t* wq_up_scales;
  const void* w_down;
  const uint8_t* wq_down;
  const uint8_t* wq_down_scales;
  void* y;
};

// wq_down == nullptr: the down projection in bf16 (w_down); else in fp8
// (wq_down, wq_down_scales), h encoded as MX-FP8 in the workspace.  sh: the
// shared experts (c.num_shared of them), or nullptr.
hipError_t launch_expert_mlp_mxfp8(const moe_config_t& c, const uint8_t* xq,
                                   const uint8_t* xq_scales, const int32_t* offsets,
                                   const uint8_t* wq_gate, const uint8_t* wq_gate_scales,
                                   const uint8_t* wq_up, const uint8_t* wq_up_scales,
                                   const void* w_down, const uint8_t* wq_down,
                                   const uint8_t* wq_down_scales, void* y_sorted,
                                   void* workspace, hipStream_t s,
                                   const MxfpShared* sh = nullptr);

hipError_t launch_combine(const moe_config_t& c, const void* y_sorted, const int32_t* row_of,
                          const float* weights, const void* y_shared, void* out, hipStream_t s);
// The routed part of the combine, its fp32 sums (before any shared row and
// before the rounding) written to sums [T, d] fp32.
hipError_t launch_combine_sums(const moe_config_t& c, const void* y_sorted, const int32_t* row_of,
                               const float* weights, float* sums, hipStream_t s);
// out = round(sums + y_shared[0] + ... + y_shared[S-1]), added in that order
// exactly as launch_combine adds them.
hipError_t launch_combine_finish(const moe_config_t& c, const float* sums, const void* y_shared,
                                 void* out, hipStream_t s);

}  // namespace moe
