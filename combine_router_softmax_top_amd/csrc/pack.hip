// Packed layout of the bf16 expert weight stacks.
//
// The grouped GEMM of the expert MLP ("Efficient and portable mixture-of-
// experts communication", Dispatch: the expert-contiguous rows feed a grouped
// GEMM) streams each weight matrix as k-tiles of 64 columns over blocks of
// 128 rows.  Packed, such a k-tile is one contiguous 16 KB piece and the
// k-tiles of a row block follow each other, so a tile's weights are read
// front to back:
//   [n, rows, cols]  ->  [n, rows/128, cols/64, 128, 64]   (rows % 128 == 0, cols % 64 == 0).
#include "moe_internal.h"

namespace moe {
namespace {

// One thread per 16-byte piece (8 bf16) of the packed stack: piece o is piece
// o % 8 of row (o / 8) % 128 of k-tile block o / 1024, and block q = (m, g, kt)
// holds rows g*128.. of matrix m, columns kt*64..; in the stacked [n*rows,
// cols] view its rows start at (q / nk) * 128.
__global__ __launch_bounds__(256) void pack_weights_kernel(const u32x4* __restrict__ in,
                                                           u32x4* __restrict__ out, int cols,
                                                           long long total) {
  const long long o = (long long)blockIdx.x * 256 + threadIdx.x;
  if (o >= total) return;
  const int piece = (int)(o & 7);
  const int r = (int)((o >> 3) & 127);
  const long long q = o >> 10;
  const int nk = cols / 64;
  const int kt = (int)(q % nk);
  const long long row = (q / nk) * 128 + r;
  out[o] = in[(row * cols + kt * 64) / 8 + piece];
}

}  // namespace

hipError_t launch_pack_weights(int n, int rows, int cols, const void* in, void* out,
                               hipStream_t s) {
  const long long total = (long long)n * rows * cols / 8;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     static_cast<const u32x4*>(in), static_cast<u32x4*>(out), cols, total);
  return hipGetLastError();
}

}  // namespace moe
