// Grouped SiLU-gated expert MLP over expert-contiguous rows.
//
// Operation ("Efficient and portable mixture-of-experts communication",
// Introduction: each expert is a small MLP; Dispatch: the contiguous
// per-expert buffer is the input of a downstream grouped GEMM):
//     h = SiLU(X_e W_gate[e]^T) * (X_e W_up[e]^T),   y = h W_down[e]^T
// for the rows X_e of each local expert e, and the same MLP applied to every
// token for the shared experts.
//
// bf16 path (gfx950 MFMA, fp32 accumulation):
//   * one 512-thread workgroup computes a 256x256 output tile (gate/up pass:
//     256 rows x (128 gate + 128 up) columns, multiplied together in the
//     epilogue, so h is written once, in bf16); eight waves (two per SIMD)
//     in a 2x4 grid, each a 128x64 sub-tile of 4x2 v_mfma_f32_32x32x16_bf16
//     blocks; an expert's last row tile with at most 128 rows runs as a
//     half-height tile (each wave 64x64);
//   * 64-deep k-tiles (full 128-byte row segments) move straight from global
//     memory into LDS (global_load_lds, 16 B per lane): the activations in a
//     ring of two slots (one tile ahead), the weights in a ring of three (two
//     tiles ahead, they miss L2 more often), 160 KB in all; the rows are
//     XOR-swizzled in 16-byte chunks so the fragment reads are free of bank
//     conflicts;
//   * ragged groups: the tile list (expert, row tile, column tile) is derived
//     on the device from the expert offsets; the grid is the host's upper
//     bound and surplus workgroups exit at once (no host synchronisation);
//   * the row tiles of all experts form bands of 16; the 8 XCDs work on the
//     same band at once, each on an eighth of its columns, so a weight tile
//     streams from HBM once per band and the activations shared by the XCDs
//     come from the Infinity Cache;
//   * the k order of every output is fixed (64-wide tiles ascending, MFMA
//     k-blocks of 16 ascending) and independent of the row tiling, so a row's
//     result does not depend on which other rows share its call.
// fp32 path: a plain LDS-tiled VALU kernel (64x64 tiles, 4x4 per thread).
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ tiles

struct Tile {
  int row0;     // first row of the group in A / C
  int rows;     // rows of the group
  int group;    // expert (weight stack index)
  int m_tile;   // row tile inside the group
  int n_tile;   // column tile
};

__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Tiles of group j (lane-parallel over groups; lanes past n_groups give 0).
__device__ __forceinline__ int group_tiles(const int32_t* __restrict__ offsets, int n_groups,
                                           int j, int BM, int nN, int& a, int& b) {
  a = b = 0;
  if (j >= n_groups) return 0;
  a = offsets[j];
  b = offsets[j + 1];
  return (b - a + BM - 1) / BM * nN;
}

constexpr int kBandRows = 16;  // row tiles per band

// Maps this workgroup onto (group, row tile, column tile).  Groups are the
// local experts (from the device offsets) or, with offsets == nullptr, a single
// group of fixed_rows rows.  The row tiles of all groups, in order, form one
// list cut into bands of kBandRows row tiles; the 8 XCDs (workgroup ids go
// round-robin over them, XCD x running ids x, x+8, ...) all work on the same
// band at a time, each on an eighth of the band's tiles taken column-major, so
// an XCD holds a couple of weight column tiles across all the band's rows.
// A weight tile then streams from HBM once per band, and the activation rows,
// shared by the 8 XCDs at the same time, come from the Infinity Cache after
// the first read.  Returns false for surplus workgroups.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int n_groups,
                                          int fixed_rows, int BM, int nN, Tile& out) {
  const int lane = threadIdx.x & 63;
  int n_rt;  // row tiles in all groups
  if (offsets != nullptr) {
    n_rt = 0;
    for (int base = 0; base < n_groups; base += 64) {
      int a, b;
      const int cnt = group_tiles(offsets, n_groups, base + lane, BM, 1, a, b);
      n_rt += __shfl(wave_inclusive_sum(cnt), 63, 64);
    }
  } else {
    n_rt = (fixed_rows + BM - 1) / BM;
  }
  const int xcd = blockIdx.x & 7;
  int slot = blockIdx.x >> 3;
  const int full_bands = n_rt / kBandRows;
  const int per_full = 2 * nN;  // kBandRows * nN / 8 tiles of a full band per XCD
  int band, band_rows, t;
  if (slot < full_bands * per_full) {
    band = slot / per_full;
    band_rows = kBandRows;
    t = xcd * per_full + slot % per_full;
  } else {
    slot -= full_bands * per_full;
    band = full_bands;
    band_rows = n_rt - full_bands * kBandRows;
    const int tiles = band_rows * nN;
    const int first = xcd * tiles / 8, end = (xcd + 1) * tiles / 8;
    if (band_rows == 0 || slot >= end - first) return false;
    t = first + slot;
  }
  const int n_tile = t / band_rows;
  int rt = band * kBandRows + t % band_rows;  // global row tile
  int row0 = 0, rows = fixed_rows, group = 0;
  if (offsets != nullptr) {
    for (int base = 0;; base += 64) {
      int a, b;
      const int cnt = group_tiles(offsets, n_groups, base + lane, BM, 1, a, b);
      const int incl = wave_inclusive_sum(cnt);
      const int chunk = __shfl(incl, 63, 64);
      if (rt < chunk) {
        const int L = __builtin_ctzll(__ballot(incl > rt));
        row0 = __shfl(a, L, 64);
        rows = __shfl(b, L, 64) - row0;
        group = base + L;
        rt -= __shfl(incl - cnt, L, 64);
        break;
      }
      rt -= chunk;
    }
  }
  out.row0 = row0;
  out.rows = rows;
  out.group = group;
  out.m_tile = rt;
  out.n_tile = n_tile;
  return true;
}

// ------------------------------------------------------------------ bf16 MFMA GEMM

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 512;                             // 8 waves, 2 per SIMD
constexpr int kRowBytes = kBK * 2;                        // 128 B per staged row
constexpr int kSlotBytes = kBM * kRowBytes;               // 32 KB: one operand of one k-tile
constexpr int kAStages = 2, kBStages = 3;                 // 5 slots = 160 KB of LDS
constexpr int kDmaPerTile = 2 * kSlotBytes / (kThreads * 16);  // 8 x 16 B per thread
constexpr int kDmaA = kDmaPerTile / 2;
constexpr int kRowsPerDma = 1024 / kRowBytes;             // rows filled by one wave instruction

enum { EPI_STORE = 0, EPI_SILU_GLU = 1 };

__device__ __forceinline__ float silu_f(float z) { return z / (1.f + __expf(-z)); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS tile layout: 128-byte rows (64 bf16 of k) of eight 16-byte chunks; row
// R keeps logical chunk c in physical slot c ^ swz(R), swz(R) = (R ^ (R>>3)) & 7.
// A 64-lane ds_read_b128 of 32 consecutive rows at one logical chunk then hits
// distinct 16-byte slots within every 8-lane (128 B) and 16-lane (256 B)
// service group, i.e. no bank conflicts.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Staging one operand of a k-tile (32 KB per workgroup) with direct
// global->LDS loads: instruction j of wave w fills 1 KB of the slot = rows
// (8j + w)*8 .. +8; lane l covers row +l/8, physical chunk l%8, so its source
// is logical chunk (l%8) ^ swz(row).  NA = A instructions per wave (4 for a
// 256-row tile, 2 for a 128-row tile); B always takes 4 (rows 0..127 from
// b_lo, 128..255 from b_hi).
template <int NA>
__device__ __forceinline__ void stage_a(uint8_t* slot, const uint8_t* a_tile,
                                        const uint32_t (&off)[kDmaPerTile], int wave,
                                        int kbytes) {
#pragma unroll
  for (int j = 0; j < NA; ++j)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(a_tile + kbytes + off[j]),
                                     (lds_ptr_t)(slot + (j * 8 + wave) * 1024), 16, 0, 0);
}
__device__ __forceinline__ void stage_b(uint8_t* slot, const uint8_t* b_lo, const uint8_t* b_hi,
                                        const uint32_t (&off)[kDmaPerTile], int wave,
                                        int kbytes) {
#pragma unroll
  for (int j = 0; j < kDmaA; ++j)
    __builtin_amdgcn_global_load_lds(
        static_cast<const void*>((j < kDmaA / 2 ? b_lo : b_hi) + kbytes + off[kDmaA + j]),
        (lds_ptr_t)(slot + (j * 8 + wave) * 1024), 16, 0, 0);
}

struct Frags {
  bf16x8 a[4], b[2];
};

// Fragments of k-step ks (16 deep) of a staged tile: NFA A fragments (rows
// a_row0 + 32i) and 2 B fragments (rows b_row[j]); xa/xb hold (lane's
// k-group) ^ swz(row).
template <int NFA>
__device__ __forceinline__ void load_frags(const uint8_t* sa, const uint8_t* sb, int ks,
                                           int a_row0, const int (&b_row)[2],
                                           const int (&xa)[4], const int (&xb)[2], Frags& f) {
#pragma unroll
  for (int i = 0; i < NFA; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(sa + (a_row0 + i * 32) * kRowBytes +
                                              (((2 * ks) ^ xa[i]) << 4));
#pragma unroll
  for (int j = 0; j < 2; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(sb + b_row[j] * kRowBytes +
                                              (((2 * ks) ^ xb[j]) << 4));
}

// The weights go in the MFMA's first (row) operand, so each 32x32 block holds
// the transposed output: a lane keeps one output row and runs of 4 adjacent
// output columns, which the epilogue stores 8 bytes at a time.
template <int NFA>
__device__ __forceinline__ void mma_step(const Frags& f, f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < NFA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Wait until at most VM of this wave's global->LDS loads are in flight (loads
// complete in issue order, so every older load has landed) and its LDS reads
// have returned; then a workgroup barrier without a memory fence, so the
// younger loads stay in flight across it.
template <int VM>
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(VM) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling of one k-step (one basic block between sched_barriers): the
// k-step's NM MFMAs, each of the first ones followed by two of the ND LDS
// reads of the next k-step's fragments, the later ones by the NV global->LDS
// loads (the loads follow the reads in program order: they write LDS the
// compiler cannot tell apart from what the reads read).  The reads thus
// have most of the k-step to land.  Without this the compiler sinks each
// fragment read to just before its MFMA and waits on it there.
template <int NM, int ND, int NV, int I = 0>
__device__ __forceinline__ void pin_kstep_schedule() {
  if constexpr (I == NM) {
    __builtin_amdgcn_sched_barrier(0);
  } else {
    constexpr int kWithReads = (ND + 1) / 2;
    constexpr int kRest = NM - kWithReads;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (I < kWithReads) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * I + 2 <= ND ? 2 : 1, 0);  // DS read
    } else if constexpr (NV > 0) {
      constexpr int j = I - kWithReads;
      constexpr int n = NV * (j + 1) / kRest - NV * j / kRest;
      if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x020, n, 0);  // VMEM
    }
    pin_kstep_schedule<NM, ND, NV, I + 1>();
  }
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Four floats rounded to bf16 and written as one 8-byte store.
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, const float (&v)[4]) {
  const u32x2 w = {(uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16),
                   (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16)};
  *reinterpret_cast<u32x2*>(dst) = w;
}

struct TileArgs {
  const uint16_t* A;
  int lda;
  const uint16_t* bg;
  const uint16_t* bu;
  uint16_t* C;
  int ldc;
  int row0, rows, m0, n0, N, Kdim;
};

// One output tile.  NFA = 4: 256 rows, the 8 waves as 2 x 4, each 128 rows x
// 64 columns.  NFA = 2: the last row tile of an expert with at most 128 rows,
// each wave 64 rows x 64 columns (half the A staging and half the MFMAs).
// The k order of every output element is the same in both.
template <int EPI, int NFA>
__device__ __forceinline__ void gemm_tile(const TileArgs& ta, uint8_t* lds) {
  constexpr int kNOut = EPI == EPI_SILU_GLU ? kBN / 2 : kBN;
  constexpr int kWaveRows = NFA * 32;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = ta.m0, n0 = ta.n0, N = ta.N, Kdim = ta.Kdim;

  // Per-lane byte offsets of the staged rows inside the tile's operand blocks.
  // B rows 0..127 come from b_lo, rows 128..255 from b_hi (the up weights in
  // the gate/up pass, the next 128 rows of the same weights otherwise).
  const uint8_t* a_tile =
      reinterpret_cast<const uint8_t*>(ta.A + (long long)(ta.row0 + m0) * ta.lda);
  const uint8_t* b_lo = reinterpret_cast<const uint8_t*>(ta.bg + (long long)n0 * Kdim);
  const uint8_t* b_hi = EPI == EPI_SILU_GLU
                            ? reinterpret_cast<const uint8_t*>(ta.bu + (long long)n0 * Kdim)
                            : b_lo;
  const int a_last = ta.rows - 1 - m0;
  const int b_last = N - 1 - n0;
  uint32_t off[kDmaPerTile];
#pragma unroll
  for (int j = 0; j < kDmaPerTile; ++j) {
    const int r = ((j % kDmaA) * 8 + wave) * kRowsPerDma + lane / (kRowBytes / 16);
    const int lchunk = (lane % (kRowBytes / 16)) ^ swz(r);
    if (j < kDmaA) {
      off[j] = (uint32_t)(min(r, a_last) * ta.lda * 2 + lchunk * 16);
    } else {
      // r is the B-tile row; rows 128.. come from b_hi
      const int br = EPI == EPI_SILU_GLU ? (r & (kNOut - 1)) : r;
      off[j] = (uint32_t)(min(br, b_last) * Kdim * 2 + lchunk * 16);
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragment rows: A rows wm*kWaveRows + i*32 + (lane & 31); B rows: the
  // wave's 64 output columns (gate/up pass: 32 gate rows and the matching 32
  // up rows).
  int b_row[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (EPI == EPI_SILU_GLU)
      b_row[j] = j * kNOut + wn * 32 + (lane & 31);
    else
      b_row[j] = wn * 64 + j * 32 + (lane & 31);
  }
  const int a_row0 = wm * kWaveRows + (lane & 31);
  const int kgrp = lane >> 5;
  int xa[4], xb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) xa[i] = kgrp ^ swz(a_row0 + i * 32);
#pragma unroll
  for (int j = 0; j < 2; ++j) xb[j] = kgrp ^ swz(b_row[j]);

  // LDS: A k-tiles in a ring of 2 slots, B k-tiles in a ring of 3.  Right
  // after the barrier that ends the reads of tile kt (its last k-step's
  // fragments are already in registers) the slots of tile kt take A(kt+2)
  // and B(kt+3): the activations are in flight for five k-steps before they
  // are needed, the weights (which miss L2 more often) for nine.  The wait
  // before that barrier needs tile kt+1, so only the B(kt+2) loads issued
  // after A(kt+1) may still be in flight.  Fragments are double-buffered
  // across the four k-steps; the barrier comes before the last k-step's
  // MFMAs, which overlap the next tile's first fragment reads and the new
  // loads.  The body has no branches: past the last tile the loads re-read
  // the last tile into free slots and the next-tile fragments go unused.
  constexpr int NA = NFA == 4 ? kDmaA : kDmaA / 2;
  constexpr int kMfma = NFA * 2, kReads = NFA + 2;  // per k-step
  uint8_t* a_slots = lds;
  uint8_t* b_slots = lds + kAStages * kSlotBytes;
  const int nk = Kdim / kBK;
  const int last = (nk - 1) * kRowBytes;
  stage_a<NA>(a_slots, a_tile, off, wave, 0);
  stage_b(b_slots, b_lo, b_hi, off, wave, 0);
  stage_a<NA>(a_slots + kSlotBytes, a_tile, off, wave, min(kRowBytes, last));
  stage_b(b_slots + kSlotBytes, b_lo, b_hi, off, wave, min(kRowBytes, last));
  stage_b(b_slots + 2 * kSlotBytes, b_lo, b_hi, off, wave, min(2 * kRowBytes, last));
  wait_loads_and_barrier<NA + 2 * kDmaA>();  // tile 0 landed
  Frags f0, f1;
  load_frags<NFA>(a_slots, b_slots, 0, a_row0, b_row, xa, xb, f0);
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* sa = a_slots + (kt & 1) * kSlotBytes;
    uint8_t* sb = b_slots + (kt % kBStages) * kSlotBytes;
    const uint8_t* na = a_slots + ((kt + 1) & 1) * kSlotBytes;
    const uint8_t* nb = b_slots + ((kt + 1) % kBStages) * kSlotBytes;
    load_frags<NFA>(sa, sb, 1, a_row0, b_row, xa, xb, f1);
    mma_step<NFA>(f0, acc);
    pin_kstep_schedule<kMfma, kReads, 0>();
    load_frags<NFA>(sa, sb, 2, a_row0, b_row, xa, xb, f0);
    mma_step<NFA>(f1, acc);
    pin_kstep_schedule<kMfma, kReads, 0>();
    load_frags<NFA>(sa, sb, 3, a_row0, b_row, xa, xb, f1);
    mma_step<NFA>(f0, acc);
    pin_kstep_schedule<kMfma, kReads, 0>();
    wait_loads_and_barrier<kDmaA>();  // tile kt+1 landed; tile kt's slots free
    load_frags<NFA>(na, nb, 0, a_row0, b_row, xa, xb, f0);
    stage_a<NA>(sa, a_tile, off, wave, min((kt + 2) * kRowBytes, last));
    stage_b(sb, b_lo, b_hi, off, wave, min((kt + 3) * kRowBytes, last));
    mma_step<NFA>(f1, acc);
    pin_kstep_schedule<kMfma, kReads, NA + kDmaA>();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue.  Element r of lane l in a (transposed) 32x32 block is output
  // row l%32, column (r/4)*8 + (l/32)*4 + r%4: four adjacent bf16 per
  // (lane, r/4), stored as one 8-byte write.  N is a multiple of 64, so a
  // group of four columns is either wholly inside or wholly past N.
  const int row_l = lane & 31;
  const int col_l = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < NFA; ++i) {
    const int m = m0 + wm * kWaveRows + i * 32 + row_l;
    if (m >= ta.rows) continue;
    uint16_t* crow = ta.C + (long long)(ta.row0 + m) * ta.ldc;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (EPI == EPI_SILU_GLU) {
        const int n = n0 + wn * 32 + g * 8 + col_l;
        if (n < N) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = silu_f(acc[i][0][4 * g + q]) * acc[i][1][4 * g + q];
          store_bf16x4(crow + n, v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + j * 32 + g * 8 + col_l;
          if (n < N) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
            store_bf16x4(crow + n, v);
          }
        }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int lda, long long strideA_batch,
    const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, long long strideB_group, long long strideB_batch,
    uint16_t* __restrict__ C, int ldc, long long strideC_batch,
    const int32_t* __restrict__ offsets, int n_groups, int fixed_rows, int N, int Kdim) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(kAStages + kBStages) * kSlotBytes];

  // Output columns per tile: EPI_STORE 256, EPI_SILU_GLU 128 (gate and up 128 each).
  constexpr int kNOut = EPI == EPI_SILU_GLU ? kBN / 2 : kBN;
  const int nN = (N + kNOut - 1) / kNOut;
  Tile tl;
  if (!find_tile(offsets, n_groups, fixed_rows, kBM, nN, tl)) return;

  const long long zb = (long long)blockIdx.z * strideB_batch;
  TileArgs ta;
  ta.A = A + (long long)blockIdx.z * strideA_batch;
  ta.lda = lda;
  ta.bg = B0 + zb + (long long)tl.group * strideB_group;
  ta.bu = EPI == EPI_SILU_GLU ? B1 + zb + (long long)tl.group * strideB_group : ta.bg;
  ta.C = C + (long long)blockIdx.z * strideC_batch;
  ta.ldc = ldc;
  ta.row0 = tl.row0;
  ta.rows = tl.rows;
  ta.m0 = tl.m_tile * kBM;
  ta.n0 = tl.n_tile * kNOut;
  ta.N = N;
  ta.Kdim = Kdim;
  if (tl.rows - ta.m0 <= kBM / 2)
    gemm_tile<EPI, 2>(ta, lds);
  else
    gemm_tile<EPI, 4>(ta, lds);
}

// ------------------------------------------------------------------ fp32 VALU GEMM

constexpr int kFM = 64, kFN = 64, kFK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int lda, long long strideA_batch, const float* __restrict__ B0,
    const float* __restrict__ B1, long long strideB_group, long long strideB_batch,
    float* __restrict__ C, int ldc, long long strideC_batch, const int32_t* __restrict__ offsets,
    int n_groups, int fixed_rows, int N, int Kdim) {
  __shared__ float sa[kFK][kFM + 1];
  __shared__ float sg[kFK][kFN + 1];
  __shared__ float su[kFK][kFN + 1];
  const int nN = (N + kFN - 1) / kFN;
  Tile tl;
  if (!find_tile(offsets, n_groups, fixed_rows, kFM, nN, tl)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = tl.m_tile * kFM, n0 = tl.n_tile * kFN;
  const long long zb = (long long)blockIdx.z * strideB_batch;
  A += (long long)blockIdx.z * strideA_batch;
  const float* bg = B0 + zb + (long long)tl.group * strideB_group;
  const float* bu = EPI == EPI_SILU_GLU ? B1 + zb + (long long)tl.group * strideB_group : bg;
  float* Cz = C + (long long)blockIdx.z * strideC_batch;
  float ag[4][4] = {}, au[4][4] = {};
  for (int k0 = 0; k0 < Kdim; k0 += kFK) {
    // 64 rows x 16 k per operand: each thread stages 4 elements of each.
    for (int q = tid; q < kFM * kFK; q += 256) {
      const int r = q / kFK, kk = q % kFK;
      const int am = min(m0 + r, tl.rows - 1);
      sa[kk][r] = A[(long long)(tl.row0 + am) * lda + k0 + kk];
      const int bn = min(n0 + r, N - 1);
      sg[kk][r] = bg[(long long)bn * Kdim + k0 + kk];
      if (EPI == EPI_SILU_GLU) su[kk][r] = bu[(long long)bn * Kdim + k0 + kk];
    }
    __syncthreads();
    for (int kk = 0; kk < kFK; ++kk) {
      float a[4], g[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sa[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g[j] = sg[kk][tx * 4 + j];
        u[j] = EPI == EPI_SILU_GLU ? su[kk][tx * 4 + j] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ag[i][j] = fmaf(a[i], g[j], ag[i][j]);
          if (EPI == EPI_SILU_GLU) au[i][j] = fmaf(a[i], u[j], au[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= tl.rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float v = EPI == EPI_SILU_GLU ? silu_f(ag[i][j]) * au[i][j] : ag[i][j];
      Cz[(long long)(tl.row0 + m) * ldc + n] = v;
    }
  }
}

// ------------------------------------------------------------------ launch helpers

struct GemmArgs {
  const void* A; int lda; long long strideA_batch;
  const void* B0; const void* B1; long long strideB_group; long long strideB_batch;
  void* C; int ldc; long long strideC_batch;
  const int32_t* offsets; int n_groups; int fixed_rows; int max_row_tiles_bound;
  int N; int Kdim; int batch;
};

// Workgroups for an upper bound of row tiles: a multiple of 8, with room for
// the uneven split of the last band over the XCDs.
inline int grid_for(int row_tiles, int col_tiles) {
  const int g = row_tiles * col_tiles;
  return (g + 7) / 8 * 8 + 8;
}

template <int EPI>
hipError_t run_gemm(int dtype, const GemmArgs& g, hipStream_t s) {
  if (dtype == MOE_BF16) {
    constexpr int nout = EPI == EPI_SILU_GLU ? kBN / 2 : kBN;
    const int rt = g.offsets ? g.max_row_tiles_bound : ceil_div(g.fixed_rows, kBM);
    const dim3 grid(grid_for(rt, ceil_div(g.N, nout)), 1, g.batch);
    hipLaunchKernelGGL(gemm_bf16_kernel<EPI>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(g.A), g.lda, g.strideA_batch,
                       static_cast<const uint16_t*>(g.B0), static_cast<const uint16_t*>(g.B1),
                       g.strideB_group, g.strideB_batch, static_cast<uint16_t*>(g.C), g.ldc,
                       g.strideC_batch, g.offsets, g.n_groups, g.fixed_rows, g.N, g.Kdim);
  } else {
    const int rt = g.offsets ? g.max_row_tiles_bound : ceil_div(g.fixed_rows, kFM);
    const dim3 grid(grid_for(rt, ceil_div(g.N, kFN)), 1, g.batch);
    hipLaunchKernelGGL(gemm_f32_kernel<EPI>, grid, dim3(256), 0, s,
                       static_cast<const float*>(g.A), g.lda, g.strideA_batch,
                       static_cast<const float*>(g.B0),
                       static_cast<const float*>(g.B1), g.strideB_group, g.strideB_batch,
                       static_cast<float*>(g.C), g.ldc, g.strideC_batch, g.offsets, g.n_groups,
                       g.fixed_rows, g.N, g.Kdim);
  }
  return hipGetLastError();
}

}  // namespace

// Workspace: h for the routed rows [T*K, I] and for the shared experts [S, T, I].
size_t mlp_workspace_bytes(const moe_config_t& c) {
  const size_t elem = c.dtype == MOE_BF16 ? 2 : 4;
  size_t b = align_up((size_t)c.num_tokens * c.top_k * c.intermediate * elem, 256);
  b += align_up((size_t)c.num_shared * c.num_tokens * c.intermediate * elem, 256);
  return b;
}

hipError_t launch_expert_mlp(const moe_config_t& c, const void* x_sorted, const int32_t* offsets,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* y_sorted, const void* x, const void* ws_gate,
                             const void* ws_up, const void* ws_down, void* y_shared,
                             void* workspace, hipStream_t s) {
  const int T = c.num_tokens, K = c.top_k, d = c.hidden, I = c.intermediate;
  const int n_loc = c.expert_end - c.expert_begin;
  const size_t elem = c.dtype == MOE_BF16 ? 2 : 4;
  char* ws = static_cast<char*>(workspace);
  void* h = ws;
  void* h_sh = ws + align_up((size_t)T * K * I * elem, 256);
  const int bm = c.dtype == MOE_BF16 ? kBM : kFM;
  const int row_bound = ceil_div(T * K, bm) + n_loc;

  GemmArgs up{x_sorted, d, 0, w_gate, w_up, (long long)I * d, 0, h, I, 0,
              offsets, n_loc, 0, row_bound, I, d, 1};
  hipError_t err = run_gemm<EPI_SILU_GLU>(c.dtype, up, s);
  if (err != hipSuccess) return err;
  GemmArgs down{h, I, 0, w_down, nullptr, (long long)d * I, 0, y_sorted, d, 0,
                offsets, n_loc, 0, row_bound, d, I, 1};
  err = run_gemm<EPI_STORE>(c.dtype, down, s);
  if (err != hipSuccess || c.num_shared == 0) return err;

  GemmArgs sup{x, d, 0, ws_gate, ws_up, 0, (long long)I * d, h_sh, I, (long long)T * I,
               nullptr, 1, T, 0, I, d, c.num_shared};
  err = run_gemm<EPI_SILU_GLU>(c.dtype, sup, s);
  if (err != hipSuccess) return err;
  GemmArgs sdown{h_sh, I, (long long)T * I, ws_down, nullptr, 0, (long long)d * I, y_shared, d, (long long)T * d,
                 nullptr, 1, T, 0, d, I, c.num_shared};
  return run_gemm<EPI_STORE>(c.dtype, sdown, s);
}

}  // namespace moe
