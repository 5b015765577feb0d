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
//     blocks; an expert's last row tile with at most 192 rows runs at the
//     height of its rows rounded up to 64 (each wave 32, 64 or 96 rows x 64);
//   * 64-deep k-tiles (full 128-byte row segments) move straight from global
//     memory into LDS (global_load_lds, 16 B per lane): the activations in a
//     ring of two slots (one tile ahead), the weights in a ring of three (close
//     to two tiles ahead, they miss L2 more often, and issued a k-step apart
//     from the activation loads), 160 KB in all; tiles of at most 64 rows,
//     which mostly stream their weights, run a ring of four slots for each
//     operand instead, every k-tile's loads issued three k-tiles ahead; the
//     rows are XOR-swizzled in 16-byte chunks so the fragment reads are free
//     of bank conflicts;
//   * the epilogue stages the rounded tile through LDS, so each store
//     instruction writes whole row segments;
//   * ragged groups: the tile list (expert, row tile, column tile) is derived
//     on the device from the expert offsets; the grid is the host's upper
//     bound and surplus workgroups exit at once (no host synchronisation); the
//     shared experts join the same two launches as extra groups of T rows;
//   * the row tiles of all experts (full-height first, then the shorter last
//     tiles, tallest first) form bands of 16; the 8 XCDs work on the same band
//     at once as a 2 x 4 grid (8 rows x a quarter of the columns each), so a
//     weight tile streams from memory at most twice per band and an
//     activation tile is shared by 4 XCDs, the repeats served by the
//     Infinity Cache;
//   * the k order of every output is fixed (64-wide tiles ascending, MFMA
//     k-blocks of 16 ascending) and independent of the row tiling, so a row's
//     result does not depend on which other rows share its call.
// fp32 path: a plain LDS-tiled VALU kernel (64x64 tiles, 4x4 per thread,
// 64-deep k-steps), on the same tile list.
#include <math.h>

#include "grouped_gemm.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ bf16 MFMA GEMM

constexpr int kBK = kRowBytes / 2;  // bf16 k per k-tile

struct Frags {
  bf16x8 a[4], b[kBF];
};

// Fragments of k-step ks (16 deep) of a staged tile: NFA A fragments (rows
// a_row0 + 32i) and 2 B fragments (rows b_row[j]); xa/xb hold (lane's
// k-group) ^ swz(row).
template <int NFA>
__device__ __forceinline__ void load_frags(const uint8_t* sa, const uint8_t* sb, int ks,
                                           int a_row0, const int (&b_row)[kBF],
                                           const int (&xa)[4], const int (&xb)[kBF], Frags& f) {
#pragma unroll
  for (int i = 0; i < NFA; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(sa + (a_row0 + i * 32) * kRowBytes +
                                              (((2 * ks) ^ xa[i]) << 4));
#pragma unroll
  for (int j = 0; j < kBF; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(sb + b_row[j] * kRowBytes +
                                              (((2 * ks) ^ xb[j]) << 4));
}

// The weights go in the MFMA's first (row) operand, so each 32x32 block holds
// the transposed output: a lane keeps one output row and runs of 4 adjacent
// output columns, which the epilogue writes to LDS 8 bytes at a time.
template <int NFA>
__device__ __forceinline__ void mma_step(const Frags& f, f32x16 (&acc)[4][kBF]) {
#pragma unroll
  for (int i = 0; i < NFA; ++i)
#pragma unroll
    for (int j = 0; j < kBF; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

struct TileArgs {
  const uint16_t* A;
  int lda;
  const uint16_t* bg;
  const uint16_t* bu;
  uint16_t* C;
  int ldc;
  int row0, rows, m0, n0, N, Kdim;
  int b_packed;  // weights in the packed layout (16 KB k-tile blocks of 128 rows)
};

// One output tile of NFA * 64 rows: the 8 waves as 2 x 4, each NFA * 32 rows
// x 64 columns.  NFA = 4 for full tiles; 1..3 for the last row tile of an
// expert with at most 192 rows (that fraction of the A staging and of the
// MFMAs).  The k order of every output element is the same at every height.
// DEEP (64-row tiles only): a tile that little more than streams its weights
// keeps more of them in flight -- rings of 4 slots for both operands (A slots
// of 8 KB), each k-tile's A and B loads issued together three k-tiles ahead.
template <int EPI, int NFA, bool DEEP = false>
__device__ __forceinline__ void gemm_tile(const TileArgs& ta, uint8_t* lds) {
  static_assert(!DEEP || NFA == 1, "the deep ring holds 64-row activation tiles");
  constexpr int kNOut = EPI == EPI_SILU_GLU ? kBN / 2 : kBN;
  constexpr int kWaveRows = NFA * 32;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / kWN, wn = wave % kWN;
  constexpr int kWaveCols = kNOut / kWN;  // output (or h) columns per wave
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
  uint32_t off[2 * kDmaB];
#pragma unroll
  for (int j = 0; j < 2 * kDmaB; ++j) {
    const int r = ((j % kDmaB) * kWaves + wave) * kRowsPerDma + lane / kChunks;
    const int lchunk = (lane % kChunks) ^ swz(r);
    if (j < kDmaB) {
      off[j] = (uint32_t)(min(r, a_last) * ta.lda * 2 + lchunk * 16);
    } else {
      // r is the B-tile row; rows 128.. come from b_hi
      const int br = min(EPI == EPI_SILU_GLU ? (r & (kNOut - 1)) : r, b_last);
      // packed: row br is row br % 128 of the tile's row block br / 128, whose
      // k-tiles are 16 KB apart (a row block takes 128 * Kdim * 2 bytes in
      // either layout, so the tile's base is the same)
      off[j] = (uint32_t)(ta.b_packed ? (br & ~127) * Kdim * 2 + (br & 127) * kRowBytes
                                      : br * Kdim * 2) + lchunk * 16;
    }
  }

  f32x16 acc[4][kBF];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kBF; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragment rows: A rows wm*kWaveRows + i*32 + (lane & 31); B rows: the
  // wave's 64 output columns (gate/up pass: 32 gate rows and the matching 32
  // up rows).
  int b_row[kBF];
#pragma unroll
  for (int j = 0; j < kBF; ++j) {
    if (EPI == EPI_SILU_GLU)  // gate rows for j < kBF/2, the matching up rows after
      b_row[j] = (j / (kBF / 2)) * kNOut + wn * kWaveCols + (j % (kBF / 2)) * 32 + (lane & 31);
    else
      b_row[j] = wn * kWaveCols + j * 32 + (lane & 31);
  }
  const int a_row0 = wm * kWaveRows + (lane & 31);
  const int kgrp = lane >> 5;
  int xa[4], xb[kBF];
#pragma unroll
  for (int i = 0; i < 4; ++i) xa[i] = kgrp ^ swz(a_row0 + i * 32);
#pragma unroll
  for (int j = 0; j < kBF; ++j) xb[j] = kgrp ^ swz(b_row[j]);

  // LDS: A k-tiles in a ring of kAStages (2) slots, B k-tiles in a ring of
  // kBStages (3).  Right after the barrier that ends the reads of tile kt
  // (its last k-step's fragments are already in registers) tile kt's A slot
  // takes A(kt+2); during the first k-step of iteration kt the B slot of tile
  // kt-1 (free since barrier kt-1) takes B(kt+2).  Issuing the weight loads a
  // k-step away from the activation loads, instead of all of them in one
  // burst after the barrier, measured 3-4 % faster.  A load is thus in flight
  // for about one (A) or one and three quarters (B) k-tiles before the
  // barrier that needs it.  Loads complete in issue order; the wait before
  // barrier kt needs tile kt+1 and leaves only the B(kt+2) loads in flight
  // (kVmBarrier).  Fragments are double-buffered across the k-steps; the
  // barrier comes before the last k-step's MFMAs, which overlap the next
  // tile's first fragment reads and the new A loads.  The body has no
  // branches: past the last tile the loads re-read the last tile into free
  // slots and the next-tile fragments go unused.
  constexpr int NA = NFA;  // A loads per wave: 64 rows each across the 8 waves
  constexpr int kMfma = NFA * kBF, kReads = NFA + kBF;  // per k-step
  constexpr int kMaxStages = kAStages > kBStages ? kAStages : kBStages;
  // Loads issued after tile 0's in the prologue (A1, B1); after tile kt+1's
  // by barrier kt (the B(kt+2) loads of iteration kt, issued after A(kt+1)).
  // DEEP: k-tiles kt+2 and kt+3 in both cases.
  constexpr int kDeep = 4;                                   // DEEP ring slots
  constexpr int kASlot = DEEP ? kSlotBytes / 4 : kSlotBytes;  // A slot bytes
  constexpr int kVmPrologue =
      DEEP ? 2 * (NA + kDmaB) : (kAStages - 1) * NA + (kBStages - 2) * kDmaB;
  constexpr int kVmBarrier = DEEP ? 2 * (NA + kDmaB) : kDmaB;
  static_assert(kAStages == 2 && kBStages == 3 && kVmPrologue < 64, "vmcnt immediates");
  static_assert(!DEEP || kDeep * (kASlot + kSlotBytes) <= (kAStages + kBStages) * kSlotBytes,
                "LDS budget");
  uint8_t* a_slots = lds;
  uint8_t* b_slots = lds + (DEEP ? kDeep * kASlot : kAStages * kSlotBytes);
  const int nk = Kdim / kBK;
  const int last = (nk - 1) * kRowBytes;
  // The weights' k-tile step: 128 bytes along a row, or a packed 16 KB block.
  const int b_step = ta.b_packed ? 128 * kRowBytes : kRowBytes;
  const int b_lastk = (nk - 1) * b_step;
  if constexpr (DEEP) {
#pragma unroll
    for (int t = 0; t < kDeep - 1; ++t) {
      stage_a<NA>(a_slots + t * kASlot, a_tile, off, wave, min(t * kRowBytes, last));
      stage_b(b_slots + t * kSlotBytes, b_lo, b_hi, off, wave, min(t * b_step, b_lastk));
    }
  } else {
#pragma unroll
    for (int t = 0; t < kMaxStages; ++t) {
      if (t < kAStages) stage_a<NA>(a_slots + t * kSlotBytes, a_tile, off, wave, min(t * kRowBytes, last));
      if (t < kBStages - 1)  // B2 comes in iteration 0
        stage_b(b_slots + t * kSlotBytes, b_lo, b_hi, off, wave, min(t * b_step, b_lastk));
    }
  }
  wait_loads_and_barrier<kVmPrologue>();  // tile 0 landed
  Frags f0, f1;
  load_frags<NFA>(a_slots, b_slots, 0, a_row0, b_row, xa, xb, f0);
  constexpr int kAS = DEEP ? kDeep : kAStages, kBS = DEEP ? kDeep : kBStages;
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* sa = a_slots + (kt % kAS) * kASlot;
    uint8_t* sb = b_slots + (kt % kBS) * kSlotBytes;
    const uint8_t* na = a_slots + ((kt + 1) % kAS) * kASlot;
    const uint8_t* nb = b_slots + ((kt + 1) % kBS) * kSlotBytes;
    load_frags<NFA>(sa, sb, 1, a_row0, b_row, xa, xb, f1);
    if constexpr (DEEP) {  // k-tile kt+3 into the slots of kt-1, free since barrier kt-1
      const int t3 = (kt + kDeep - 1) % kDeep;
      stage_a<NA>(a_slots + t3 * kASlot, a_tile, off, wave, min((kt + kDeep - 1) * kRowBytes, last));
      stage_b(b_slots + t3 * kSlotBytes, b_lo, b_hi, off, wave,
              min((kt + kDeep - 1) * b_step, b_lastk));
    } else {
      stage_b(b_slots + ((kt + kBStages - 1) % kBStages) * kSlotBytes, b_lo, b_hi, off, wave,
              min((kt + kBStages - 1) * b_step, b_lastk));
    }
    mma_step<NFA>(f0, acc);
    pin_kstep_schedule<kMfma, kReads, DEEP ? NA + kDmaB : kDmaB>();
    load_frags<NFA>(sa, sb, 2, a_row0, b_row, xa, xb, f0);
    mma_step<NFA>(f1, acc);
    pin_kstep_schedule<kMfma, kReads, 0>();
    load_frags<NFA>(sa, sb, 3, a_row0, b_row, xa, xb, f1);
    mma_step<NFA>(f0, acc);
    pin_kstep_schedule<kMfma, kReads, 0>();
    wait_loads_and_barrier<kVmBarrier>();  // tile kt+1 landed; tile kt's slots free
    load_frags<NFA>(na, nb, 0, a_row0, b_row, xa, xb, f0);
    if constexpr (!DEEP) stage_a<NA>(sa, a_tile, off, wave, min((kt + kAStages) * kRowBytes, last));
    mma_step<NFA>(f1, acc);
    pin_kstep_schedule<kMfma, kReads, DEEP ? 0 : NA>();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue, through LDS.  Element r of lane l in a (transposed) 32x32 block
  // is output row l%32, column (r/4)*8 + (l/32)*4 + r%4: four adjacent bf16
  // per (lane, r/4), one 8-byte LDS write, into a row-major copy of the output
  // tile (row pitch padded by 16 bytes, so the 32 rows of one write share a
  // bank two rows at most).  Then each lane moves 16 bytes of a row to
  // memory, the lanes of a wave covering whole rows: a store instruction
  // writes 2 (or 4) full 512 (256)-byte row segments instead of 16-byte
  // pieces of 32 rows.  The barrier first waits for every wave's loads and
  // fragment reads, so the rings are free.
  constexpr int kOutBytes = kNOut * 2;
  constexpr int kPitch = kOutBytes + 16;
  static_assert(kBM * kPitch <= (kAStages + kBStages) * kSlotBytes, "output tile fits the rings");
  __syncthreads();
  {
    const int row_l = lane & 31;
    const int col_l = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < NFA; ++i) {
      uint8_t* lrow = lds + (wm * kWaveRows + i * 32 + row_l) * kPitch;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (EPI == EPI_SILU_GLU) {
#pragma unroll
          for (int j = 0; j < kBF / 2; ++j) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              v[q] = silu_f(acc[i][j][4 * g + q]) * acc[i][j + kBF / 2][4 * g + q];
            store_bf16x4(reinterpret_cast<uint16_t*>(lrow) + wn * kWaveCols + j * 32 + g * 8 + col_l, v);
          }
        } else {
#pragma unroll
          for (int j = 0; j < kBF; ++j) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * g + q];
            store_bf16x4(reinterpret_cast<uint16_t*>(lrow) + wn * kWaveCols + j * 32 + g * 8 + col_l, v);
          }
        }
      }
    }
  }
  __syncthreads();
  // Rows past the group's last one are not stored; N is a multiple of 64, so
  // a 16-byte piece (8 columns) is either wholly inside or wholly past N.
  constexpr int kLanesPerRow = kOutBytes / 16;
  constexpr int kRowsPerPass = kThreads / kLanesPerRow;
  constexpr int kTileRows = NFA * 64;
  static_assert(kTileRows % kRowsPerPass == 0, "whole passes");
  const int piece = tid % kLanesPerRow;
  const int n = n0 + piece * 8;
#pragma unroll
  for (int r = tid / kLanesPerRow; r < kTileRows; r += kRowsPerPass) {
    const int m = m0 + r;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * kPitch + piece * 16);
    if (m < ta.rows && n < N)
      *reinterpret_cast<u32x4*>(ta.C + (long long)(ta.row0 + m) * ta.ldc + n) = v;
  }
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int lda, long long strideA_batch,
    const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, long long strideB_group, long long strideB_batch,
    uint16_t* __restrict__ C, int ldc, long long strideC_batch,
    const int32_t* __restrict__ offsets, int n_groups, int fixed_rows, int N, int Kdim,
    const uint16_t* __restrict__ A2, long long strideA2, const uint16_t* __restrict__ B2_0,
    const uint16_t* __restrict__ B2_1, long long strideB2, uint16_t* __restrict__ C2,
    long long strideC2, int n_extra, int extra_rows, int b_packed) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(kAStages + kBStages) * kSlotBytes];

  // Output columns per tile: EPI_STORE 256, EPI_SILU_GLU 128 (gate and up 128 each).
  constexpr int kNOut = EPI == EPI_SILU_GLU ? kBN / 2 : kBN;
  const int nN = (N + kNOut - 1) / kNOut;
  Tile tl;
  if (!find_tile(offsets, n_groups, n_extra, extra_rows, fixed_rows, kBM, nN, tl)) return;

  TileArgs ta;
  ta.lda = lda;
  ta.ldc = ldc;
  if (tl.group < n_groups || offsets == nullptr) {
    const long long zb = (long long)blockIdx.z * strideB_batch;
    ta.A = A + (long long)blockIdx.z * strideA_batch;
    ta.bg = B0 + zb + (long long)tl.group * strideB_group;
    ta.bu = EPI == EPI_SILU_GLU ? B1 + zb + (long long)tl.group * strideB_group : ta.bg;
    ta.C = C + (long long)blockIdx.z * strideC_batch;
    ta.row0 = tl.row0;
  } else {  // an extra group: its own operands, rows from 0
    const int e = tl.group - n_groups;
    ta.A = A2 + (long long)e * strideA2;
    ta.bg = B2_0 + (long long)e * strideB2;
    ta.bu = EPI == EPI_SILU_GLU ? B2_1 + (long long)e * strideB2 : ta.bg;
    ta.C = C2 + (long long)e * strideC2;
    ta.row0 = 0;
  }
  ta.rows = tl.rows;
  ta.m0 = tl.m_tile * kBM;
  ta.n0 = tl.n_tile * kNOut;
  ta.N = N;
  ta.Kdim = Kdim;
  ta.b_packed = b_packed;
  // Height of the tile: its rows rounded up to 64 (a full tile when more
  // than 192), as find_tile classed it.
  const int left = tl.rows - ta.m0;
  if (left > 3 * kBM / 4)
    gemm_tile<EPI, 4>(ta, lds);
  else if (left > kBM / 2)
    gemm_tile<EPI, 3>(ta, lds);
  else if (left > kBM / 4)
    gemm_tile<EPI, 2>(ta, lds);
  else
    gemm_tile<EPI, 1, true>(ta, lds);
}

// ------------------------------------------------------------------ fp32 VALU GEMM

constexpr int kFM = 64, kFN = 64, kFK = 64;
constexpr int kFKT = kFK / 4;            // staging threads along k per row (4 k each)
constexpr int kFRowsPass = 256 / kFKT;   // rows staged per pass
constexpr int kFPass = kFM / kFRowsPass; // passes per operand tile
static_assert(kFM == kFN && kFPass * kFRowsPass == kFM, "fp32 staging shape");

// fp32 layers: 64 x 64 output tiles, 256 threads with 4 x 4 outputs each (and
// the matching up outputs in the gate/up pass), 64-deep k-steps through two
// LDS buffers: the next step's operands are loaded (16-byte loads) while the
// current one is multiplied (small layers are bound by the round trip of
// each step's loads, so the steps are deep).  k runs in ascending order for
// every output.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int lda, long long strideA_batch, const float* __restrict__ B0,
    const float* __restrict__ B1, long long strideB_group, long long strideB_batch,
    float* __restrict__ C, int ldc, long long strideC_batch, const int32_t* __restrict__ offsets,
    int n_groups, int fixed_rows, int N, int Kdim, const float* __restrict__ A2,
    long long strideA2, const float* __restrict__ B2_0, const float* __restrict__ B2_1,
    long long strideB2, float* __restrict__ C2, long long strideC2, int n_extra,
    int extra_rows) {
  constexpr bool kGlu = EPI == EPI_SILU_GLU;
  __shared__ __attribute__((aligned(16))) float sa[2][kFK][kFM + 4];
  __shared__ __attribute__((aligned(16))) float sg[2][kFK][kFN + 4];
  __shared__ __attribute__((aligned(16))) float su[kGlu ? 2 : 1][kFK][kFN + 4];
  const int nN = (N + kFN - 1) / kFN;
  Tile tl;
  if (!find_tile(offsets, n_groups, n_extra, extra_rows, fixed_rows, kFM, nN, tl)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = tl.m_tile * kFM, n0 = tl.n_tile * kFN;
  const float* bg;
  const float* bu;
  float* Cz;
  if (tl.group < n_groups || offsets == nullptr) {
    const long long zb = (long long)blockIdx.z * strideB_batch;
    A += (long long)blockIdx.z * strideA_batch;
    bg = B0 + zb + (long long)tl.group * strideB_group;
    bu = kGlu ? B1 + zb + (long long)tl.group * strideB_group : bg;
    Cz = C + (long long)blockIdx.z * strideC_batch;
  } else {  // an extra group: its own operands, rows from 0
    const int e = tl.group - n_groups;
    A = A2 + (long long)e * strideA2;
    bg = B2_0 + (long long)e * strideB2;
    bu = kGlu ? B2_1 + (long long)e * strideB2 : bg;
    Cz = C2 + (long long)e * strideC2;
    tl.row0 = 0;
  }

  // Staging: thread t loads 4 consecutive k (k4 = 4 (t % kFKT)) of rows
  // t/kFKT + kFRowsPass*j of each operand; rows past the tile's last one repeat
  // it, k past Kdim reads as zero (Kdim is a multiple of 16, so a group of 4 is
  // wholly inside or wholly past).
  const int k4 = (tid % kFKT) * 4;
  const float* pa[kFPass];
  const float* pg[kFPass];
  const float* pu[kFPass];
  int rr[kFPass];
#pragma unroll
  for (int j = 0; j < kFPass; ++j) {
    rr[j] = tid / kFKT + kFRowsPass * j;
    pa[j] = A + (long long)(tl.row0 + min(m0 + rr[j], tl.rows - 1)) * lda + k4;
    const int bn = min(n0 + rr[j], N - 1);
    pg[j] = bg + (long long)bn * Kdim + k4;
    pu[j] = bu + (long long)bn * Kdim + k4;
  }
  f32x4 ra[kFPass], rg[kFPass], ru[kFPass];
  auto load = [&](int k0) {
    const bool in = k0 + k4 < Kdim;
#pragma unroll
    for (int j = 0; j < kFPass; ++j) {
      ra[j] = in ? *reinterpret_cast<const f32x4*>(pa[j] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
      rg[j] = in ? *reinterpret_cast<const f32x4*>(pg[j] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
      if (kGlu) ru[j] = in ? *reinterpret_cast<const f32x4*>(pu[j] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kFPass; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sa[buf][k4 + c][rr[j]] = ra[j][c];
        sg[buf][k4 + c][rr[j]] = rg[j][c];
        if (kGlu) su[buf][k4 + c][rr[j]] = ru[j][c];
      }
  };
  float ag[4][4] = {}, au[4][4] = {};
  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < Kdim; k0 += kFK) {
    const bool more = k0 + kFK < Kdim;
    if (more) load(k0 + kFK);
#pragma unroll 8
    for (int kk = 0; kk < kFK; ++kk) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sa[buf][kk][ty * 4]);
      const f32x4 g = *reinterpret_cast<const f32x4*>(&sg[buf][kk][tx * 4]);
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
      if (kGlu) u = *reinterpret_cast<const f32x4*>(&su[buf][kk][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ag[i][j] = fmaf(a[i], g[j], ag[i][j]);
          if (kGlu) au[i][j] = fmaf(a[i], u[j], au[i][j]);
        }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= tl.rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float v = kGlu ? silu_f(ag[i][j]) * au[i][j] : ag[i][j];
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
  // Extra groups after the offset groups (the shared experts): operand bases
  // and strides per group, and their common row count.
  const void* A2; long long strideA2; const void* B2_0; const void* B2_1; long long strideB2;
  void* C2; long long strideC2; int n_extra; int extra_rows;
  int b_packed;  // bf16 weights in the packed layout (moe_pack_weights)
};

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
                       g.strideC_batch, g.offsets, g.n_groups, g.fixed_rows, g.N, g.Kdim,
                       static_cast<const uint16_t*>(g.A2), g.strideA2,
                       static_cast<const uint16_t*>(g.B2_0), static_cast<const uint16_t*>(g.B2_1),
                       g.strideB2, static_cast<uint16_t*>(g.C2), g.strideC2, g.n_extra,
                       g.extra_rows, g.b_packed);
  } else {
    const int rt = g.offsets ? g.max_row_tiles_bound : ceil_div(g.fixed_rows, kFM);
    const dim3 grid(grid_for(rt, ceil_div(g.N, kFN)), 1, g.batch);
    hipLaunchKernelGGL(gemm_f32_kernel<EPI>, grid, dim3(256), 0, s,
                       static_cast<const float*>(g.A), g.lda, g.strideA_batch,
                       static_cast<const float*>(g.B0),
                       static_cast<const float*>(g.B1), g.strideB_group, g.strideB_batch,
                       static_cast<float*>(g.C), g.ldc, g.strideC_batch, g.offsets, g.n_groups,
                       g.fixed_rows, g.N, g.Kdim, static_cast<const float*>(g.A2), g.strideA2,
                       static_cast<const float*>(g.B2_0), static_cast<const float*>(g.B2_1),
                       g.strideB2, static_cast<float*>(g.C2), g.strideC2, g.n_extra, g.extra_rows);
  }
  return hipGetLastError();
}

}  // namespace

// The launch grids of launch_expert_mlp, in 64-bit: grid_for over the row-tile
// bound and the column tiles of each pass, times the threads per workgroup.
long long expert_mlp_max_workitems(const moe_config_t& c) {
  const bool bf16 = c.dtype == MOE_BF16;
  const long long T = c.num_tokens, K = c.top_k, S = c.num_shared;
  const long long n_loc = c.expert_end - c.expert_begin;
  const long long bm = bf16 ? kBM : kFM;
  const long long rt = ceil_div_ll(T * K, bm) + n_loc + S * ceil_div_ll(T, bm);
  auto workitems = [&](long long col_tiles) {
    const long long rx = xcd_row_groups(col_tiles >= 4 ? 4 : (int)col_tiles), cx = 8 / rx;
    const long long per_xcd = ceil_div_ll(col_tiles, cx) * (ceil_div_ll(rt, rx) + 1);
    return 8 * per_xcd * (bf16 ? kThreads : 256);
  };
  const long long up = workitems(ceil_div_ll(c.intermediate, bf16 ? kBN / 2 : kFN));
  const long long down = workitems(ceil_div_ll(c.hidden, bf16 ? kBN : kFN));
  return up > down ? up : down;
}

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
                             void* workspace, hipStream_t s, int parts) {
  const int T = c.num_tokens, K = c.top_k, d = c.hidden, I = c.intermediate;
  const size_t elem = c.dtype == MOE_BF16 ? 2 : 4;
  char* ws = static_cast<char*>(workspace);
  void* h = ws;
  void* h_sh = ws + align_up((size_t)T * K * I * elem, 256);
  const int bm = c.dtype == MOE_BF16 ? kBM : kFM;
  // Routed groups (the local experts, rows from the offsets) unless only the
  // shared experts are asked for; shared experts unless only the routed ones.
  const int n_loc = (parts & kMlpRouted) ? c.expert_end - c.expert_begin : 0;
  const int S = (parts & kMlpShared) ? c.num_shared : 0;
  // The shared experts run in the same launches as the routed ones, as extra
  // groups of T rows, so their tiles fill the routed launches' last rounds.
  const int row_bound = (n_loc > 0 ? ceil_div(T * K, bm) + n_loc : 0) + S * ceil_div(T, bm);
  if (row_bound == 0) return hipSuccess;

  GemmArgs up{x_sorted, d, 0, w_gate, w_up, (long long)I * d, 0, h, I, 0,
              offsets, n_loc, 0, row_bound, I, d, 1,
              x, 0, ws_gate, ws_up, (long long)I * d, h_sh, (long long)T * I, S, T,
              c.weight_layout == MOE_WEIGHTS_PACKED};
  hipError_t err = run_gemm<EPI_SILU_GLU>(c.dtype, up, s);
  if (err != hipSuccess) return err;
  GemmArgs down{h, I, 0, w_down, nullptr, (long long)d * I, 0, y_sorted, d, 0,
                offsets, n_loc, 0, row_bound, d, I, 1,
                h_sh, (long long)T * I, ws_down, nullptr, (long long)d * I, y_shared,
                (long long)T * d, S, T, c.weight_layout == MOE_WEIGHTS_PACKED};
  return run_gemm<EPI_STORE>(c.dtype, down, s);
}

// The down projection alone (bf16 h and weights), for the block-scaled gate/up
// path: the same launch as launch_expert_mlp's second GEMM, the S shared
// experts (h_sh [S, T, I], ws_down, y_shared) as extra groups.
hipError_t launch_grouped_down_bf16(const moe_config_t& c, const void* h, const int32_t* offsets,
                                    const void* w_down, void* y_sorted, hipStream_t s,
                                    const void* h_sh, const void* ws_down, void* y_shared, int S) {
  const int T = c.num_tokens, K = c.top_k, d = c.hidden, I = c.intermediate;
  const int n_loc = c.expert_end - c.expert_begin;
  const int row_bound = ceil_div(T * K, kBM) + n_loc + S * ceil_div(T, kBM);
  GemmArgs down{h, I, 0, w_down, nullptr, (long long)d * I, 0, y_sorted, d, 0,
                offsets, n_loc, 0, row_bound, d, I, 1,
                h_sh, (long long)T * I, ws_down, nullptr, (long long)d * I, y_shared,
                (long long)T * d, S, T, c.weight_layout == MOE_WEIGHTS_PACKED};
  return run_gemm<EPI_STORE>(MOE_BF16, down, s);
}

}  // namespace moe
