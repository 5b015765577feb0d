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
//     from the activation loads), 160 KB in all; the rows are
//     XOR-swizzled in 16-byte chunks so the fragment reads are free of bank
//     conflicts;
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

// Row tiles of a group of `rows` rows: `full` tiles computed at full height
// (BM rows, including a last tile of more than 3BM/4 rows) and, when the
// remainder is at most 3BM/4 rows, one short last tile of q quarters (q = 1..3,
// its rows rounded up to BM/4), which runs at that height.  q = 0: none.
__device__ __forceinline__ void group_row_tiles(int rows, int BM, int& full, int& q) {
  const int qr = BM / 4;
  const int qq = (rows % BM + qr - 1) / qr;  // 0..4
  full = rows / BM + (qq == 4 ? 1 : 0);
  q = qq == 4 ? 0 : qq;
}

// Groups per lane, at most (the local experts and the shared experts).
constexpr int kMaxGroupChunks = (MOE_MAX_EXPERTS + MOE_MAX_SHARED + 63) / 64;

constexpr int kBandRows = 16;  // row tiles per band

// XCD row groups of a band: the 8 XCDs form a grid of row groups x column
// groups over each band (2 x 4; 8 x 1 when there are fewer than 4 column
// tiles, so every XCD gets work).
__host__ __device__ inline int xcd_row_groups(int nN) { return nN >= 4 ? 2 : 8; }

// Upper bound of the tiles one XCD gets, for a bound of row tiles.
__host__ __device__ inline int tiles_per_xcd_bound(int row_tiles, int nN) {
  const int rx = xcd_row_groups(nN), cx = 8 / rx;
  return (nN + cx - 1) / cx * ((row_tiles + rx - 1) / rx + 1);
}

// Maps this workgroup onto (group, row tile, column tile).  Groups are the
// local experts (from the device offsets) followed by n_extra groups of
// extra_rows rows each (the shared experts, numbered from n_groups on; their
// rows count on from the last routed row), or, with offsets == nullptr, a
// single group of fixed_rows rows.  The row tiles form one list -- every
// group's full-height tiles in group order, then the short last tiles of 3, 2
// and 1 quarters, each kind in group order -- cut into bands of kBandRows row
// tiles.  The 8 XCDs (workgroup ids go round-robin over them, XCD x running
// ids x, x+8, ...) all work on the same band at a time: they form a grid of row groups x column groups over it, and XCD x
// takes its block of the band column by column.  An XCD thus holds a few
// weight column tiles across half the band's rows: a weight tile streams
// from memory once or twice per band, an activation row tile is shared by
// the few XCDs of its row group (the Infinity Cache serves the repeats), and
// within an XCD both operands are reused from L2.  The cheap short tiles come
// last, smallest at the very end, where the final round of tiles is only
// partly filled.
// Returns false for surplus workgroups.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int n_groups,
                                          int n_extra, int extra_rows, int fixed_rows, int BM,
                                          int nN, Tile& out) {
  const int lane = threadIdx.x & 63;
  const int n_all = n_groups + n_extra;
  // The offsets are read once, all at once: lane l holds group c*64 + l.
  int g0[kMaxGroupChunks], g1[kMaxGroupChunks];
  int n_full = 0, n_part[3] = {0, 0, 0};  // short last tiles of 3, 2, 1 quarters
  if (offsets != nullptr) {
    const int extra0 = n_extra > 0 ? offsets[n_groups] : 0;
#pragma unroll
    for (int c = 0; c < kMaxGroupChunks; ++c) {
      const int j = c * 64 + lane;
      g0[c] = g1[c] = 0;
      if (c * 64 < n_all && j < n_groups) {
        g0[c] = offsets[j];
        g1[c] = offsets[j + 1];
      } else if (c * 64 < n_all && j < n_all) {
        g0[c] = extra0 + (j - n_groups) * extra_rows;
        g1[c] = g0[c] + extra_rows;
      }
    }
#pragma unroll
    for (int c = 0; c < kMaxGroupChunks; ++c) {
      if (c * 64 >= n_all) break;
      int f, q;
      group_row_tiles(g1[c] - g0[c], BM, f, q);
      n_full += __shfl(wave_inclusive_sum(f), 63, 64);
#pragma unroll
      for (int p = 0; p < 3; ++p) n_part[p] += __shfl(wave_inclusive_sum(q == 3 - p ? 1 : 0), 63, 64);
    }
  } else {
    int q;
    group_row_tiles(fixed_rows, BM, n_full, q);
    if (q > 0) n_part[3 - q] = 1;
  }
  const int n_rt = n_full + n_part[0] + n_part[1] + n_part[2];
  const int xcd = blockIdx.x & 7;
  int slot = blockIdx.x >> 3;
  const int rx = xcd_row_groups(nN), cx = 8 / rx;
  const int rg = xcd / cx, cg = xcd % cx;
  const int c0 = cg * nN / cx, nc = (cg + 1) * nN / cx - c0;  // this XCD's columns
  const int full_bands = n_rt / kBandRows;
  int r0 = rg * kBandRows / rx, nr = (rg + 1) * kBandRows / rx - r0;  // its rows of a band
  const int per_full = nr * nc;
  int band;
  if (slot < full_bands * per_full) {
    band = slot / per_full;
    slot -= band * per_full;
  } else {
    slot -= full_bands * per_full;
    band = full_bands;
    const int rows_b = n_rt - full_bands * kBandRows;
    r0 = rg * rows_b / rx;
    nr = (rg + 1) * rows_b / rx - r0;
    if (slot >= nr * nc) return false;
  }
  const int n_tile = c0 + slot / nr;
  int rt = band * kBandRows + r0 + slot % nr;  // index in the row-tile list
  int row0 = 0, rows = fixed_rows, group = 0, m_tile = rt;
  if (offsets != nullptr) {
    // Full-height tiles: the rt-th in group order.  Short tiles of kind p (3 - p
    // quarters): the rt-th group, past the full tiles and the earlier kinds,
    // that has one; it is that group's last row tile.
    const bool is_short = rt >= n_full;
    int want = -1;  // quarters of the wanted short tile
    if (is_short) {
      rt -= n_full;
      int p = 0;
      while (p < 2 && rt >= n_part[p]) rt -= n_part[p++];
      want = 3 - p;
    }
    bool found = false;
#pragma unroll
    for (int c = 0; c < kMaxGroupChunks; ++c) {
      if (found || c * 64 >= n_all) break;
      int f, q;
      group_row_tiles(g1[c] - g0[c], BM, f, q);
      const int cnt = is_short ? (q == want ? 1 : 0) : f;
      const int incl = wave_inclusive_sum(cnt);
      const int chunk = __shfl(incl, 63, 64);
      if (rt < chunk) {
        const int L = __builtin_ctzll(__ballot(incl > rt));
        row0 = __shfl(g0[c], L, 64);
        rows = __shfl(g1[c], L, 64) - row0;
        group = c * 64 + L;
        m_tile = is_short ? __shfl(f, L, 64) : rt - __shfl(incl - cnt, L, 64);
        found = true;
      } else {
        rt -= chunk;
      }
    }
  }
  out.row0 = row0;
  out.rows = rows;
  out.group = group;
  out.m_tile = m_tile;
  out.n_tile = n_tile;
  return true;
}

// ------------------------------------------------------------------ bf16 MFMA GEMM

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWaves = 8;                                 // 2 x 4 wave grid, 2 waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWN = kWaves / 2;                           // waves along the columns
constexpr int kBF = kBN / kWN / 32;                       // B fragments (32 columns) per wave
constexpr int kRowBytes = kBK * 2;                        // bytes per staged row
constexpr int kChunks = kRowBytes / 16;                   // 16-byte chunks per row
constexpr int kSlotBytes = kBM * kRowBytes;               // one operand of one k-tile
// Ring slots per operand (160 KB of LDS in all).
constexpr int kAStages = 2, kBStages = 3;
constexpr int kDmaB = kSlotBytes / 1024 / kWaves;         // 1-KB loads per wave per operand
constexpr int kRowsPerDma = 1024 / kRowBytes;             // rows filled by one wave instruction
static_assert(kAStages * kSlotBytes + kBStages * kSlotBytes == 160 * 1024, "LDS budget");

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
// is logical chunk (l%8) ^ swz(row).  NA = A instructions per wave (one per
// 64 rows of the tile); B always takes 4 (rows 0..127 from b_lo, 128..255
// from b_hi).
template <int NA>
__device__ __forceinline__ void stage_a(uint8_t* slot, const uint8_t* a_tile,
                                        const uint32_t (&off)[2 * kDmaB], int wave,
                                        int kbytes) {
#pragma unroll
  for (int j = 0; j < NA; ++j)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(a_tile + kbytes + off[j]),
                                     (lds_ptr_t)(slot + (j * kWaves + wave) * 1024), 16, 0, 0);
}
__device__ __forceinline__ void stage_b(uint8_t* slot, const uint8_t* b_lo, const uint8_t* b_hi,
                                        const uint32_t (&off)[2 * kDmaB], int wave,
                                        int kbytes) {
#pragma unroll
  for (int j = 0; j < kDmaB; ++j)
    __builtin_amdgcn_global_load_lds(
        static_cast<const void*>((j < kDmaB / 2 ? b_lo : b_hi) + kbytes + off[kDmaB + j]),
        (lds_ptr_t)(slot + (j * kWaves + wave) * 1024), 16, 0, 0);
}

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
// output columns, which the epilogue stores 8 bytes at a time.
template <int NFA>
__device__ __forceinline__ void mma_step(const Frags& f, f32x16 (&acc)[4][kBF]) {
#pragma unroll
  for (int i = 0; i < NFA; ++i)
#pragma unroll
    for (int j = 0; j < kBF; ++j)
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

// One output tile of NFA * 64 rows: the 8 waves as 2 x 4, each NFA * 32 rows
// x 64 columns.  NFA = 4 for full tiles; 1..3 for the last row tile of an
// expert with at most 192 rows (that fraction of the A staging and of the
// MFMAs).  The k order of every output element is the same at every height.
template <int EPI, int NFA>
__device__ __forceinline__ void gemm_tile(const TileArgs& ta, uint8_t* lds) {
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
      const int br = EPI == EPI_SILU_GLU ? (r & (kNOut - 1)) : r;
      off[j] = (uint32_t)(min(br, b_last) * Kdim * 2 + lchunk * 16);
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
  constexpr int kVmPrologue = (kAStages - 1) * NA + (kBStages - 2) * kDmaB;
  constexpr int kVmBarrier = kDmaB;
  static_assert(kAStages == 2 && kBStages == 3 && kVmPrologue < 64, "vmcnt immediates");
  uint8_t* a_slots = lds;
  uint8_t* b_slots = lds + kAStages * kSlotBytes;
  const int nk = Kdim / kBK;
  const int last = (nk - 1) * kRowBytes;
#pragma unroll
  for (int t = 0; t < kMaxStages; ++t) {
    if (t < kAStages) stage_a<NA>(a_slots + t * kSlotBytes, a_tile, off, wave, min(t * kRowBytes, last));
    if (t < kBStages - 1)  // B2 comes in iteration 0
      stage_b(b_slots + t * kSlotBytes, b_lo, b_hi, off, wave, min(t * kRowBytes, last));
  }
  wait_loads_and_barrier<kVmPrologue>();  // tile 0 landed
  Frags f0, f1;
  load_frags<NFA>(a_slots, b_slots, 0, a_row0, b_row, xa, xb, f0);
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* sa = a_slots + (kt % kAStages) * kSlotBytes;
    uint8_t* sb = b_slots + (kt % kBStages) * kSlotBytes;
    const uint8_t* na = a_slots + ((kt + 1) % kAStages) * kSlotBytes;
    const uint8_t* nb = b_slots + ((kt + 1) % kBStages) * kSlotBytes;
    load_frags<NFA>(sa, sb, 1, a_row0, b_row, xa, xb, f1);
    stage_b(b_slots + ((kt + kBStages - 1) % kBStages) * kSlotBytes, b_lo, b_hi, off, wave,
            min((kt + kBStages - 1) * kRowBytes, last));
    mma_step<NFA>(f0, acc);
    pin_kstep_schedule<kMfma, kReads, kDmaB>();
    load_frags<NFA>(sa, sb, 2, a_row0, b_row, xa, xb, f0);
    mma_step<NFA>(f1, acc);
    pin_kstep_schedule<kMfma, kReads, 0>();
    load_frags<NFA>(sa, sb, 3, a_row0, b_row, xa, xb, f1);
    mma_step<NFA>(f0, acc);
    pin_kstep_schedule<kMfma, kReads, 0>();
    wait_loads_and_barrier<kVmBarrier>();  // tile kt+1 landed; tile kt's slots free
    load_frags<NFA>(na, nb, 0, a_row0, b_row, xa, xb, f0);
    stage_a<NA>(sa, a_tile, off, wave, min((kt + kAStages) * kRowBytes, last));
    mma_step<NFA>(f1, acc);
    pin_kstep_schedule<kMfma, kReads, NA>();
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
#pragma unroll
        for (int j = 0; j < kBF / 2; ++j) {
          const int n = n0 + wn * kWaveCols + j * 32 + g * 8 + col_l;
          if (n < N) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              v[q] = silu_f(acc[i][j][4 * g + q]) * acc[i][j + kBF / 2][4 * g + q];
            store_bf16x4(crow + n, v);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kBF; ++j) {
          const int n = n0 + wn * kWaveCols + j * 32 + g * 8 + col_l;
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
    const int32_t* __restrict__ offsets, int n_groups, int fixed_rows, int N, int Kdim,
    const uint16_t* __restrict__ A2, long long strideA2, const uint16_t* __restrict__ B2_0,
    const uint16_t* __restrict__ B2_1, long long strideB2, uint16_t* __restrict__ C2,
    long long strideC2, int n_extra, int extra_rows) {
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
    gemm_tile<EPI, 1>(ta, lds);
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
};

// Workgroups for an upper bound of row tiles: 8 XCDs x the most tiles one
// XCD can get.
inline int grid_for(int row_tiles, int col_tiles) {
  return 8 * tiles_per_xcd_bound(row_tiles, col_tiles);
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
                       g.strideC_batch, g.offsets, g.n_groups, g.fixed_rows, g.N, g.Kdim,
                       static_cast<const uint16_t*>(g.A2), g.strideA2,
                       static_cast<const uint16_t*>(g.B2_0), static_cast<const uint16_t*>(g.B2_1),
                       g.strideB2, static_cast<uint16_t*>(g.C2), g.strideC2, g.n_extra,
                       g.extra_rows);
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
  const int S = c.num_shared;
  // The shared experts run in the same launches as the routed ones, as extra
  // groups of T rows, so their tiles fill the routed launches' last rounds.
  const int row_bound = ceil_div(T * K, bm) + n_loc + S * ceil_div(T, bm);

  GemmArgs up{x_sorted, d, 0, w_gate, w_up, (long long)I * d, 0, h, I, 0,
              offsets, n_loc, 0, row_bound, I, d, 1,
              x, 0, ws_gate, ws_up, (long long)I * d, h_sh, (long long)T * I, S, T};
  hipError_t err = run_gemm<EPI_SILU_GLU>(c.dtype, up, s);
  if (err != hipSuccess) return err;
  GemmArgs down{h, I, 0, w_down, nullptr, (long long)d * I, 0, y_sorted, d, 0,
                offsets, n_loc, 0, row_bound, d, I, 1,
                h_sh, (long long)T * I, ws_down, nullptr, (long long)d * I, y_shared,
                (long long)T * d, S, T};
  return run_gemm<EPI_STORE>(c.dtype, down, s);
}

}  // namespace moe
