// Pieces shared by the grouped GEMMs of the expert MLP (bf16 and block-scaled
// fp8): the device-side tile list over ragged expert groups with its XCD-aware
// band order, and the 256 x 256-tile pipeline that stages 128-byte k-tile rows
// of both operands straight from global memory into swizzled LDS rings.
#pragma once

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

// Inclusive prefix sum over the 64 lanes, all in DPP moves (no LDS round
// trip): shifts of 1, 2, 4 and 8 lanes inside each row of 16 (lanes without a
// source add 0), then the last lane of rows 0 and 2 is added to rows 1 and 3
// (row_bcast:15) and the last lane of row 1 -- by then the sum of rows 0-1 --
// to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Value of lane L (uniform) of v, into a scalar register.
__device__ __forceinline__ int lane_value(int v, int L) { return __builtin_amdgcn_readlane(v, L); }

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
// ids x, x+8, ...) all work on the same band at a time: they form a grid of
// row groups x column groups over it, and XCD x takes its block of the band
// column by column.  An XCD thus holds a few
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
      n_full += lane_value(wave_inclusive_sum(f), 63);
#pragma unroll
      for (int p = 0; p < 3; ++p) n_part[p] += __popcll(__ballot(q == 3 - p));
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
      const int chunk = lane_value(incl, 63);
      if (rt < chunk) {
        const int L = __builtin_ctzll(__ballot(incl > rt));
        row0 = lane_value(g0[c], L);
        rows = lane_value(g1[c], L) - row0;
        group = c * 64 + L;
        m_tile = is_short ? lane_value(f, L) : rt - lane_value(incl - cnt, L);
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

// ------------------------------------------------------------------ MFMA tile pipeline

constexpr int kBM = 256, kBN = 256;
constexpr int kWaves = 8;                                 // 2 x 4 wave grid, 2 waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWN = kWaves / 2;                           // waves along the columns
constexpr int kBF = kBN / kWN / 32;                       // B fragments (32 columns) per wave
constexpr int kRowBytes = 128;                            // bytes per staged k-tile row
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

// LDS tile layout: 128-byte rows (64 bf16 or 128 fp8 of k) of 16-byte chunks; row
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

// Workgroups for an upper bound of row tiles: 8 XCDs x the most tiles one
// XCD can get.
inline int grid_for(int row_tiles, int col_tiles) {
  return 8 * tiles_per_xcd_bound(row_tiles, col_tiles);
}

}  // namespace
}  // namespace moe
