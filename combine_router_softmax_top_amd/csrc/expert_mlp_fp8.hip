// Grouped SiLU-gated expert MLP with a block-scaled 8-bit gate/up projection.
//
// Operation ("Efficient and portable mixture-of-experts communication",
// Dispatch: token payloads travel with block scaling factors into the grouped
// GEMM; Combine: expert outputs travel back unquantized, in 16 bits):
//     h = SiLU(Xq Gq^T) * (Xq Uq^T),   y = h W_down^T
// with Xq, Gq, Uq MX-FP8 matrices (E4M3 elements, one power-of-two scale per
// 32 consecutive k) and h, W_down, y in bf16.  Every product of two E4M3
// values and their two scales is exact in fp32, so the gate/up sums differ
// from those of the dequantized operands only by fp32 accumulation.
//
// Gate/up kernel (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3 with
// E8M0 scales, fp32 accumulation):
//   * one 256-thread workgroup per 256 x 256 tile (256 rows x 128 gate + 128
//     up columns, multiplied in the epilogue so h is written once); four
//     waves, one per SIMD, in a 2 x 2 grid, each 128 rows x (64 gate + 64 up)
//     as 4 x 4 MFMA blocks of 32 x 32, so each fragment read from LDS feeds
//     four MFMAs (the 32-byte fp8 fragments would not fit two waves per SIMD
//     in the register file); an expert's last row tile of at most 192 rows
//     runs at its rows rounded up to 64, as in the bf16 kernel;
//   * k-tiles of 128 (128-byte rows, the same bytes as the bf16 kernel's
//     64-deep tiles) go straight from global memory into swizzled LDS rings
//     of two slots per operand; a lane's operand for 64-deep k-step s is two
//     16-byte chunks of its row, 4s + h and 4s + 2 + h (h = lane / 32);
//   * the scales are stored pre-arranged for the MFMA (the MFMA scale layout
//     of moe_quantize_mxfp8) and reach LDS the same way, by 4-byte
//     global->LDS loads, a group of four k-tiles at a time into a
//     double-buffered area issued two k-tiles ahead; each lane then reads one
//     dword per fragment, whose bytes serve the group's k-steps through the
//     MFMA's op_sel (register loads mixed with the LDS loads made the
//     compiler wait for every load in flight before their first use);
//   * tile list, XCD band order and a fixed k order as in the bf16 kernel.
// The down projection runs either on bf16 h with the bf16 grouped GEMM, or,
// with MX-FP8 down weights, on h encoded in the gate/up epilogue (the
// dispatch's encoding rule, per 32 columns of a row) with this kernel's plain
// store variant (B tile = 256 rows of one weight matrix, y in bf16).
#include <type_traits>

#include "grouped_gemm.h"

namespace moe {

hipError_t launch_grouped_down_bf16(const moe_config_t& c, const void* h, const int32_t* offsets,
                                    const void* w_down, void* y_sorted, hipStream_t s,
                                    const void* h_sh, const void* ws_down, void* y_shared, int S);

namespace {

constexpr int kQWaves = 4;                            // 2 x 2, one wave per SIMD
constexpr int kQThreads = 64 * kQWaves;
constexpr int kQK = kRowBytes;                        // k per k-tile (one byte each)
constexpr int kQGroupTiles = 4;                       // k-tiles per scale load (512 k)
constexpr int kQBF = 4;                               // B fragments per wave: 2 gate + 2 up
constexpr int kQDmaB = kSlotBytes / 1024 / kQWaves;   // 1-KB loads per wave for a B k-tile
constexpr int kQNOut = kBN / 2;                       // h columns per tile

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct QFrags {
  i32x8 a[4], b[kQBF];
};

// A lane's 32-byte operand for k-step s: with base = row * 128 | (h ^
// swz(row)) * 16, logical chunk 4s + h (4s + 2 + h) sits at byte base ^ 64s
// (base ^ (64s + 32)) of the slot.
template <int S>
__device__ __forceinline__ i32x8 read_operand(const uint8_t* slot, uint32_t base) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(slot + (base ^ (64u * S)));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(slot + (base ^ (64u * S + 32u)));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Fragments of k-step S (64 deep) of a staged k-tile.  The per-fragment bases
// are passed through an empty asm first, so the compiler re-derives the four
// addresses of a fragment next to the reads (one xor each) instead of
// keeping every combination live in registers across the loop.
template <int NFA, int S>
__device__ __forceinline__ void load_qfrags(const uint8_t* sa, const uint8_t* sb,
                                            const uint32_t (&abase)[4],
                                            const uint32_t (&bbase)[kQBF], QFrags& f) {
#pragma unroll
  for (int i = 0; i < NFA; ++i) {
    uint32_t b = abase[i];
    asm volatile("" : "+v"(b));
    f.a[i] = read_operand<S>(sa, b);
  }
#pragma unroll
  for (int j = 0; j < kQBF; ++j) {
    uint32_t b = bbase[j];
    asm volatile("" : "+v"(b));
    f.b[j] = read_operand<S>(sb, b);
  }
}

// One 64-deep k-step: the weights are the MFMA's first operand (as in the
// bf16 kernel, so a lane keeps one output row), each operand with the scale
// register of its fragment; OPSEL picks the byte of that register that holds
// this lane's scale for this k-step.
template <int NFA, int OPSEL>
__device__ __forceinline__ void qmma_step(const QFrags& f, const uint32_t (&sca)[4],
                                          const uint32_t (&scb)[kQBF],
                                          f32x16 (&acc)[4][kQBF]) {
#pragma unroll
  for (int i = 0; i < NFA; ++i)
#pragma unroll
    for (int j = 0; j < kQBF; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.b[j], f.a[i], acc[i][j], 0, 0, OPSEL, (int)scb[j], OPSEL, (int)sca[i]);
}

// Staging with four waves: instruction j of wave w fills rows (4j + w) * 8 ..
// +8 of the slot; the per-lane source offsets come from `off`.
template <int N>
__device__ __forceinline__ void qstage(uint8_t* slot, const uint8_t* lo, const uint8_t* hi,
                                       int n_lo, const uint32_t* off, int wave, int kbytes) {
#pragma unroll
  for (int j = 0; j < N; ++j)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>((j < n_lo ? lo : hi) + kbytes + off[j]),
                                     (lds_ptr_t)(slot + (j * kQWaves + wave) * 1024), 16, 0, 0);
}

struct QTileArgs {
  const uint8_t* A;    // codes of the rows, pitch lda bytes
  const uint8_t* As;   // scales of A, MFMA layout over rows_as rows
  const uint8_t* Bg;   // weight codes of the group, [N, Kdim] (gate; up in Bu)
  const uint8_t* Bu;
  const uint8_t* Bgs;  // weight scales, MFMA layout over rows_bs rows (gate; up in Bus)
  const uint8_t* Bus;
  uint16_t* C;         // bf16 output, pitch ldc elements
  uint8_t* Cq;         // or MX-FP8 output codes (pitch ldc bytes) ...
  uint8_t* Cs;         // ... and scales, MFMA layout over rows_as rows
  long long rows_as, rows_bs;
  int lda, ldc, brow0;  // brow0: the group's first row in the weight stack
  int row0, rows, m0, n0, N, Kdim;
};

// LDS: activation and weight k-tiles in rings of two slots each, and the
// scales of two groups of four k-tiles, 4 KB per group and dword (region
// (b, d) holds dword d of the group in buffer b: 256 activation rows x 2
// halves, then 256 weight rows x 2 halves).
constexpr int kQStages = 2;
constexpr int kQScaleRegion = 4096;
// Scale regions: (group parity, dword) x 4, then 2 pad regions that take the
// last group's surplus scale loads (see the k-loop).
constexpr int kQLds = 2 * kQStages * kSlotBytes + 6 * kQScaleRegion;
static_assert(kQLds <= 160 * 1024, "LDS budget");

// EPI_SILU_GLU: B tile rows 0..127 gate, 128..255 the matching up rows, 128
// h columns out; EPI_STORE: 256 rows of one weight matrix, 256 columns out.
// QOUT (SiLU-GLU only): h leaves as MX-FP8 codes and MFMA-layout scales.
template <int EPI, bool QOUT, int NFA>
__device__ __forceinline__ void qgemm_tile(const QTileArgs& ta, uint8_t* lds) {
  constexpr bool kGlu = EPI == EPI_SILU_GLU;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int kWaveRows = NFA * 32;
  constexpr int NA = 2 * NFA;  // A loads per wave: NFA * 64 rows across the 4 waves
  const int m0 = ta.m0, n0 = ta.n0, N = ta.N, Kdim = ta.Kdim;

  const uint8_t* a_tile = ta.A + (long long)(ta.row0 + m0) * ta.lda;
  const uint8_t* b_lo = ta.Bg + (long long)n0 * Kdim;
  const uint8_t* b_hi = kGlu ? ta.Bu + (long long)n0 * Kdim : b_lo;
  const int a_last = ta.rows - 1 - m0;
  const int b_last = N - 1 - n0;
  // Per-lane source offsets; B instructions 4..7 fill tile rows 128..255, the
  // up rows 0..127.
  uint32_t offa[NA], offb[kQDmaB];
#pragma unroll
  for (int j = 0; j < kQDmaB; ++j) {
    const int r = (j * kQWaves + wave) * (1024 / kRowBytes) + lane / 8;
    const int lchunk = (lane & 7) ^ swz(r);
    if (j < NA) offa[j] = (uint32_t)(min(r, a_last) * ta.lda + lchunk * 16);
    const int br = (kGlu && j >= kQDmaB / 2) ? r - kQNOut : r;
    offb[j] = (uint32_t)(min(br, b_last) * Kdim + lchunk * 16);
  }

  // Fragment rows: A rows wm * kWaveRows + 32i + lane % 32; B rows: the wave's
  // 64 gate rows, then the matching 64 up rows (tile rows 128..).
  const int a_row0 = wm * kWaveRows + (lane & 31);
  uint32_t abase[4], bbase[kQBF];
#pragma unroll
  for (int j = 0; j < kQBF; ++j) {
    const int br = (j >> 1) * kQNOut + wn * 64 + (j & 1) * 32 + (lane & 31);
    bbase[j] = (uint32_t)(br * kRowBytes) | ((uint32_t)(h ^ swz(br)) << 4);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ar = a_row0 + i * 32;
    abase[i] = (uint32_t)(ar * kRowBytes) | ((uint32_t)(h ^ swz(ar)) << 4);
  }

  // Scales, MFMA layout: dword d of group g for row r, half h at dword
  // ((2g + d) R + r) 2 + h; byte 2(J % 2) + s of dword d = J / 2 serves k-step
  // s of k-tile J of the group.  A region load is four 64-lane dword DMAs per
  // wave: instruction q = wave + 4t (t = 0..3) fills dwords 64q .. 64q + 63 of
  // the region, activation rows 32q .. for q < 8, weight tile rows 32(q-8) ..
  // (gate rows, then up rows) after; rows past the group repeat its last row.
  // The host keeps every scale array below 2^31 dwords.
  const uint32_t* as32 = reinterpret_cast<const uint32_t*>(ta.As);
  const uint32_t* bgs32 = reinterpret_cast<const uint32_t*>(ta.Bgs);
  const uint32_t* bus32 = reinterpret_cast<const uint32_t*>(ta.Bus);
  uint32_t soff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int q = wave + 4 * t;
    const int r = (q & 7) * 32 + lane / 2;  // row of the A part or B tile row
    if (q < 8) {
      soff[t] = (uint32_t)(ta.row0 + min(m0 + r, ta.rows - 1)) * 2 + (lane & 1);
    } else {
      const int n = (kGlu && r >= kQNOut) ? r - kQNOut : r;
      soff[t] = (uint32_t)(ta.brow0 + min(n0 + n, N - 1)) * 2 + (lane & 1);
    }
  }
  const uint32_t a_gs = (uint32_t)ta.rows_as * 2, b_gs = (uint32_t)ta.rows_bs * 2;
  uint8_t* regions = lds + 2 * kQStages * kSlotBytes;
  // Dword d of group g into `region` (t = 0, 1: activations; 2, 3: weights;
  // waves 0..3 fill weight rows 0..127 (gate) for t = 2, 128..255 (up) for
  // t = 3).  Region (g % 2, d) holds the group's dword d.
  auto scale_region = [&](int g, int d) { return regions + ((g & 1) * 2 + d) * kQScaleRegion; };
  auto stage_scales = [&](int g, int d, uint8_t* region) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t* src = t < 2 ? as32 + (uint32_t)(2 * g + d) * a_gs
                                  : (t == 2 || !kGlu ? bgs32 : bus32) + (uint32_t)(2 * g + d) * b_gs;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + soff[t]),
                                       (lds_ptr_t)(region + (wave + 4 * t) * 256), 4, 0, 0);
    }
  };
  // This lane's scale dwords of one region: A fragment i at row a_row0 + 32i,
  // B fragment j at weight tile row (j / 2) * 128 + wn * 64 + (j % 2) * 32 + lane % 32.
  const uint32_t* rs_a = reinterpret_cast<const uint32_t*>(regions) + a_row0 * 2 + h;
  const uint32_t* rs_b =
      reinterpret_cast<const uint32_t*>(regions) + 512 + (wn * 64 + (lane & 31)) * 2 + h;
  auto read_scales = [&](int g, int d, uint32_t (&ra)[4], uint32_t (&rb)[kQBF]) {
    const int reg = ((g & 1) * 2 + d) * (kQScaleRegion / 4);
#pragma unroll
    for (int i = 0; i < NFA; ++i) ra[i] = rs_a[reg + i * 64];
#pragma unroll
    for (int j = 0; j < kQBF; ++j) rb[j] = rs_b[reg + (j >> 1) * 256 + (j & 1) * 64];
  };

  f32x16 acc[4][kQBF];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kQBF; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Pipeline: both operands in rings of two; A(kt+2) and B(kt+2) are issued
  // after barrier kt into tile kt's slots and must land by barrier kt+1, one
  // k-tile later.  Fragments are double-buffered across the two k-steps; the
  // barrier comes before the second k-step's MFMAs.  Scales: both dwords of
  // group g+1 are loaded after barrier 0 of group g, after that k-tile's tile
  // loads, into the buffer group g-1 used (its last read, dword 1, preceded
  // barrier 2 of group g-1).  Loads complete in issue order, so barrier 1 of
  // the group waits for everything but those 8 youngest loads, and barrier 2
  // (which waits for barrier 1's k-tile loads) for them too: the scale loads
  // get two k-tiles, which matters, as they miss the caches more often than
  // the tiles.  Dword 0 of group g+1 is read into registers after barrier 3
  // of group g, dword 1 after barrier 1 of group g+1.
  constexpr int kMfma = NFA * kQBF, kReads = 2 * (NFA + kQBF);
  constexpr int kVmPrologue = NA + kQDmaB;  // tile 1 still in flight
  constexpr int kScaleDma = 8;               // scale loads per wave for one group
  uint8_t* a_slots = lds;
  uint8_t* b_slots = lds + kQStages * kSlotBytes;
  const int nk = Kdim / kQK;  // a multiple of kQGroupTiles
  const int ng = nk / kQGroupTiles;
  const int last = (nk - 1) * kRowBytes;
  stage_scales(0, 0, scale_region(0, 0));
  stage_scales(0, 1, scale_region(0, 1));
#pragma unroll
  for (int t = 0; t < kQStages; ++t) {
    qstage<NA>(a_slots + t * kSlotBytes, a_tile, a_tile, NA, offa, wave, min(t * kRowBytes, last));
    qstage<kQDmaB>(b_slots + t * kSlotBytes, b_lo, b_hi, kQDmaB / 2, offb, wave,
                   min(t * kRowBytes, last));
  }
  wait_loads_and_barrier<kVmPrologue>();  // tile 0 and region 0 landed
  QFrags f0, f1;
  uint32_t sca[4], scb[kQBF];  // the current k-tile pair's scale dwords
#pragma unroll
  for (int i = NFA; i < 4; ++i) sca[i] = 0u;
  read_scales(0, 0, sca, scb);
  load_qfrags<NFA, 0>(a_slots, b_slots, abase, bbase, f0);

  // There is at least one group (Kdim >= 512).  Telling the compiler so in
  // the plain-store variant removes the zero-trip path that kept its zeroed
  // accumulators alive across the loop (246 registers spilled); the SiLU
  // variant allocates better without it.
  if constexpr (!kGlu) __builtin_assume(ng > 0);
  for (int g = 0; g < ng; ++g) {
    auto ktile = [&](auto Jc) {
      constexpr int J = decltype(Jc)::value;
      const int kt = g * kQGroupTiles + J;
      uint8_t* sa = a_slots + (kt & 1) * kSlotBytes;
      uint8_t* sb = b_slots + (kt & 1) * kSlotBytes;
      const uint8_t* na = a_slots + ((kt + 1) & 1) * kSlotBytes;
      const uint8_t* nb = b_slots + ((kt + 1) & 1) * kSlotBytes;
      load_qfrags<NFA, 1>(sa, sb, abase, bbase, f1);
      qmma_step<NFA, 2 * (J % 2)>(f0, sca, scb, acc);
      pin_kstep_schedule<kMfma, kReads, 0>();
      // Tile kt+1 landed (and, at J = 2, the scales of group g+1).
      wait_loads_and_barrier<J == 1 ? kScaleDma : 0>();
      load_qfrags<NFA, 0>(na, nb, abase, bbase, f0);
      const int kb = min((kt + kQStages) * kRowBytes, last);
      qstage<NA>(sa, a_tile, a_tile, NA, offa, wave, kb);
      qstage<kQDmaB>(sb, b_lo, b_hi, kQDmaB / 2, offb, wave, kb);
      if constexpr (J == 0) {
        // Group g+1's scales into the regions group g-1 used.  The last group
        // has no successor: it issues the same loads (so the counts the
        // barrier waits assume hold in every group) from its own scales into
        // the two pad regions, which nothing reads; no load ever writes a
        // region that is being read.
        const bool more = g + 1 < ng;
        const int gs = more ? g + 1 : g;
        stage_scales(gs, 0, more ? scale_region(gs, 0) : regions + 4 * kQScaleRegion);
        stage_scales(gs, 1, more ? scale_region(gs, 1) : regions + 5 * kQScaleRegion);
      }
      qmma_step<NFA, 2 * (J % 2) + 1>(f1, sca, scb, acc);
      // After the last MFMA of the pair that uses them, the scale registers
      // take the next pair's dwords.
      if constexpr (J == 1) read_scales(g, 1, sca, scb);
      if constexpr (J == 3) read_scales(g + 1, 0, sca, scb);
      constexpr int kScaleReads = (J == 1 || J == 3) ? NFA + kQBF : 0;
      pin_kstep_schedule<kMfma, kReads + kScaleReads, NA + kQDmaB + (J == 0 ? kScaleDma : 0)>();
    };
    ktile(std::integral_constant<int, 0>{});
    ktile(std::integral_constant<int, 1>{});
    ktile(std::integral_constant<int, 2>{});
    ktile(std::integral_constant<int, 3>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: element r of lane l in a 32 x 32 block is output row l % 32 and
  // column (r / 4) * 8 + (l / 32) * 4 + r % 4; gate block j pairs with up
  // block j + 2.  N is a multiple of 64, so a run of four (or eight) columns is
  // wholly inside or wholly past N.
  const int row_l = lane & 31;
  const int col_l = h * 4;
  if constexpr (QOUT) {
    // The codes go through LDS as below (row pitch 144 bytes); the scale bytes
    // straight to memory.
    constexpr int kPitchQ = kQNOut + 16;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NFA; ++i) {
      const int r = wm * kWaveRows + i * 32 + row_l;
      const int m = m0 + r;
      if (m >= ta.rows) continue;  // lanes l and l ^ 32 share the row
      const long long row = ta.row0 + m;
      // A 32-column block of h is one row of a 32 x 32 MFMA block, 16 values
      // in each of lanes l and l ^ 32: its MX-FP8 scale from their common
      // maximum (the encoding rule of the dispatch), 16 codes per lane written
      // as 4 dwords, the scale byte by the h = 0 lane.  I is a multiple of
      // 512, so every block is whole.
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nb = n0 + wn * 64 + j * 32;  // first column of the block
        float v[16];
        float mx = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          v[q] = silu_f(acc[i][j][q]) * acc[i][j + 2][q];
          mx = fmaxf(mx, fabsf(v[q]));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const int ef = (int)((__float_as_uint(mx) >> 23) & 0xff);
        const int sc = min(127, max(-127, ef - 127 - 8));
        const float inv = __uint_as_float((uint32_t)(127 - sc) << 23);
        uint8_t* lrow = lds + r * kPitchQ + (nb - n0);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float e[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = fminf(448.f, fmaxf(-448.f, v[4 * gq + q] * inv));
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
          *reinterpret_cast<uint32_t*>(lrow + gq * 8 + col_l) = (uint32_t)w;
        }
        if (col_l == 0) {
          const int qb = nb / 32, g = qb >> 4, mm = qb & 15;
          const int d = mm >> 3, b = ((mm >> 2) & 1) * 2 + ((mm >> 1) & 1), hh = mm & 1;
          ta.Cs[(((long long)(2 * g + d) * ta.rows_as + row) * 2 + hh) * 4 + b] =
              (uint8_t)(sc + 127);
        }
      }
    }
    __syncthreads();
    // 16 bytes per lane, 8 lanes per 128-byte row of codes.
    constexpr int kRowsPerPass = kQThreads / 8;
    constexpr int kTileRows = NFA * 64;
    static_assert(kTileRows % kRowsPerPass == 0, "whole passes");
    const int piece = tid % 8;
#pragma unroll
    for (int r = tid / 8; r < kTileRows; r += kRowsPerPass) {
      const int m = m0 + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * kPitchQ + piece * 16);
      if (m < ta.rows)
        *reinterpret_cast<u32x4*>(ta.Cq + (long long)(ta.row0 + m) * ta.ldc + n0 + piece * 16) = v;
    }
  } else {
    // bf16 out, through LDS: four adjacent values per (lane, r / 4) go into a
    // row-major copy of the tile (row pitch padded by 16 bytes), then each
    // lane moves 16 bytes of a row to memory, a wave covering whole rows.
    // The barrier first waits for every wave's loads and fragment reads.
    constexpr int kNOut = kGlu ? kQNOut : kBN;
    constexpr int kOutBytes = kNOut * 2;
    constexpr int kPitch = kOutBytes + 16;
    static_assert(kBM * kPitch <= kQLds, "output tile fits the rings");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NFA; ++i) {
      uint16_t* lrow = reinterpret_cast<uint16_t*>(lds + (wm * kWaveRows + i * 32 + row_l) * kPitch);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int j = 0; j < (kGlu ? 2 : kQBF); ++j) {
          const int c = (j >> 1) * 128 + wn * 64 + (j & 1) * 32 + gq * 8 + col_l;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            v[q] = kGlu ? silu_f(acc[i][j][4 * gq + q]) * acc[i][j + 2][4 * gq + q]
                        : acc[i][j][4 * gq + q];
          store_bf16x4(lrow + c, v);
        }
    }
    __syncthreads();
    constexpr int kLanesPerRow = kOutBytes / 16;
    constexpr int kRowsPerPass = kQThreads / kLanesPerRow;
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
}

// Groups: the local experts (rows from the offsets), then n_extra extra
// groups of extra_rows rows each with operands of their own (the shared
// experts: A2 + e * strideA2 rows from 0, B2 stacks, C2 + e * strideC2).
struct QExtra {
  const uint8_t* A;   // codes, advanced by e * strideA per group
  const uint8_t* As;  // scales (MFMA layout over rows_as rows), + e * strideAs
  long long strideA, strideAs, rows_as;
  const uint8_t* Bg;  // weight codes [n_extra, N, Kdim] (gate; up in Bu)
  const uint8_t* Bu;
  const uint8_t* Bgs;  // scales of the [n_extra * N, Kdim] stacks
  const uint8_t* Bus;
  long long strideB, rows_bs;
  uint16_t* C;        // bf16 output (or Cq / Cs), + e * strideC elements or bytes
  uint8_t* Cq;
  uint8_t* Cs;
  long long strideC, strideCs;
  int n_extra, extra_rows;
};

template <int EPI, bool QOUT>
__global__ __launch_bounds__(kQThreads, 1) void gemm_mxfp8_kernel(
    const uint8_t* __restrict__ A, int lda, const uint8_t* __restrict__ As, long long rows_as,
    const uint8_t* __restrict__ Bg, const uint8_t* __restrict__ Bu, long long strideB_group,
    const uint8_t* __restrict__ Bgs, const uint8_t* __restrict__ Bus, long long rows_bs,
    uint16_t* __restrict__ C, uint8_t* __restrict__ Cq, uint8_t* __restrict__ Cs, int ldc,
    const int32_t* __restrict__ offsets, int n_groups, int N, int Kdim, QExtra ex) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kQLds];
  constexpr int kNOut = EPI == EPI_SILU_GLU ? kQNOut : kBN;  // output columns per tile
  const int nN = (N + kNOut - 1) / kNOut;
  Tile tl;
  if (!find_tile(offsets, n_groups, ex.n_extra, ex.extra_rows, 0, kBM, nN, tl)) return;
  QTileArgs ta;
  if (tl.group < n_groups) {
    ta.A = A;
    ta.As = As;
    ta.rows_as = rows_as;
    ta.Bg = Bg + (long long)tl.group * strideB_group;
    ta.Bu = Bu + (long long)tl.group * strideB_group;
    ta.Bgs = Bgs;
    ta.Bus = Bus;
    ta.rows_bs = rows_bs;
    ta.brow0 = tl.group * N;
    ta.C = C;
    ta.Cq = Cq;
    ta.Cs = Cs;
    ta.row0 = tl.row0;
  } else {  // an extra group: its own operands, rows from 0
    const int e = tl.group - n_groups;
    ta.A = ex.A + (long long)e * ex.strideA;
    ta.As = ex.As + (long long)e * ex.strideAs;
    ta.rows_as = ex.rows_as;
    ta.Bg = ex.Bg + (long long)e * ex.strideB;
    ta.Bu = ex.Bu + (long long)e * ex.strideB;
    ta.Bgs = ex.Bgs;
    ta.Bus = ex.Bus;
    ta.rows_bs = ex.rows_bs;
    ta.brow0 = e * N;
    ta.C = ex.C ? ex.C + (long long)e * ex.strideC : nullptr;
    ta.Cq = ex.Cq ? ex.Cq + (long long)e * ex.strideC : nullptr;
    ta.Cs = ex.Cs ? ex.Cs + (long long)e * ex.strideCs : nullptr;
    ta.row0 = 0;
  }
  ta.lda = lda;
  ta.ldc = ldc;
  ta.rows = tl.rows;
  ta.m0 = tl.m_tile * kBM;
  ta.n0 = tl.n_tile * kNOut;
  ta.N = N;
  ta.Kdim = Kdim;
  const int left = tl.rows - ta.m0;
  if (left > 3 * kBM / 4)
    qgemm_tile<EPI, QOUT, 4>(ta, lds);
  else if (left > kBM / 2)
    qgemm_tile<EPI, QOUT, 3>(ta, lds);
  else if (left > kBM / 4)
    qgemm_tile<EPI, QOUT, 2>(ta, lds);
  else
    qgemm_tile<EPI, QOUT, 1>(ta, lds);
}

}  // namespace

hipError_t launch_expert_mlp_mxfp8(const moe_config_t& c, const uint8_t* xq, const uint8_t* xq_scales,
                                   const int32_t* offsets, const uint8_t* wq_gate,
                                   const uint8_t* wq_gate_scales, const uint8_t* wq_up,
                                   const uint8_t* wq_up_scales, const void* w_down,
                                   const uint8_t* wq_down, const uint8_t* wq_down_scales,
                                   void* y_sorted, void* workspace, hipStream_t s,
                                   const MxfpShared* sh) {
  const int T = c.num_tokens, K = c.top_k, d = c.hidden, I = c.intermediate;
  const int n_loc = c.expert_end - c.expert_begin;
  const int S = sh ? c.num_shared : 0;
  const int row_bound = ceil_div(T * K, kBM) + n_loc + S * ceil_div(T, kBM);
  const long long rows = (long long)T * K;
  // Workspace: h of the routed rows, then of the shared experts ([S, T, I]):
  // bf16, or MX-FP8 codes followed by their scales (per shared expert a
  // [T, I] matrix with its own MFMA layout).
  const size_t h_bytes = align_up((size_t)T * K * I * 2, 256);
  char* ws = static_cast<char*>(workspace);
  const bool fp8_down = wq_down != nullptr;
  QExtra up{};
  up.n_extra = S;
  up.extra_rows = T;
  if (S > 0) {
    up.A = sh->xq;
    up.As = sh->xq_scales;
    up.rows_as = T;
    up.Bg = sh->wq_gate;
    up.Bu = sh->wq_up;
    up.Bgs = sh->wq_gate_scales;
    up.Bus = sh->wq_up_scales;
    up.strideB = (long long)I * d;
    up.rows_bs = (long long)S * I;
    up.strideC = (long long)T * I;
    up.strideCs = (long long)T * I / 32;
  }
  char* hsh = ws + h_bytes;
  if (!fp8_down) {  // gate/up in fp8, h and the down projection in bf16
    uint16_t* h = reinterpret_cast<uint16_t*>(ws);
    if (S > 0) up.C = reinterpret_cast<uint16_t*>(hsh);
    hipLaunchKernelGGL((gemm_mxfp8_kernel<EPI_SILU_GLU, false>),
                       dim3(grid_for(row_bound, ceil_div(I, kQNOut))), dim3(kQThreads), 0, s, xq,
                       d, xq_scales, rows, wq_gate, wq_up, (long long)I * d, wq_gate_scales,
                       wq_up_scales, (long long)n_loc * I, h, nullptr, nullptr, I, offsets, n_loc,
                       I, d, up);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_grouped_down_bf16(c, h, offsets, w_down, y_sorted, s, S > 0 ? hsh : nullptr,
                                    S > 0 ? sh->w_down : nullptr, S > 0 ? sh->y : nullptr, S);
  }
  // Both projections in fp8: h leaves the gate/up kernel as MX-FP8 codes
  // [T*K, I] and MFMA-layout scales (T*K rows), the down kernel's A operand.
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws);
  uint8_t* hs = hq + align_up((size_t)T * K * I, 256);
  uint8_t* hshq = reinterpret_cast<uint8_t*>(hsh);
  uint8_t* hshs = hshq + align_up((size_t)S * T * I, 256);
  if (S > 0) {
    up.Cq = hshq;
    up.Cs = hshs;
  }
  hipLaunchKernelGGL((gemm_mxfp8_kernel<EPI_SILU_GLU, true>),
                     dim3(grid_for(row_bound, ceil_div(I, kQNOut))), dim3(kQThreads), 0, s, xq, d,
                     xq_scales, rows, wq_gate, wq_up, (long long)I * d, wq_gate_scales,
                     wq_up_scales, (long long)n_loc * I, nullptr, hq, hs, I, offsets, n_loc, I, d,
                     up);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  QExtra dn{};
  dn.n_extra = S;
  dn.extra_rows = T;
  if (S > 0) {
    dn.A = hshq;
    dn.As = hshs;
    dn.strideA = (long long)T * I;
    dn.strideAs = (long long)T * I / 32;
    dn.rows_as = T;
    dn.Bg = dn.Bu = sh->wq_down;
    dn.Bgs = dn.Bus = sh->wq_down_scales;
    dn.strideB = (long long)d * I;
    dn.rows_bs = (long long)S * d;
    dn.C = static_cast<uint16_t*>(sh->y);
    dn.strideC = (long long)T * d;
  }
  hipLaunchKernelGGL((gemm_mxfp8_kernel<EPI_STORE, false>),
                     dim3(grid_for(row_bound, ceil_div(d, kBN))), dim3(kQThreads), 0, s, hq, I, hs,
                     rows, wq_down, wq_down, (long long)d * I, wq_down_scales, wq_down_scales,
                     (long long)n_loc * d, static_cast<uint16_t*>(y_sorted), nullptr, nullptr, d,
                     offsets, n_loc, d, I, dn);
  return hipGetLastError();
}

}  // namespace moe
