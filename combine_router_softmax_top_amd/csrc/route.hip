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
// 64 tokens x up to 256 experts x one slice of the reduction dimension, its
// operands streamed through a four-slot LDS ring (each chunk loaded three
// chunks ahead), then a selection kernel that adds the slices in a fixed
// order (deterministic).
// fp32: each wave takes one token and reduces every dot product across its 64
// lanes with a butterfly.
// Selection: one wave per token, the partial slices read as 16-byte pieces (4
// adjacent experts per lane), K rounds of an arg-max ordered by (logit desc,
// expert id asc): the largest logit by a DPP reduction into lane 63 read back
// as a scalar, the lowest id holding it by a ballot.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokTile = 4;  // fp32 router: tokens per workgroup, one per wave

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Butterfly sum: every lane ends with the same bits (fp addition is commutative).
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Selection keys: (logit, expert) packed so that a larger key is a larger
// logit, and among equal logits the lower expert id.  The high word is the
// logit's bit pattern made order-preserving as an unsigned integer (flip all
// bits of a negative, the sign bit of a non-negative); the low word is ~id.
__device__ __forceinline__ unsigned long long sel_key(float v, int e) {
  const uint32_t u = __float_as_uint(v) == 0x80000000u ? 0u : __float_as_uint(v);  // -0 == +0
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ float key_value(unsigned long long k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(unsigned long long k) { return (int)~(uint32_t)k; }

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max(unsigned long long k) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xf, 0xf, false);
  const unsigned long long o = ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
  return o > k ? o : k;
}
__device__ __forceinline__ unsigned long long xor_max(unsigned long long k, int off) {
  const int lo = __shfl_xor((int)(uint32_t)k, off);
  const int hi = __shfl_xor((int)(uint32_t)(k >> 32), off);
  const unsigned long long o = ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
  return o > k ? o : k;
}

// Largest key of the wave, in every lane: within each row of 16 lanes by DPP
// (swap neighbours, swap pairs, rotate by 4, rotate by 8), then across rows.
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
  k = dpp_max<0xB1>(k);   // quad_perm [1,0,3,2]
  k = dpp_max<0x4E>(k);   // quad_perm [2,3,0,1]
  k = dpp_max<0x124>(k);  // row_ror 4
  k = dpp_max<0x128>(k);  // row_ror 8
  k = xor_max(k, 16);
  return xor_max(k, 32);
}

// Score of a selected logit z: softmax numerator exp(z - m) (m the largest
// logit), or sigmoid.  Renormalised sigmoid weights are ratios of scores.
// When the first (largest) selected logit is at most -17 they are taken from
// exp(z - first): there sigmoid(z) = e^z (1 + O(e^z)), so the ratios agree to
// a relative 4e-8, where the plain scores would lose about 1e-6 near -50 (an
// exponential of a large fp32 argument) and underflow to 0 below about -88
// (0/0 when every selected one does).  Above -17 the plain scores lose less
// than 7e-7, and a selected logit whose score underflows weighs less than
// e^-71 against the first.
__device__ __forceinline__ float score_of(float z, int score, int renorm, float m, float first) {
  if (score != MOE_SCORE_SIGMOID) return __expf(z - m);
  if (renorm && first <= -17.f) return __expf(z - first);
  return 1.f / (1.f + __expf(-z));
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
  // Candidate keys; experts past E and already chosen ones hold key 0, below
  // every real key.
  unsigned long long kv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    kv[i] = e < E ? sel_key(v[i], e) : 0ull;
  }
  int my_e = 0;
  float my_s = 0.f, sum_sel = 0.f, first = 0.f;
  for (int k = 0; k < K; ++k) {
    unsigned long long best = kv[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) best = kv[i] > best ? kv[i] : best;
    best = wave_max_key(best);
    const int be = key_expert(best);
    const float bv = key_value(best);
    if ((be & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i == (be >> 6)) kv[i] = 0ull;
    }
    if (k == 0) first = bv;
    const float sc = score_of(bv, score, renorm, m, first);
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

// route_logits_kernel<NT>: workgroup = 64 tokens x NT*16 experts x one slice
// of the reduction dimension, 4 waves.  With NT >= 4 each wave owns all 64
// tokens and a quarter of the experts; with fewer expert blocks each wave
// owns 16 tokens and all the experts.  Token rows and router rows move in
// 64-deep chunks straight from global memory into LDS (global_load_lds) in a
// ring of 4 slots: right after the barrier that ends the reads of chunk c its
// slot takes chunk c+4, so each load has three chunks of MFMA work to land.
// 16x16x32 bf16 MFMAs, fp32 accumulation.  Partial logits of slice s go to
// part[s][t][e] (fp32); the select kernel adds the slices in ascending s.
// The number of slices depends only on d and E, never on the token count, so
// a token's logits do not depend on how the batch is split.
constexpr int kRtTok = 64, kRtKc = 64, kRtStages = 4;

// LDS rows of 128 B (64 bf16): logical 16-byte chunk c of row r sits in slot
// c ^ rsw(r); 16 lanes reading rows r..r+15 at one logical chunk then touch
// distinct slots in every 256-byte window (no bank conflicts).
__device__ __forceinline__ int rsw(int r) { return (r ^ (r >> 3)) & 7; }

typedef __attribute__((address_space(3))) void* rt_lds_ptr_t;

// Router-tile schedule of one 32-deep k-step: NM MFMAs, the ND fragment
// reads of the next k-step two after each of the first MFMAs, and NV
// global->LDS loads spread over the rest.
template <int NM, int ND, int NV, int I = 0>
__device__ __forceinline__ void rt_pin_schedule() {
  constexpr int kWithReads = (ND + 1) / 2;
  if constexpr (NM < kWithReads + 1) {
    __builtin_amdgcn_sched_barrier(0);
  } else if constexpr (I == NM) {
    __builtin_amdgcn_sched_barrier(0);
  } else {
    constexpr int kRest = NM - kWithReads;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (I < kWithReads) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * I + 2 <= ND ? 2 : 1, 0);  // DS read
    } else if constexpr (NV > 0) {
      constexpr int j = I - kWithReads;
      constexpr int n = NV * (j + 1) / kRest - NV * j / kRest;
      if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x020, n, 0);  // VMEM
    }
    rt_pin_schedule<NM, ND, NV, I + 1>();
  }
}

template <int VM>
__device__ __forceinline__ void rt_wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(VM) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup -> (token tile, expert tile, slice): workgroup ids go round-robin
// over the 8 XCDs; XCD x works on slice x % ks only (ks divides 8), so its L2
// holds one slice of the router matrix while the token rows stream through.
template <int NT>
__global__ __launch_bounds__(256, 1) void route_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    int e_pad, int k_slice, int ks, int n_tok_tiles, float* __restrict__ part) {
  constexpr int NE = NT * 16;
  constexpr int kBRows = NE < 32 ? 32 : NE;          // staged router rows (>= one load per wave)
  constexpr int kSlotA = kRtTok * 128;                 // 8 KB
  constexpr int kSlotB = kBRows * 128;
  constexpr int kStage = kSlotA + kSlotB;
  constexpr int NA = kSlotA / 1024 / 4;                // 2 loads per wave
  constexpr int NB = kSlotB / 1024 / 4;                // 1..8 loads per wave
  constexpr int AF = NT >= 4 ? 4 : 1;                  // token fragments per wave
  constexpr int BF = NT >= 4 ? NT / 4 : NT;            // expert fragments per wave
  constexpr int kLoads = NA + NB;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kRtStages * kStage];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int xcd = blockIdx.x & 7, per = 8 / ks;
  const int z = xcd % ks;
  const int pair = xcd / ks + per * (blockIdx.x >> 3);  // (token tile, expert tile)
  const int n_exp_tiles = e_pad / NE;
  if (pair >= n_tok_tiles * n_exp_tiles) return;
  const int t0 = (pair % n_tok_tiles) * kRtTok;
  const int e0 = (pair / n_tok_tiles) * NE;
  const int k0 = z * k_slice;
  const int tok0 = NT >= 4 ? 0 : wave * 16;
  const int exp0 = NT >= 4 ? wave * BF * 16 : 0;

  // Load j of wave w fills rows (4j + w)*8 .. +8 of a slot; lane l covers row
  // +l/8, physical chunk l%8, whose source is logical chunk (l%8) ^ rsw(row).
  // Rows past the last token / expert repeat it.
  const uint8_t* xa = reinterpret_cast<const uint8_t*>(x + (size_t)t0 * d + k0);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(wr + (size_t)e0 * d + k0);
  uint32_t offa[NA], offb[NB];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = (j * 4 + wave) * 8 + lane / 8;
    offa[j] = (uint32_t)(min(r, T - 1 - t0) * d * 2 + (((lane & 7) ^ rsw(r)) << 4));
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r = (j * 4 + wave) * 8 + lane / 8;
    offb[j] = (uint32_t)(min(r, E - 1 - e0) * d * 2 + (((lane & 7) ^ rsw(r)) << 4));
  }
  auto stage = [&](int slot, int kbytes) {
    uint8_t* sa = lds + slot * kStage;
    uint8_t* sb = sa + kSlotA;
    const uint8_t* xs = xa + kbytes;  // uniform base, per-lane 32-bit offsets
    const uint8_t* ws = wb + kbytes;
#pragma unroll
    for (int j = 0; j < NA; ++j)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(xs + offa[j]),
                                       (rt_lds_ptr_t)(sa + (j * 4 + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(ws + offb[j]),
                                       (rt_lds_ptr_t)(sb + (j * 4 + wave) * 1024), 16, 0, 0);
  };

  // Fragments of 32-deep k-step ks (0, 1) of a chunk: lane l reads row
  // base + l%16 at logical chunk 4 ks + l/16.
  // Per-lane byte offsets of the fragments in a slot for k-step 0; k-step 1
  // reads logical chunk +4, i.e. the offset ^ 64 (the chunk's bit 2).
  const int kg = lane >> 4;
  int fa[AF], fb[BF];
#pragma unroll
  for (int i = 0; i < AF; ++i) {
    const int r = tok0 + i * 16 + (lane & 15);
    fa[i] = r * 128 + ((kg ^ rsw(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < BF; ++j) {
    const int r = exp0 + j * 16 + (lane & 15);
    fb[j] = kSlotA + r * 128 + ((kg ^ rsw(r)) << 4);
  }
  struct RFrags {
    bf16x8 a[AF], b[BF];
  };
  auto frags = [&](int slot, int ks, RFrags& f) {
    const uint8_t* st = lds + slot * kStage;
    const int x = ks * 64;
#pragma unroll
    for (int i = 0; i < AF; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(st + (fa[i] ^ x));
#pragma unroll
    for (int j = 0; j < BF; ++j) f.b[j] = *reinterpret_cast<const bf16x8*>(st + (fb[j] ^ x));
  };
  f32x4 acc[AF][BF];
#pragma unroll
  for (int i = 0; i < AF; ++i)
#pragma unroll
    for (int j = 0; j < BF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const RFrags& f) {
#pragma unroll
    for (int i = 0; i < AF; ++i)
#pragma unroll
      for (int j = 0; j < BF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  const int nkc = k_slice / kRtKc;
  const int last = (nkc - 1) * kRtKc * 2;
#pragma unroll
  for (int t = 0; t < kRtStages; ++t) stage(t, min(t * kRtKc * 2, last));
  rt_wait_and_barrier<(kRtStages - 1) * kLoads>();  // chunk 0 landed
  RFrags f0, f1;
  frags(0, 0, f0);
  for (int kc = 0; kc < nkc; ++kc) {
    const int slot = kc % kRtStages;
    frags(slot, 1, f1);
    mma(f0);
    rt_pin_schedule<AF * BF, AF + BF, 0>();
    rt_wait_and_barrier<(kRtStages - 2) * kLoads>();  // chunk kc+1 landed; slot free
    frags((kc + 1) % kRtStages, 0, f0);
    stage(slot, min((kc + kRtStages) * kRtKc * 2, last));
    mma(f1);
    rt_pin_schedule<AF * BF, AF + BF, kLoads>();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane holds tokens (lane/16)*4 + r and expert lane%16 of each 16 x 16
  // block; experts past E hold sums of a repeated row and are never read.
  float* out = part + (size_t)z * T * e_pad;
#pragma unroll
  for (int i = 0; i < AF; ++i)
#pragma unroll
    for (int j = 0; j < BF; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + tok0 + i * 16 + (lane >> 4) * 4 + r;
        if (t < T) out[(size_t)t * e_pad + e0 + exp0 + j * 16 + (lane & 15)] = acc[i][j][r];
      }
}

// The larger of v and the value DPP control CTRL moves into this lane (lanes
// outside ROWS keep their own value); no NaN handling, the values are finite
// or -inf.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_fmax(float v) {
  const int b = __float_as_int(v);
  // A pattern that writes every lane needs no old value.
  const float o = __int_as_float(ROWS == 0xf ? __builtin_amdgcn_update_dpp(0, b, CTRL, ROWS, 0xf, false)
                                             : __builtin_amdgcn_update_dpp(b, b, CTRL, ROWS, 0xf, false));
  return o > v ? o : v;
}

// Largest value of the wave as a scalar: within each row
// of 16 lanes (swap neighbours, swap pairs, rotate by 4, rotate by 8), then
// row 1 and row 3 take lane 15 of the row below (row_bcast:15) and rows 2 and
// 3 take lane 31 (row_bcast:31), which leaves the maximum in lane 63.
__device__ __forceinline__ float wave_fmax_uniform(float v) {
  v = dpp_fmax<0xB1>(v);       // quad_perm [1,0,3,2]
  v = dpp_fmax<0x4E>(v);       // quad_perm [2,3,0,1]
  v = dpp_fmax<0x124>(v);      // row_ror 4
  v = dpp_fmax<0x128>(v);      // row_ror 8
  v = dpp_fmax<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_fmax<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One wave per token: logits = sum of the k-slice partials (ascending) + bias,
// then the score and the top-K.  Lane l holds experts 4l + r + 256v (r < 4,
// v < NV4), read as one 16-byte load per slice and v.  K rounds: the wave's
// largest remaining logit M by DPP into a scalar; of the candidates equal to
// M the lowest expert id wins -- within a block of 256 ids the lowest lane
// holding one (a ballot), in that lane the lowest slot -- and is then marked
// taken (-inf, like the slots past E; the logits of finite inputs are finite,
// and K <= E).  This is the order (logit desc, expert asc) of sel_key.
template <int NV4>
__global__ __launch_bounds__(256) void route_select_kernel(
    const float* __restrict__ part, int n_slices, int e_pad, const float* __restrict__ bias,
    int T, int E, int K, int score, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ weights, float* __restrict__ logits) {
  constexpr int NC = 4 * NV4;  // candidates per lane
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // All slice loads first (at most 8 slices), then the sums in ascending
  // slice order.
  f32x4 p[8][NV4];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int v = 0; v < NV4; ++v) {
      const int e = min(4 * lane + 256 * v, e_pad - 4);
      p[s][v] = s < n_slices
                    ? *reinterpret_cast<const f32x4*>(part + ((size_t)s * T + t) * e_pad + e)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float z[NC];
#pragma unroll
  for (int v = 0; v < NV4; ++v) {
    f32x4 a = p[0][v];
#pragma unroll
    for (int s = 1; s < 8; ++s)
      if (s < n_slices) a += p[s][v];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 4 * lane + 256 * v + r;
      z[4 * v + r] = e < E ? a[r] + (bias ? bias[e] : 0.f) : -INFINITY;
    }
  }
  if (logits) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int e = 4 * lane + 256 * (c / 4) + c % 4;
      if (e < E) logits[(size_t)t * E + e] = z[c];
    }
  }
  float m = 0.f, denom = 1.f;
  if (score == MOE_SCORE_SOFTMAX) {
    float lm = -INFINITY;
#pragma unroll
    for (int c = 0; c < NC; ++c) lm = fmaxf(lm, z[c]);
    m = wave_max(lm);
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (4 * lane + 256 * (c / 4) + c % 4 < E) sum += __expf(z[c] - m);
    denom = wave_sum(sum);
  }
  const float kTaken = -INFINITY;  // the slots past E already hold it
  int my_e = 0;
  float my_s = 0.f, sum_sel = 0.f, first = 0.f;
  for (int k = 0; k < K; ++k) {
    float lm = z[0];
#pragma unroll
    for (int c = 1; c < NC; ++c) lm = z[c] > lm ? z[c] : lm;
    const float bv = wave_fmax_uniform(lm);
    // The lowest block holding bv, its lowest lane, that lane's lowest slot.
    int L = 0, slot = 0;
#pragma unroll
    for (int v = NV4 - 1; v >= 0; --v) {
      const bool h0 = z[4 * v] == bv, h1 = z[4 * v + 1] == bv, h2 = z[4 * v + 2] == bv;
      const bool h3 = z[4 * v + 3] == bv;
      const unsigned long long mask = __ballot(h0 || h1 || h2 || h3);
      if (mask) {
        L = __builtin_ctzll(mask);
        const int r = h0 ? 0 : h1 ? 1 : h2 ? 2 : 3;
        slot = 4 * v + __builtin_amdgcn_readlane(r, L);
      }
    }
    const int be = 4 * L + (slot & 3) + 256 * (slot >> 2);
    if (lane == L) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c == slot) z[c] = kTaken;
    }
    if (k == 0) first = bv;
    const float sc = score_of(bv, score, renorm, m, first);
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

template <int NV>
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int K, int score, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ weights, float* __restrict__ logits) {
  constexpr int kGrp = 8;  // experts reduced together (independent butterflies)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  {
    const int t = blockIdx.x * kTokTile + wave;
    if (t >= T) return;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = -INFINITY;
    const float* xr = x + (size_t)t * d;
    for (int e0 = 0; e0 < E; e0 += kGrp) {
      // lane-partial dot products of kGrp experts, each in ascending i
      float p[kGrp];
#pragma unroll
      for (int g = 0; g < kGrp; ++g) p[g] = 0.f;
      for (int i = lane; i < d; i += kWave) {
        const float xv = xr[i];
#pragma unroll
        for (int g = 0; g < kGrp; ++g)
          if (e0 + g < E) p[g] = fmaf(xv, wr[(size_t)(e0 + g) * d + i], p[g]);
      }
      // kGrp independent butterfly sums (every lane ends with the same bits)
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int g = 0; g < kGrp; ++g) p[g] += __shfl_xor(p[g], off);
#pragma unroll
      for (int g = 0; g < kGrp; ++g) {
        const int e = e0 + g;
        if (e < E && (e & (kWave - 1)) == lane) {
          const float z = p[g] + (bias ? bias[e] : 0.f);
#pragma unroll
          for (int i = 0; i < NV; ++i)
            if (i == (e >> 6)) v[i] = z;
        }
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
// fraction of the token traffic, and at most 8 (a power of two, so it
// divides the 8 XCDs); slices are 64-multiples.
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
  const int n_tok = ceil_div(c.num_tokens, kRtTok);
  const int pairs = n_tok * (e_pad / (NT * 16));
  const int per = 8 / ks;  // XCDs per slice
  const dim3 grid(8 * ceil_div(pairs, per));
  hipLaunchKernelGGL(route_logits_kernel<NT>, grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr),
                     c.num_tokens, c.hidden, c.num_experts, e_pad, c.hidden / ks, ks, n_tok, part);
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
  // 4 experts per lane and 16-byte load: one or two of them per slice
  if (e_pad <= 256) return launch_select<1>(c, part, ks, e_pad, bias, ids, w, logits, s);
  return launch_select<2>(c, part, ks, e_pad, bias, ids, w, logits, s);
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
