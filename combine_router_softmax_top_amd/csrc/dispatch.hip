// Dispatch: per-expert counts, expert offsets and a stable scatter of the
// routed tokens into expert-contiguous rows.
//
// Operation ("Efficient and portable mixture-of-experts communication",
// Dispatch): count the tokens bound for each expert, copy the tokens into a
// contiguous per-expert buffer that feeds the grouped GEMM, and record for
// each row where it came from so that the combine can send it back.  The
// pages' receive side fills slots in arbitrary order; here the order is fixed
// (expert ascending, then token ascending), so the layout has one answer.
//
// Two kernels (one for batches of at most 2048 assignments, see self_count;
// three for very large histograms), no host synchronisation and no memset:
//  1. count: one workgroup per chunk of 1024 assignments (t*K + k in
//     ascending order, one per thread).  Each local expert gets a 1024-bit
//     mask over the chunk's assignment slots in LDS (64-bit LDS atomic OR);
//     the rank of an assignment inside its chunk is the popcount of the mask
//     bits below its slot, so a token that names an expert twice gets two
//     ranks in (t, k) order, like any other pair of assignments.  Every
//     expert's chunk count goes to a histogram row (LDS atomic add); invalid
//     ids are tallied into an extra column.
//  2. scatter: one wave per token, four per workgroup.  Each workgroup first
//     turns the local columns of the chunk histograms into expert offsets and
//     the row bases of its own chunks (inline_scan; the lowest workgroups
//     also write the global counts, the offsets and n_invalid); the token
//     row's loads are already in flight meanwhile.  The row (16-byte loads,
//     held in registers) is then written to each of its local rows, with the
//     row maps.  Tokens with no local expert are not read at all.
//  When the local chunk counts do not fit a scatter workgroup's LDS, a
//  one-workgroup scan kernel computes the offsets and per-(chunk, expert)
//  row bases first, and the scatter reads them.
// Block-scaled payload ([PPLX] Dispatch sends tokens with block scaling
// factors): the scatter can instead encode each bf16 token row once, while it
// holds it, as MX-FP8 (E4M3 codes, one E8M0 scale per 32 elements, the rule of
// moe_quantize_mxfp8) and write the codes and the scale words in the MFMA
// scale layout to every local row of the token: half the row bytes.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCA = kDispatchChunk;  // assignments per count chunk = threads per workgroup
constexpr int kWords = kCA / 64;     // 64-bit mask words per expert and chunk

__global__ __launch_bounds__(kCA) void dispatch_count_kernel(
    const int32_t* __restrict__ ids, int n_assign, int E, int eb, int ee,
    int32_t* __restrict__ hist /*[n_chunks][E+1]*/, int32_t* __restrict__ rank /*[n_assign]*/) {
  __shared__ unsigned long long mask[MOE_MAX_EXPERTS * kWords];  // [local expert][word]
  __shared__ int cnt[MOE_MAX_EXPERTS + 1];                        // [expert], [E] = invalid
  const int tid = threadIdx.x;
  const int n_loc = ee - eb;
  for (int i = tid; i < n_loc * kWords; i += kCA) mask[i] = 0ull;
  for (int i = tid; i <= E; i += kCA) cnt[i] = 0;
  __syncthreads();
  const long long a = (long long)blockIdx.x * kCA + tid;
  const bool in = a < n_assign;
  const int word = tid >> 6;
  const unsigned long long bit = 1ull << (tid & 63);
  const int e = in ? ids[a] : -1;
  const bool valid = e >= 0 && e < E;
  const bool local = in && e >= eb && e < ee;
  if (in) atomicAdd(&cnt[valid ? e : E], 1);
  if (local) atomicOr(&mask[(e - eb) * kWords + word], bit);
  __syncthreads();
  if (in) {
    int r = -1;
    if (local) {
      const unsigned long long* m = mask + (e - eb) * kWords;
      r = __popcll(m[word] & (bit - 1ull));
      for (int w = 0; w < word; ++w) r += __popcll(m[w]);
    }
    rank[a] = r;
  }
  int32_t* h = hist + (size_t)blockIdx.x * (E + 1);
  for (int i = tid; i <= E; i += kCA) h[i] = cnt[i];
}

constexpr int kScanThreads = 1024;
constexpr int kScanLdsInts = 32768;  // chunk histograms staged in LDS when they fit (128 KB)

__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(
    const int32_t* __restrict__ hist, int n_chunks, int E, int eb, int ee,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ base,
    int32_t* __restrict__ n_invalid) {
  __shared__ int32_t hs[kScanLdsInts];
  __shared__ int32_t loc[MOE_MAX_EXPERTS];
  __shared__ int32_t scan[2][MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int n_loc = ee - eb;
  const int n_hist = n_chunks * (E + 1);
  // One coalesced pass over the histograms into LDS (else read them in place).
  const bool staged = n_hist <= kScanLdsInts;
  if (staged)
    for (int i = tid; i < n_hist; i += kScanThreads) hs[i] = hist[i];
  __syncthreads();
  const int32_t* h = staged ? hs : hist;
  for (int e = tid; e <= E; e += kScanThreads) {
    int s = 0;
    for (int c = 0; c < n_chunks; ++c) s += h[(size_t)c * (E + 1) + e];
    if (e == E) *n_invalid = s;
    else {
      counts[e] = s;
      if (e >= eb && e < ee) loc[e - eb] = s;
    }
  }
  __syncthreads();
  // Inclusive Hillis-Steele scan over the local experts' counts.
  int cur = 0;
  for (int j = tid; j < n_loc; j += kScanThreads) scan[0][j] = loc[j];
  __syncthreads();
  for (int off = 1; off < n_loc; off <<= 1) {
    for (int j = tid; j < n_loc; j += kScanThreads)
      scan[cur ^ 1][j] = scan[cur][j] + (j >= off ? scan[cur][j - off] : 0);
    cur ^= 1;
    __syncthreads();
  }
  if (tid == 0) offsets[0] = 0;
  for (int j = tid; j < n_loc; j += kScanThreads) offsets[j + 1] = scan[cur][j];
  // Row base of (chunk c, local expert j) = offset of j + rows of j in earlier chunks.
  for (int j = tid; j < n_loc; j += kScanThreads) {
    int run = scan[cur][j] - loc[j];
    for (int c = 0; c < n_chunks; ++c) {
      base[(size_t)c * n_loc + j] = run;
      run += h[(size_t)c * (E + 1) + eb + j];
    }
  }
}

constexpr int kInlineScanInts = 4096;  // local chunk counts a scatter workgroup stages

// Row numbers for the scatter, computed inside each scatter workgroup (when
// the local chunk counts fit in kInlineScanInts): the workgroup stages the
// counts of the local experts in every chunk, totals them per expert, scans
// the totals into expert offsets, and keeps, for the (at most two) chunks its
// assignments fall in, offset + rows of the expert in earlier chunks.  The
// workgroups with the lowest ids also write the global counts, n_invalid and
// the offsets.  Every thread of the workgroup takes part (barriers).
struct InlineScan {
  int32_t hl[kInlineScanInts];         // [chunk][local expert]
  int32_t sc[2][MOE_MAX_EXPERTS];      // scan ping-pong
  int32_t base[2][MOE_MAX_EXPERTS];    // row base of chunks c_lo, c_lo + 1
};

__device__ void inline_scan(InlineScan& L, const int32_t* __restrict__ hist, int n_chunks, int E,
                            int eb, int n_loc, int c_lo, int32_t* __restrict__ counts,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ n_invalid) {
  const int tid = threadIdx.x;
  // Global counts of all E experts and the invalid column (grid-stride).
  for (int e = blockIdx.x * 256 + tid; e <= E; e += gridDim.x * 256) {
    int sum = 0;
    for (int c = 0; c < n_chunks; ++c) sum += hist[(size_t)c * (E + 1) + e];
    if (e == E) *n_invalid = sum;
    else counts[e] = sum;
  }
  const int n_h = n_chunks * n_loc;
  for (int i = tid; i < n_h; i += 256) {
    const int c = i / n_loc;
    L.hl[i] = hist[(size_t)c * (E + 1) + eb + (i - c * n_loc)];
  }
  __syncthreads();
  for (int j = tid; j < n_loc; j += 256) {
    int tot = 0, before = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const int v = L.hl[c * n_loc + j];
      before += c < c_lo ? v : 0;
      tot += v;
    }
    L.sc[0][j] = tot;
    L.base[0][j] = before;
    L.base[1][j] = before + L.hl[c_lo * n_loc + j];
  }
  __syncthreads();
  // Inclusive Hillis-Steele scan of the totals.
  int cur = 0;
  for (int off = 1; off < n_loc; off <<= 1) {
    for (int j = tid; j < n_loc; j += 256)
      L.sc[cur ^ 1][j] = L.sc[cur][j] + (j >= off ? L.sc[cur][j - off] : 0);
    cur ^= 1;
    __syncthreads();
  }
  for (int j = tid; j < n_loc; j += 256) {
    const int incl = L.sc[cur][j];
    const int excl = j > 0 ? L.sc[cur][j - 1] : 0;
    L.base[0][j] += excl;
    L.base[1][j] += excl;
    if (blockIdx.x == 0) offsets[j + 1] = incl;
  }
  if (blockIdx.x == 0 && tid == 0) offsets[0] = 0;
  __syncthreads();
}

// Batches of at most kSelfAssign assignments skip the count kernel: every
// scatter workgroup reads all the ids itself (8 KB at most, from L2), counts
// them per expert (LDS atomics; invalid ids in an extra column) and counts the
// local experts' assignments before its own first one, scans the local totals
// into offsets, and ranks its own assignments among themselves.  A local
// assignment a to expert e gets row offset(e) + (assignments to e before a),
// the count kernel's rank plus row base, so the layout is the same.  Workgroup
// 0 also writes the counts, n_invalid and the offsets.  Every thread of the
// workgroup takes part (barriers).  Measured: a decode batch (128 tokens x 6)
// 12.1 -> 9.5 us with cold caches; at 8192 assignments (4096 tokens x 2, 8
// experts) 23 -> 30 us -- each of 1024 workgroups then counts 8192 ids into 8
// contended LDS counters -- so larger batches keep the count kernel.
constexpr int kSelfAssign = 2048;

struct SelfCount {
  int32_t cnt[MOE_MAX_EXPERTS + 1];  // per expert over the batch; [E] = invalid ids
  int32_t bef[MOE_MAX_EXPERTS];      // local experts: assignments before the workgroup's first
  int32_t sc[2][MOE_MAX_EXPERTS];    // scan ping-pong over the local totals
  int32_t own[4 * MOE_MAX_TOPK];     // the workgroup's own ids
};

// Returns which sc buffer holds the inclusive scan of the local totals.
__device__ int self_count(SelfCount& L, const int32_t* __restrict__ ids, int n_assign, int E,
                          int eb, int n_loc, int a0, int n_own, int32_t* __restrict__ counts,
                          int32_t* __restrict__ offsets, int32_t* __restrict__ n_invalid) {
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += 256) L.cnt[i] = 0;
  for (int i = tid; i < n_loc; i += 256) L.bef[i] = 0;
  __syncthreads();
  for (int i = tid; i < n_assign; i += 256) {
    const int e = ids[i];
    atomicAdd(&L.cnt[e >= 0 && e < E ? e : E], 1);
    if (i < a0 && e >= eb && e < eb + n_loc) atomicAdd(&L.bef[e - eb], 1);
    if (i >= a0 && i < a0 + n_own) L.own[i - a0] = e;
  }
  __syncthreads();
  for (int j = tid; j < n_loc; j += 256) L.sc[0][j] = L.cnt[eb + j];
  __syncthreads();
  int cur = 0;
  for (int off = 1; off < n_loc; off <<= 1) {  // inclusive Hillis-Steele scan
    for (int j = tid; j < n_loc; j += 256)
      L.sc[cur ^ 1][j] = L.sc[cur][j] + (j >= off ? L.sc[cur][j - off] : 0);
    cur ^= 1;
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += 256) counts[e] = L.cnt[e];
    for (int j = tid; j < n_loc; j += 256) offsets[j + 1] = L.sc[cur][j];
    if (tid == 0) {
      *n_invalid = L.cnt[E];
      offsets[0] = 0;
    }
  }
  return cur;
}

// NV = 16-byte pieces of the row each lane holds at once.  SELF: row numbers
// from self_count (no count kernel); else INLINE: from inline_scan (hist),
// else from the scan kernel (base).
// Q: encode the (bf16) row as MX-FP8 into codes xq [T*K, d] and scale words
// xs (MFMA layout over T*K rows) instead of copying it to x_sorted.
template <int NV, bool INLINE, bool Q, bool SELF = false>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ hist, int n_chunks, int E, int T, int K, int eb, int n_loc,
    int row_vecs, u32x4* __restrict__ x_sorted, int32_t* __restrict__ src_index,
    int32_t* __restrict__ row_of, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_invalid, uint8_t* __restrict__ xq, uint32_t* __restrict__ xs) {
  __shared__ typename std::conditional<
      SELF, SelfCount, typename std::conditional<INLINE, InlineScan, int>::type>::type lds;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool tok = t < T;  // wave-uniform
  int a = -1, r = -1, j = 0;
  if (tok && lane < K) {
    a = t * K + lane;
    if constexpr (SELF) {  // r >= 0 marks a local assignment; its rank comes below
      const int e = ids[a];
      if (e >= eb && e < eb + n_loc) {
        r = 0;
        j = e - eb;
      }
    } else {
      r = rank[a];
      if (r >= 0) j = ids[a] - eb;
    }
  }
  const bool any = __ballot(r >= 0) != 0ull;  // any local row (wave-uniform)
  // The first piece of the token row does not depend on the row numbers:
  // its loads go out before the scan.
  const u32x4* src = x + (size_t)(tok ? t : 0) * row_vecs;
  u32x4 buf[NV];
  auto load_piece = [&](int v0) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v < row_vecs) buf[u] = src[v];
    }
  };
  if (tok && any) load_piece(0);
  int myrow = -1;
  if constexpr (SELF) {
    const int a0 = blockIdx.x * 4 * K;
    const int n_own = min(4, T - blockIdx.x * 4) * K;
    const int cur = self_count(lds, ids, T * K, E, eb, n_loc, a0, n_own, counts, offsets, n_invalid);
    if (r >= 0) {
      int rk = lds.bef[j];
      for (int i = a0; i < a; ++i) rk += lds.own[i - a0] == eb + j ? 1 : 0;
      myrow = lds.sc[cur][j] - lds.cnt[eb + j] + rk;
    }
  } else if constexpr (INLINE) {
    const int c_lo = blockIdx.x * 4 * K / kCA;  // chunk of the workgroup's first assignment
    inline_scan(lds, hist, n_chunks, E, eb, n_loc, c_lo, counts, offsets, n_invalid);
    if (r >= 0) myrow = lds.base[a / kCA - c_lo][j] + r;
  } else {
    if (r >= 0) myrow = base[(size_t)(a / kCA) * n_loc + j] + r;
  }
  if (!tok) return;
  if (lane < K) {
    if (myrow >= 0) src_index[myrow] = a;
    row_of[a] = myrow;
  }
  if (!any) return;
  for (int v0 = 0; v0 < row_vecs; v0 += kWave * NV) {
    if (v0 > 0) load_piece(v0);
    if constexpr (Q) {
      // Piece v (8 elements) sits in lane v % 64 of step u, so a step holds
      // 16 whole blocks (block q = v / 4, its 4 pieces in lanes 4q'..4q'+3,
      // q' = q % 16): one scale group g = v0 / 64 + u of the MFMA layout.
      // row_vecs is a multiple of 64, so a step is wholly in or out.
      uint32_t code_lo[NV], code_hi[NV], word[NV];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        if (v0 + u * kWave >= row_vecs) break;
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = __uint_as_float(buf[u][i] << 16);
          f[2 * i + 1] = __uint_as_float(buf[u][i] & 0xffff0000u);
        }
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        const int ef = (int)((__float_as_uint(m) >> 23) & 0xff);
        const int sc = min(127, max(-127, ef - 127 - 8));
        const float inv = __uint_as_float((uint32_t)(127 - sc) << 23);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = fminf(448.f, fmaxf(-448.f, f[i] * inv));
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
        code_lo[u] = (uint32_t)lo;
        code_hi[u] = (uint32_t)hi;
        // Scale word (d, h) of the group: bytes b = 0..3 are blocks
        // m = 8d + 2b + h, i.e. lanes 32d + 4h + 8b; lanes 0, 4, 32, 36 write.
        const int sb = sc + 127;
        word[u] = (uint32_t)__shfl(sb, lane) | ((uint32_t)__shfl(sb, lane + 8) << 8) |
                  ((uint32_t)__shfl(sb, lane + 16) << 16) | ((uint32_t)__shfl(sb, lane + 24) << 24);
      }
      const bool writer = (lane & ~36) == 0;  // lanes 0, 4, 32, 36
      const int wd = lane >> 5, wh = (lane >> 2) & 1;
      for (int k = 0; k < K; ++k) {
        const int rk = __builtin_amdgcn_readlane(myrow, k);
        if (rk < 0) continue;
        uint8_t* dst = xq + (size_t)rk * row_vecs * 8;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          if (v0 + u * kWave >= row_vecs) break;
          const int v = v0 + u * kWave + lane;
          *reinterpret_cast<u32x2*>(dst + (size_t)v * 8) = u32x2{code_lo[u], code_hi[u]};
          if (writer) {
            const size_t g = (size_t)(v0 / kWave + u);
            xs[((2 * g + wd) * (size_t)T * K + rk) * 2 + wh] = word[u];
          }
        }
      }
    } else {
      for (int k = 0; k < K; ++k) {
        const int rk = __builtin_amdgcn_readlane(myrow, k);
        if (rk < 0) continue;
        u32x4* dst = x_sorted + (size_t)rk * row_vecs;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int v = v0 + u * kWave + lane;
          if (v < row_vecs) dst[v] = buf[u];
        }
      }
    }
  }
}

template <int NV>
void launch_scatter(bool self, bool inl, dim3 grid, hipStream_t s, const void* x, const int32_t* ids,
                    const int32_t* rank, const int32_t* base, const int32_t* hist, int n_chunks,
                    int E, int T, int K, int eb, int n_loc, int row_vecs, void* x_sorted,
                    int32_t* src_index, int32_t* row_of, int32_t* counts, int32_t* offsets,
                    int32_t* n_invalid, uint8_t* xq, uint32_t* xs) {
  auto kern = xq ? (self  ? dispatch_scatter_kernel<NV, false, true, true>
                   : inl ? dispatch_scatter_kernel<NV, true, true>
                         : dispatch_scatter_kernel<NV, false, true>)
                 : (self  ? dispatch_scatter_kernel<NV, false, false, true>
                   : inl ? dispatch_scatter_kernel<NV, true, false>
                         : dispatch_scatter_kernel<NV, false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, static_cast<const u32x4*>(x), ids, rank, base,
                     hist, n_chunks, E, T, K, eb, n_loc, row_vecs,
                     static_cast<u32x4*>(x_sorted), src_index, row_of, counts, offsets,
                     n_invalid, xq, xs);
}

}  // namespace

// Workspace: [n_invalid (256 B)] [hist n_chunks*(E+1)] [rank T*K] [base n_chunks*E_loc]
size_t dispatch_workspace_bytes(const moe_config_t& c) {
  const size_t n_chunks = (size_t)ceil_div(c.num_tokens * c.top_k, kCA);
  const size_t n_loc = (size_t)(c.expert_end - c.expert_begin);
  size_t b = 256;
  b += align_up(n_chunks * (c.num_experts + 1) * 4, 256);
  b += align_up((size_t)c.num_tokens * c.top_k * 4, 256);
  b += align_up(n_chunks * n_loc * 4, 256);
  return b;
}

hipError_t launch_dispatch(const moe_config_t& c, const void* x, const int32_t* ids,
                           int32_t* counts, int32_t* offsets, void* x_sorted, int32_t* src_index,
                           int32_t* row_of, void* workspace, hipStream_t s, uint8_t* xq,
                           uint32_t* xs, int32_t* n_invalid_out) {
  const int T = c.num_tokens, K = c.top_k, E = c.num_experts;
  const int eb = c.expert_begin, ee = c.expert_end, n_loc = ee - eb;
  const int n_assign = T * K;
  const int n_chunks = ceil_div(n_assign, kCA);
  char* ws = static_cast<char*>(workspace);
  int32_t* n_invalid = n_invalid_out ? n_invalid_out : reinterpret_cast<int32_t*>(ws);
  ws += 256;
  int32_t* hist = reinterpret_cast<int32_t*>(ws);
  ws += align_up((size_t)n_chunks * (E + 1) * 4, 256);
  int32_t* rank = reinterpret_cast<int32_t*>(ws);
  ws += align_up((size_t)T * K * 4, 256);
  int32_t* base = reinterpret_cast<int32_t*>(ws);

  // Small batches: the scatter counts for itself (no count kernel).  Else the
  // count kernel, and the scan inside the scatter when the local chunk counts
  // fit its LDS.
  const bool self = n_assign <= kSelfAssign;
  hipError_t err = hipSuccess;
  if (!self) {
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(n_chunks), dim3(kCA), 0, s, ids, n_assign, E,
                       eb, ee, hist, rank);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const bool inl = (size_t)n_chunks * n_loc <= (size_t)kInlineScanInts;
  if (!self && !inl) {
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, hist, n_chunks,
                       E, eb, ee, counts, offsets, base, n_invalid);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int elem = c.dtype == MOE_BF16 ? 2 : 4;
  const int row_vecs = c.hidden * elem / 16;
  const int per_lane = ceil_div(row_vecs, kWave);
  const dim3 grid(ceil_div(T, 4));
  if (per_lane <= 4)
    launch_scatter<4>(self, inl, grid, s, x, ids, rank, base, hist, n_chunks, E, T, K, eb, n_loc,
                      row_vecs, x_sorted, src_index, row_of, counts, offsets, n_invalid, xq, xs);
  else if (per_lane <= 8)
    launch_scatter<8>(self, inl, grid, s, x, ids, rank, base, hist, n_chunks, E, T, K, eb, n_loc,
                      row_vecs, x_sorted, src_index, row_of, counts, offsets, n_invalid, xq, xs);
  else
    launch_scatter<16>(self, inl, grid, s, x, ids, rank, base, hist, n_chunks, E, T, K, eb, n_loc,
                       row_vecs, x_sorted, src_index, row_of, counts, offsets, n_invalid, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
