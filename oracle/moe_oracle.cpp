// CPU oracle for one GPU's share of a Mixture-of-Experts layer.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
// call this file: only the tests, the smoke check and the benchmark's CPU
// baseline use it.  It shares no code, header, table or helper with the HIP
// library; the two meet only through the seeded inputs.
//
// What it computes (the plain definitions, written as literal loops):
//   * router: a small linear layer producing per-expert logits, turned into a
//     probability distribution; the top-K experts by score are selected and
//     their router-derived weights kept
//     ("Efficient and portable mixture-of-experts communication", Introduction);
//   * dispatch: per-expert token counts and an expert-contiguous copy of the
//     routed tokens, plus the source-index records that tell the combine where
//     each row goes back (same page, Dispatch section).  Unlike the pages'
//     receive kernels, whose slot order is non-deterministic, rows here are
//     ordered by expert, then token index, so the layout has one answer;
//   * expert MLP: each expert a small SiLU-gated MLP (same page, Introduction:
//     experts are small MLPs evaluated by a grouped GEMM, Dispatch section);
//   * combine: the weighted sum of the selected experts' outputs, written to a
//     caller-owned tensor (same page, Introduction and Combine section);
//   * the block-scaled payload: MX-FP8 encoding of rows (E4M3 elements, one
//     power-of-two scale per 32) and the layer with the dispatched rows and
//     the gate / up weights replaced by their decodings (same page, Dispatch:
//     block scaling factors travel with the tokens; Combine: results return
//     unquantized);
//   * the dual-microbatch split: the token range cut at the midpoint of the
//     padded token count, or on a request boundary for a uniform batch of
//     multi-token queries, only above a token threshold ("Dual Batch
//     Overlap", UBatchRunner and Running with DBO), each part run on its own
//     and the results concatenated.
//
// Arithmetic: every value is read exactly (bf16 and fp32 inputs are exact in
// fp64), every sum is accumulated in fp64 in ascending index order, compiled
// with -ffp-contract=off and without fast-math.  OpenMP, when enabled, only
// splits independent output rows between threads, so results do not depend on
// the thread count.
//
// Parity status: every function below is pinned by the CPU tests against
// closed forms, brute force on tiny inputs, textbook special cases and
// invariants; none is "parity unpinned".

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_F64 = 2 };
enum { OSCORE_SOFTMAX = 0, OSCORE_SIGMOID = 1 };

// Exact value of element i of a typed array.
inline double value_at(const void* p, size_t i, int dt) {
  if (dt == ODT_F32) return static_cast<double>(static_cast<const float*>(p)[i]);
  if (dt == ODT_BF16) {
    uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return static_cast<double>(f);
  }
  return static_cast<const double*>(p)[i];
}

inline size_t dtype_bytes(int dt) { return dt == ODT_F32 ? 4 : (dt == ODT_BF16 ? 2 : 8); }

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// Score of one logit given the full logit row (softmax needs all of it).
// Softmax: p_e = exp(z_e - max z) / sum_j exp(z_j - max z); sigmoid: 1/(1+exp(-z)).
void scores_of_row(const double* z, int E, int score, double* s) {
  if (score == OSCORE_SIGMOID) {
    for (int e = 0; e < E; ++e) s[e] = 1.0 / (1.0 + std::exp(-z[e]));
    return;
  }
  double m = z[0];
  for (int e = 1; e < E; ++e) m = std::max(m, z[e]);
  double denom = 0.0;
  for (int e = 0; e < E; ++e) denom += std::exp(z[e] - m);
  for (int e = 0; e < E; ++e) s[e] = std::exp(z[e] - m) / denom;
}

// Select the K largest keys of one row: repeated maximum search, a strictly
// greater key replaces the candidate, so equal keys go to the lower expert id;
// slots come out in descending key order.
void topk_of_row(const double* key, int E, int K, int32_t* ids) {
  std::vector<char> taken(E, 0);
  for (int k = 0; k < K; ++k) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e;
    }
    taken[best] = 1;
    ids[k] = best;
  }
}

void weights_of_row(const double* s, const int32_t* ids, int K, int renorm, double* w) {
  double total = 0.0;
  for (int k = 0; k < K; ++k) total += s[ids[k]];
  for (int k = 0; k < K; ++k) w[k] = renorm ? s[ids[k]] / total : s[ids[k]];
}

}  // namespace

extern "C" {

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

// Router logits: z[t,e] = sum_i x[t,i] * w_router[e,i] (+ bias[e]).
// x [T,d] and w_router [E,d] of dtype dt; bias [E] fp32 or NULL; z [T,E] fp64.
void oracle_router_logits(int T, int d, int E, int dt, const void* x, const void* w_router,
                          const float* bias, double* z) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i)
        acc += value_at(x, (size_t)t * d + i, dt) * value_at(w_router, (size_t)e * d + i, dt);
      if (bias) acc += static_cast<double>(bias[e]);
      z[(size_t)t * E + e] = acc;
    }
  }
}

// Top-K selection and weights from given logits z [T,E] (dtype dt_z).
// Selection is on the logits themselves: both score functions are increasing,
// so the K largest logits are the K largest scores.  Weights are the selected
// scores, divided by their sum when renorm is set.
void oracle_topk(int T, int E, int K, int dt_z, const void* z, int score, int renorm,
                 int32_t* ids, double* weights) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    std::vector<double> key(E), s(E);
    for (int e = 0; e < E; ++e) key[e] = value_at(z, (size_t)t * E + e, dt_z);
    scores_of_row(key.data(), E, score, s.data());
    topk_of_row(key.data(), E, K, ids + (size_t)t * K);
    weights_of_row(s.data(), ids + (size_t)t * K, K, renorm, weights + (size_t)t * K);
  }
}

// Full router step: logits then top-K.  logits_out may be NULL.
void oracle_route(int T, int d, int E, int K, int dt, const void* x, const void* w_router,
                  const float* bias, int score, int renorm, int32_t* ids, double* weights,
                  double* logits_out) {
  std::vector<double> z((size_t)T * E);
  oracle_router_logits(T, d, E, dt, x, w_router, bias, z.data());
  oracle_topk(T, E, K, ODT_F64, z.data(), score, renorm, ids, weights);
  if (logits_out) std::memcpy(logits_out, z.data(), sizeof(double) * z.size());
}

// Dispatch layout.  counts[e] over all E experts (ids outside [0,E) are not
// counted but tallied in *n_invalid); offsets [E_loc+1] is the exclusive scan
// of the local experts' counts; rows are filled expert by expert (ascending),
// token by token (ascending): src_index[row] = t*K + k, row_of[t*K+k] = row,
// and row_of = -1 for assignments to non-local or invalid experts.
// If x is not NULL, x_sorted[row] is a byte copy of x[t] (row_bytes each).
// Returns the number of local rows.
int oracle_dispatch(int T, int E, int K, int e_begin, int e_end, const int32_t* ids,
                    int32_t* counts, int32_t* offsets, int32_t* src_index, int32_t* row_of,
                    int32_t* n_invalid, const void* x, void* x_sorted, long long row_bytes) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  int bad = 0;
  for (int a = 0; a < T * K; ++a) {
    int e = ids[a];
    if (e < 0 || e >= E) ++bad;
    else ++counts[e];
  }
  if (n_invalid) *n_invalid = bad;
  const int n_loc = e_end - e_begin;
  offsets[0] = 0;
  for (int j = 0; j < n_loc; ++j) offsets[j + 1] = offsets[j] + counts[e_begin + j];
  for (int a = 0; a < T * K; ++a) row_of[a] = -1;
  int row = 0;
  for (int e = e_begin; e < e_end; ++e) {
    for (int t = 0; t < T; ++t) {
      for (int k = 0; k < K; ++k) {
        if (ids[(size_t)t * K + k] != e) continue;
        src_index[row] = t * K + k;
        row_of[(size_t)t * K + k] = row;
        if (x && x_sorted)
          std::memcpy(static_cast<char*>(x_sorted) + (size_t)row * row_bytes,
                      static_cast<const char*>(x) + (size_t)t * row_bytes, (size_t)row_bytes);
        ++row;
      }
    }
  }
  return row;
}

// SiLU-gated expert MLP on a list of rows.  Row r uses expert row_expert[r]
// (an index into the weight stacks, i.e. local expert number).
//   h[j]   = SiLU(sum_i x[r,i] * w_gate[e,j,i]) * (sum_i x[r,i] * w_up[e,j,i])
//   y[r,c] = sum_j h[j] * w_down[e,c,j]
// x_rows [n,d] dtype dt_x; w_gate, w_up [E_loc,I,d] and w_down [E_loc,d,I]
// dtype dt_w; y [n,d] fp64.  h stays in fp64.
void oracle_expert_mlp(int n_rows, int d, int I, int dt_x, const void* x_rows,
                       const int32_t* row_expert, int dt_w, const void* w_gate,
                       const void* w_up, const void* w_down, double* y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    const size_t e = (size_t)row_expert[r];
    std::vector<double> xr(d), h(I);
    for (int i = 0; i < d; ++i) xr[i] = value_at(x_rows, (size_t)r * d + i, dt_x);
    for (int j = 0; j < I; ++j) {
      double g = 0.0, u = 0.0;
      const size_t base = (e * I + j) * (size_t)d;
      for (int i = 0; i < d; ++i) {
        g += xr[i] * value_at(w_gate, base + i, dt_w);
        u += xr[i] * value_at(w_up, base + i, dt_w);
      }
      h[j] = silu(g) * u;
    }
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      const size_t base = (e * d + c) * (size_t)I;
      for (int j = 0; j < I; ++j) acc += h[j] * value_at(w_down, base + j, dt_w);
      y[(size_t)r * d + c] = acc;
    }
  }
}

// Weighted-sum combine for the tokens listed in `tokens` (n_tok of them):
//   out[i,c] = sum_{k ascending, row_of[t,k] >= 0} w[t,k] * y_sorted[row_of[t,k], c]
//            + sum_{s ascending} y_shared[s, t, c]
// with t = tokens[i].  y_sorted [*,d] dtype dt_y; weights [T,K] dtype dt_w;
// y_shared [n_shared,T,d] dtype dt_y or NULL; out [n_tok,d] fp64.
void oracle_combine_tokens(int n_tok, const int32_t* tokens, int T, int d, int K, int dt_y,
                           const void* y_sorted, const int32_t* row_of, int dt_w,
                           const void* weights, int n_shared, const void* y_shared,
                           double* out) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n_tok; ++i) {
    const size_t t = (size_t)tokens[i];
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        const int32_t r = row_of[t * K + k];
        if (r < 0) continue;
        acc += value_at(weights, t * K + k, dt_w) * value_at(y_sorted, (size_t)r * d + c, dt_y);
      }
      for (int s = 0; s < n_shared; ++s)
        acc += value_at(y_shared, ((size_t)s * T + t) * d + c, dt_y);
      out[(size_t)i * d + c] = acc;
    }
  }
}

void oracle_combine(int T, int d, int K, int dt_y, const void* y_sorted, const int32_t* row_of,
                    int dt_w, const void* weights, int n_shared, const void* y_shared,
                    double* out) {
  std::vector<int32_t> all(T);
  for (int t = 0; t < T; ++t) all[t] = t;
  oracle_combine_tokens(T, all.data(), T, d, K, dt_y, y_sorted, row_of, dt_w, weights,
                        n_shared, y_shared, out);
}

// Whole layer on tokens [0,T): route, dispatch, routed experts, shared
// experts (applied to every token with weight one), combine.  All
// intermediates stay fp64.  x [T,d] dtype dt; w_router [E,d] dtype dt;
// bias fp32 [E] or NULL; routed weights [E_loc,...] dtype dt; shared weights
// [n_shared,...] dtype dt or NULL.  Outputs: out [T,d] fp64; ids [T,K];
// weights_out [T,K] fp64; counts [E] (any of the last three may be NULL).
// Returns the number of local rows.
int oracle_forward(int T, int d, int E, int K, int I, int e_begin, int e_end, int n_shared,
                   int score, int renorm, int dt, const void* x, const void* w_router,
                   const float* bias, const void* w_gate, const void* w_up, const void* w_down,
                   const void* ws_gate, const void* ws_up, const void* ws_down, double* out,
                   int32_t* ids_out, double* weights_out, int32_t* counts_out) {
  const int n_loc = e_end - e_begin;
  std::vector<int32_t> ids((size_t)T * K), counts(E), offsets(n_loc + 1),
      src((size_t)T * K), row_of((size_t)T * K);
  std::vector<double> w((size_t)T * K);
  oracle_route(T, d, E, K, dt, x, w_router, bias, score, renorm, ids.data(), w.data(), nullptr);
  int32_t bad = 0;
  const size_t rb = (size_t)d * dtype_bytes(dt);
  std::vector<char> xs((size_t)T * K * rb);
  const int n_rows = oracle_dispatch(T, E, K, e_begin, e_end, ids.data(), counts.data(),
                                     offsets.data(), src.data(), row_of.data(), &bad, x,
                                     xs.data(), (long long)rb);
  std::vector<int32_t> row_expert(std::max(n_rows, 1));
  for (int j = 0; j < n_loc; ++j)
    for (int r = offsets[j]; r < offsets[j + 1]; ++r) row_expert[r] = j;
  std::vector<double> y((size_t)std::max(n_rows, 1) * d);
  if (n_rows > 0)
    oracle_expert_mlp(n_rows, d, I, dt, xs.data(), row_expert.data(), dt, w_gate, w_up,
                      w_down, y.data());
  std::vector<double> ysh;
  if (n_shared > 0) {
    ysh.resize((size_t)n_shared * T * d);
    std::vector<int32_t> sh_expert(T);
    for (int s = 0; s < n_shared; ++s) {
      for (int t = 0; t < T; ++t) sh_expert[t] = s;
      oracle_expert_mlp(T, d, I, dt, x, sh_expert.data(), dt, ws_gate, ws_up, ws_down,
                        ysh.data() + (size_t)s * T * d);
    }
  }
  oracle_combine(T, d, K, ODT_F64, y.data(), row_of.data(), ODT_F64, w.data(), n_shared,
                 n_shared > 0 ? ysh.data() : nullptr, out);
  if (ids_out) std::memcpy(ids_out, ids.data(), sizeof(int32_t) * ids.size());
  if (weights_out) std::memcpy(weights_out, w.data(), sizeof(double) * w.size());
  if (counts_out) std::memcpy(counts_out, counts.data(), sizeof(int32_t) * counts.size());
  return n_rows;
}

void oracle_mxfp8_quantize(int rows, int cols, int dt, const void* in, long long ld,
                           uint8_t* codes, uint8_t* scales);
void oracle_mxfp8_dequantize(int rows, int cols, const uint8_t* codes, const uint8_t* scales,
                             double* out);

// The expert MLP of the block-scaled layer on n_rows rows x_rows [n_rows, d]
// (dtype dt; row r uses expert row_expert[r] of the n_exp in the stacks):
// the rows and every row of the gate / up stacks [n_exp*I, d] replaced by
// their MX-FP8 decodings, then as oracle_expert_mlp, with the down projection
// either on the fp64 h and the dtype-dt down weights (down_mx = 0) or on the
// decodings of h (32-element blocks along I) and of the down stack
// [n_exp*d, I] (down_mx = 1).  y [n_rows, d] fp64.
void oracle_expert_mlp_mxfp8(int n_rows, int d, int I, int n_exp, int dt, const void* x_rows,
                             const int32_t* row_expert, const void* w_gate, const void* w_up,
                             const void* w_down, int down_mx, double* y) {
  // The MX-FP8 decoding of a rows x cols matrix of element type t.
  auto decoded = [&](int rows, int cols, int t, const void* m) {
    std::vector<uint8_t> codes((size_t)rows * cols), scales((size_t)rows * (cols / 32));
    std::vector<double> v((size_t)rows * cols);
    oracle_mxfp8_quantize(rows, cols, t, m, cols, codes.data(), scales.data());
    oracle_mxfp8_dequantize(rows, cols, codes.data(), scales.data(), v.data());
    return v;
  };
  const std::vector<double> xq = decoded(n_rows, d, dt, x_rows);
  const std::vector<double> gq = decoded(n_exp * I, d, dt, w_gate);
  const std::vector<double> uq = decoded(n_exp * I, d, dt, w_up);
  if (!down_mx) {
    std::vector<double> wd((size_t)n_exp * d * I);
    for (size_t i = 0; i < wd.size(); ++i) wd[i] = value_at(w_down, i, dt);
    oracle_expert_mlp(n_rows, d, I, ODT_F64, xq.data(), row_expert, ODT_F64, gq.data(),
                      uq.data(), wd.data(), y);
    return;
  }
  // h of every row as in oracle_expert_mlp, then its decoding, then the down
  // projection on the decoded h and the decoded down weights.
  std::vector<double> hh((size_t)n_rows * I);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    const size_t e = (size_t)row_expert[r];
    for (int j = 0; j < I; ++j) {
      double g = 0.0, u = 0.0;
      const size_t base = (e * I + j) * (size_t)d;
      for (int i = 0; i < d; ++i) {
        g += xq[(size_t)r * d + i] * gq[base + i];
        u += xq[(size_t)r * d + i] * uq[base + i];
      }
      hh[(size_t)r * I + j] = silu(g) * u;
    }
  }
  const std::vector<double> hq = decoded(n_rows, I, ODT_F64, hh.data());
  const std::vector<double> wdq = decoded(n_exp * d, I, dt, w_down);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    const size_t e = (size_t)row_expert[r];
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      const size_t base = (e * d + c) * (size_t)I;
      for (int j = 0; j < I; ++j) acc += hq[(size_t)r * I + j] * wdq[base + j];
      y[(size_t)r * d + c] = acc;
    }
  }
}

// Whole layer with a block-scaled 8-bit payload ("Efficient and portable
// mixture-of-experts communication", Dispatch: tokens travel to the experts
// with block scaling factors; Combine: the expert outputs travel back
// unquantized): as oracle_forward, except that every dispatched row and every
// row of the gate and up weight stacks is replaced by its MX-FP8 decoding
// (oracle_mxfp8_quantize, then oracle_mxfp8_dequantize) before the expert
// MLP.  The router sees the original tokens; the combine stays in dtype dt.
// down_mx = 0: the down projection on the fp64 h and the dtype-dt down weights.
// down_mx = 1: the down projection encoded too -- every row of h (32-element
// blocks along I) and every row of the [E_loc*d, I] down stack replaced by
// its MX-FP8 decoding.  Shared experts (n_shared > 0, stacks ws_*) run the
// same block-scaled MLP on every token, the token encoded like a dispatched
// row.  Same outputs as oracle_forward.
int oracle_forward_mxfp8(int T, int d, int E, int K, int I, int e_begin, int e_end, int n_shared,
                         int score, int renorm, int dt, const void* x, const void* w_router,
                         const float* bias, const void* w_gate, const void* w_up,
                         const void* w_down, const void* ws_gate, const void* ws_up,
                         const void* ws_down, int down_mx, double* out, int32_t* ids_out,
                         double* weights_out, int32_t* counts_out) {
  const int n_loc = e_end - e_begin;
  std::vector<int32_t> ids((size_t)T * K), counts(E), offsets(n_loc + 1),
      src((size_t)T * K), row_of((size_t)T * K);
  std::vector<double> w((size_t)T * K);
  oracle_route(T, d, E, K, dt, x, w_router, bias, score, renorm, ids.data(), w.data(), nullptr);
  int32_t bad = 0;
  const size_t rb = (size_t)d * dtype_bytes(dt);
  std::vector<char> xs((size_t)T * K * rb);
  const int n_rows = oracle_dispatch(T, E, K, e_begin, e_end, ids.data(), counts.data(),
                                     offsets.data(), src.data(), row_of.data(), &bad, x,
                                     xs.data(), (long long)rb);
  std::vector<int32_t> row_expert(std::max(n_rows, 1));
  for (int j = 0; j < n_loc; ++j)
    for (int r = offsets[j]; r < offsets[j + 1]; ++r) row_expert[r] = j;
  std::vector<double> y((size_t)std::max(n_rows, 1) * d);
  if (n_rows > 0)
    oracle_expert_mlp_mxfp8(n_rows, d, I, n_loc, dt, xs.data(), row_expert.data(), w_gate, w_up,
                            w_down, down_mx, y.data());
  // Shared experts: the same block-scaled MLP on every token (its input, the
  // token, encoded like a dispatched row), weight one in the combine.
  std::vector<double> ysh;
  if (n_shared > 0) {
    ysh.resize((size_t)n_shared * T * d);
    std::vector<int32_t> sh_expert(T);
    for (int s = 0; s < n_shared; ++s) {
      for (int t = 0; t < T; ++t) sh_expert[t] = s;
      oracle_expert_mlp_mxfp8(T, d, I, n_shared, dt, x, sh_expert.data(), ws_gate, ws_up, ws_down,
                              down_mx, ysh.data() + (size_t)s * T * d);
    }
  }
  oracle_combine(T, d, K, ODT_F64, y.data(), row_of.data(), ODT_F64, w.data(), n_shared,
                 n_shared > 0 ? ysh.data() : nullptr, out);
  if (ids_out) std::memcpy(ids_out, ids.data(), sizeof(int32_t) * ids.size());
  if (weights_out) std::memcpy(weights_out, w.data(), sizeof(double) * w.size());
  if (counts_out) std::memcpy(counts_out, counts.data(), sizeof(int32_t) * counts.size());
  return n_rows;
}

// Split point of the dual-microbatch forward: the token count padded up to a
// multiple of `pad`, halved.  Microbatch 0 is [0, min(mid,T)), microbatch 1 is
// [mid, T) and may be empty.
int oracle_split_point(int T, int pad) {
  const int t_pad = (T + pad - 1) / pad * pad;
  return t_pad / 2;
}

// Whether and where a batch of T tokens is split into two microbatches
// ("Dual Batch Overlap": Running with DBO -- one token threshold for batches
// of decodes only, another for batches that contain a prefill; UBatchRunner --
// the cut is at the midpoint of the padded token count, except that a uniform
// batch of multi-token queries is cut on a request boundary so that both
// halves stay uniform).  q = tokens per query of a uniform decode batch (T a
// multiple of q), or 1.  The request boundary taken is the one nearest the
// midpoint, the lower one when two are equally near.  Returns the first token
// of microbatch 1, or 0 when the batch is not split (below its threshold, or
// microbatch 1 would be empty).
int oracle_dbo_split(int T, int has_prefill, int decode_threshold, int prefill_threshold, int q,
                     int pad) {
  const int threshold = has_prefill ? prefill_threshold : decode_threshold;
  if (T < threshold) return 0;
  int split = oracle_split_point(T, pad);
  if (!has_prefill && q > 1 && T % q == 0) {
    const int below = split / q * q;
    const int above = below + q;
    split = (split - below <= above - split) ? below : above;
  }
  if (split <= 0 || split >= T) return 0;
  return split;
}

// Dual-microbatch forward: the layer run separately on the token ranges
// [0, split) and [split, T), outputs concatenated in token order (split <= 0
// or >= T: one range).
void oracle_forward_split_at(int T, int d, int E, int K, int I, int e_begin, int e_end,
                             int n_shared, int score, int renorm, int dt, const void* x,
                             const void* w_router, const float* bias, const void* w_gate,
                             const void* w_up, const void* w_down, const void* ws_gate,
                             const void* ws_up, const void* ws_down, int split, double* out) {
  const int t0 = (split <= 0 || split >= T) ? T : split;
  const size_t rb = (size_t)d * dtype_bytes(dt);
  oracle_forward(t0, d, E, K, I, e_begin, e_end, n_shared, score, renorm, dt, x, w_router, bias,
                 w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out, nullptr, nullptr, nullptr);
  if (t0 < T)
    oracle_forward(T - t0, d, E, K, I, e_begin, e_end, n_shared, score, renorm, dt,
                   static_cast<const char*>(x) + (size_t)t0 * rb, w_router, bias, w_gate, w_up,
                   w_down, ws_gate, ws_up, ws_down, out + (size_t)t0 * d, nullptr, nullptr,
                   nullptr);
}

// The midpoint split (an empty microbatch 1 runs nothing).
void oracle_forward_split(int T, int d, int E, int K, int I, int e_begin, int e_end,
                          int n_shared, int score, int renorm, int dt, const void* x,
                          const void* w_router, const float* bias, const void* w_gate,
                          const void* w_up, const void* w_down, const void* ws_gate,
                          const void* ws_up, const void* ws_down, int pad, double* out) {
  oracle_forward_split_at(T, d, E, K, I, e_begin, e_end, n_shared, score, renorm, dt, x,
                          w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                          oracle_split_point(T, pad), out);
}

// ---------------------------------------------------------------- MX-FP8 blocks
// Block-scaled 8-bit payload ("Efficient and portable mixture-of-experts
// communication", Dispatch: tokens travel with block scaling factors; the
// pages fix no format).  Reading: OCP MX-FP8 -- every 32 consecutive elements
// along a row share one power-of-two scale 2^s stored as the biased byte
// s + 127 (E8M0), and each element is an E4M3 code (1 sign, 4 exponent bits
// with bias 7, 3 mantissa bits; largest magnitude 448, subnormals down to
// 2^-9, no infinities).  s = floor(log2(max |x|)) - 8, kept within
// [-127, 127] (an all-zero block takes -127), so that the block's largest
// element lands in [256, 512); elements are x / 2^s clamped to +-448 and
// rounded to the nearest E4M3 value, ties to even.

// E4M3 code of a value already clamped to [-448, 448].
uint8_t oracle_e4m3_encode(double v) {
  const int sign = std::signbit(v) ? 0x80 : 0;
  const double a = std::fabs(v);
  if (a == 0.0) return (uint8_t)sign;
  // Spacing of E4M3 values around a: 2^-9 below 2^-6 (subnormals), else
  // 2^(e-3) in the binade [2^e, 2^(e+1)).
  int e;
  std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1): the binade starts at 2^(e-1)
  const int binade = e - 1;
  const double q = binade < -6 ? std::ldexp(1.0, -9) : std::ldexp(1.0, binade - 3);
  const double r = std::nearbyint(a / q) * q;  // round to nearest, ties to even
  if (r == 0.0) return (uint8_t)sign;
  if (r < std::ldexp(1.0, -6)) return (uint8_t)(sign | (int)(r / std::ldexp(1.0, -9)));
  int re;
  const double rf = std::frexp(r, &re);  // r = rf * 2^re, rf in [0.5, 1)
  const int exp_field = re - 1 + 7;
  const int mant = (int)((rf * 2.0 - 1.0) * 8.0);
  return (uint8_t)(sign | (exp_field << 3) | mant);
}

double oracle_e4m3_decode(uint8_t c) {
  const double sign = (c & 0x80) ? -1.0 : 1.0;
  const int ef = (c >> 3) & 0xf, m = c & 7;
  if (ef == 0) return sign * std::ldexp((double)m, -9);
  return sign * std::ldexp(1.0 + m / 8.0, ef - 7);
}

// rows x cols values (dtype dt, row pitch ld elements; cols a multiple of 32)
// -> codes [rows, cols] and scale bytes [rows, cols/32].
void oracle_mxfp8_quantize(int rows, int cols, int dt, const void* in, long long ld,
                           uint8_t* codes, uint8_t* scales) {
  const int nb = cols / 32;
  for (int r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        amax = std::max(amax, std::fabs(value_at(in, (size_t)r * ld + b * 32 + i, dt)));
      int s = -127;
      if (amax > 0.0) {
        int e;
        std::frexp(amax, &e);  // floor(log2(amax)) = e - 1
        s = std::min(127, std::max(-127, e - 1 - 8));
      }
      scales[(size_t)r * nb + b] = (uint8_t)(s + 127);
      for (int i = 0; i < 32; ++i) {
        const double v = value_at(in, (size_t)r * ld + b * 32 + i, dt) / std::ldexp(1.0, s);
        codes[(size_t)r * cols + b * 32 + i] = oracle_e4m3_encode(std::min(448.0, std::max(-448.0, v)));
      }
    }
  }
}

// The values an MX-FP8 block encodes: code value * 2^(scale - 127), in fp64.
void oracle_mxfp8_dequantize(int rows, int cols, const uint8_t* codes, const uint8_t* scales,
                             double* out) {
  const int nb = cols / 32;
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c)
      out[(size_t)r * cols + c] = oracle_e4m3_decode(codes[(size_t)r * cols + c]) *
                                  std::ldexp(1.0, (int)scales[(size_t)r * nb + c / 32] - 127);
}

// Round fp64 values to bf16 bit patterns, to nearest, ties to even, directly
// from fp64 (no intermediate fp32 rounding).  Finite inputs within the bf16
// range only.
void oracle_round_bf16(long long n, const double* in, uint16_t* out) {
  for (long long i = 0; i < n; ++i) {
    const double v = in[i];
    double r = 0.0;
    if (v != 0.0) {
      int ex;
      std::frexp(v, &ex);                   // v = f * 2^ex, 0.5 <= |f| < 1
      const int q = std::max(ex - 8, -133);  // bf16 keeps 8 significant bits
      r = std::ldexp(std::nearbyint(std::ldexp(v, -q)), q);
    }
    const float f = static_cast<float>(r);  // exact: r has at most 8 significant bits
    uint32_t bits;
    std::memcpy(&bits, &f, 4);
    out[i] = static_cast<uint16_t>(bits >> 16);
  }
}

}  // extern "C"
