// Chain verification kernels (modified rejection sampling over K proposals).
//
// Pass 1 — chain_stats_kernel, one workgroup per (sequence, row, segment):
//   streams a segment of one logit row (the K+1 target rows and K draft rows
//   of each sequence) with coalesced 16-byte loads and keeps, per thread, the
//   running maximum m of the logits and the sum of 2^(l*c - m*c), c = log2(e)/T
//   (one-pass max/sum; the sum is rescaled only when a batch raises the max).
//   The block combines its threads in fp64 and publishes (max*c, sum). The
//   last block to finish a sequence combines all segments of its 2K+1 rows
//   and makes the decision: p_k(x_k), q_k(x_k) in fp64, alpha_k = min(1, p/q),
//   accept while u_k < alpha_k, j = first rejection (wave ballot).
//   [Topologies] "Speculative Decoding & Draft Model Topologies", section 2
//   (acceptance-probability equation, timeline figure steps 2-3);
//   [In Production] "Speculative Decoding in Production", section 2.
//
// Pass 2 — chain_sample_kernel, one workgroup per (sequence, tile group):
//   re-reads row j (target, and draft when j < K), forms the weights
//   max(0, p_j - q_j) (or p_K for the bonus draw) tile by tile, and publishes
//   each tile's total. The last block of a sequence scans the tile totals,
//   finds the tile holding u_K * total, rescans that tile with a block-wide
//   prefix sum and picks the first token whose cumulative weight exceeds it.
//   [Topologies] section 2 (residual equation, step 4); [At Scale]
//   "Speculative Decoding at Scale", section 1; [Draft-and-Verify]
//   "Speculative Decoding for LLM Inference", "The draft-and-verify loop"
//   (the bonus token when every proposal is kept).
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

template <class T>
__device__ __forceinline__ const void* chain_row(const ChainParams& P, int b, int r) {
  const char* base;
  int64_t row;
  if (r <= P.K) {
    base = static_cast<const char*>(P.target);
    row = static_cast<int64_t>(b) * (P.K + 1) + r;
  } else {
    base = static_cast<const char*>(P.draft);
    row = static_cast<int64_t>(b) * P.K + (r - P.K - 1);
  }
  return base + row * static_cast<int64_t>(P.V) * T::kBytes;
}

__device__ __forceinline__ float temperature_of(const float* temperature, int b) {
  return temperature != nullptr ? temperature[b] : 1.0f;
}

// c = log2(e) / T as an unevaluated sum of two fp32 values (c_hi carries the
// leading 24 bits, c_lo the next ones), so that exponents x*c are formed at
// the requested temperature rather than at the nearest fp32 one. c_hi is
// rounded toward zero and c_lo is kept strictly positive: an x of -inf then
// gives -inf in both products (never -inf + inf), i.e. a weight of exactly 0.
struct Scale {
  float hi;
  float lo;
};

__device__ __forceinline__ Scale exponent_scale(float T) {
  const double c = 1.4426950408889634 / static_cast<double>(T);
  float hi = __double2float_rz(c);
  // exactly representable c (c_lo would be 0): step c_hi one ulp toward zero
  if (static_cast<double>(hi) == c && hi > 0.0f) hi = __uint_as_float(__float_as_uint(hi) - 1u);
  return Scale{hi, static_cast<float>(c - static_cast<double>(hi))};
}

// The fp32 reference of a running maximum: fl(mx * c_hi), and -inf while
// nothing finite has been seen (so that -inf logits contribute 0, not NaN).
__device__ __forceinline__ float neg_reference(float mx, Scale c) {
  return mx == -INFINITY ? -INFINITY : -(mx * c.hi);
}

// x*c - m with m an fp32 reference: one product exact inside each fma.
__device__ __forceinline__ float scaled_arg(float x, Scale c, float neg_m) {
  return fmaf(x, c.lo, fmaf(x, c.hi, neg_m));
}

// Running (max, sum) of one thread. `mx` is the largest raw logit seen and
// `s` = sum of 2^(x*c - fl(mx*c_hi)) over the logits seen.
struct Running {
  float mx;
  float s;
};

template <int N>
__device__ __forceinline__ void running_add(Running& st, const float (&x)[N], Scale c) {
  float bm = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
  if (bm > st.mx) {
    st.s = (st.mx == -INFINITY) ? 0.0f : st.s * fast_exp2(st.mx * c.hi - bm * c.hi);
    st.mx = bm;
  }
  const float neg_m = neg_reference(st.mx, c);
  // pairwise within each group of 8, then sequential over the groups
  float acc = 0.0f;
#pragma unroll
  for (int g = 0; g < N; g += 8) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (g + i < N) ? fast_exp2(scaled_arg(x[g + i], c, neg_m)) : 0.0f;
    const float e01 = e[0] + e[1], e23 = e[2] + e[3], e45 = e[4] + e[5], e67 = e[6] + e[7];
    acc += (e01 + e23) + (e45 + e67);
  }
  st.s += acc;
}

__device__ __forceinline__ void running_add1(Running& st, float x, Scale c) {
  if (x > st.mx) {
    st.s = (st.mx == -INFINITY) ? 0.0f : st.s * fast_exp2(st.mx * c.hi - x * c.hi);
    st.mx = x;
  }
  st.s += fast_exp2(scaled_arg(x, c, neg_reference(st.mx, c)));
}

__device__ __forceinline__ void split(double v, float& hi, float& lo) {
  hi = static_cast<float>(v);
  lo = static_cast<float>(v - static_cast<double>(hi));
}

// ---------------------------------------------------------------- decision

template <class T>
__device__ void chain_decide(const ChainParams& P, int b, Scale c) {
  __shared__ double s_L[2 * SV_MAX_K + 1];
  __shared__ uint32_t s_err;
  __shared__ int s_j;
  const int K = P.K;
  const int R = 2 * K + 1;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_err = 0u;
    s_j = K;
  }
  __syncthreads();

  // Log-normaliser of every row at scale c: L = M + log2(sum_s S_s 2^(M_s - M)).
  for (int r = tid; r < R; r += kThreads) {
    const int64_t base = (static_cast<int64_t>(b) * R + r) * P.nseg;
    uint32_t err = 0u;
    float M = -INFINITY;
    for (int s = 0; s < P.nseg; ++s) M = fmaxf(M, untag_float(await_slot(&P.part_m[base + s], &err)));
    double Z = 0.0;
    for (int s = 0; s < P.nseg; ++s) {
      const float ms = untag_float(await_slot(&P.part_m[base + s], &err));
      const double ss = untag_nonneg_double(await_slot(&P.part_s[base + s], &err));
      if (ms != -INFINITY) Z += ss * exp2(static_cast<double>(ms) - static_cast<double>(M));
    }
    s_L[r] = static_cast<double>(M) + log2(Z);
    if (!(Z > 0.0) || !isfinite(Z) || !isfinite(M)) err |= SV_ERRF_NONFINITE;
    if (err != 0u) atomicOr(&s_err, err);
  }
  __syncthreads();

  const double c64 = static_cast<double>(c.hi) + static_cast<double>(c.lo);
  if (tid < kWave) {
    const int k = tid;
    uint32_t err = 0u;
    bool reject = false;
    const float Tv = temperature_of(P.temperature, b);
    if (!(Tv > 0.0f) || !isfinite(Tv)) err |= SV_ERRF_TEMPERATURE;
    if (k < K) {
      const int x = P.tokens[static_cast<int64_t>(b) * K + k];
      float pf = NAN, qf = NAN;
      if (x < 0 || x >= P.V) {
        err |= SV_ERRF_TOKEN;
      } else {
        const double lt = load_elem<T>(chain_row<T>(P, b, k), x);
        const double ld = load_elem<T>(chain_row<T>(P, b, K + 1 + k), x);
        const double p = exp2(lt * c64 - s_L[k]);
        const double q = exp2(ld * c64 - s_L[K + 1 + k]);
        const double alpha = (p > 0.0) ? ((q > 0.0) ? fmin(1.0, p / q) : 1.0) : 0.0;
        const double u = static_cast<double>(P.uniforms[static_cast<int64_t>(b) * (K + 1) + k]);
        reject = !(u < alpha);
        pf = static_cast<float>(p);
        qf = static_cast<float>(q);
      }
      if (P.p_draft != nullptr) P.p_draft[static_cast<int64_t>(b) * K + k] = pf;
      if (P.q_draft != nullptr) P.q_draft[static_cast<int64_t>(b) * K + k] = qf;
    }
    if (err != 0u) atomicOr(&s_err, err);
    const uint64_t rej = __ballot(reject);
    if (tid == 0) s_j = (rej != 0ull) ? (__ffsll(static_cast<unsigned long long>(rej)) - 1) : K;
  }
  __syncthreads();

  const bool bad = s_err != 0u;
  const int j = s_j;
  for (int i = tid; i <= K; i += kThreads) {
    int32_t v;
    if (bad || i > j) {
      v = -1;
    } else if (i < j) {
      v = P.tokens[static_cast<int64_t>(b) * K + i];
    } else {
      continue;  // position j: written by the sampling pass
    }
    P.out_tokens[static_cast<int64_t>(b) * (K + 1) + i] = v;
  }
  if (tid == 0) {
    P.accept_len[b] = bad ? -1 : j;
    SeqPlan pl;
    pl.j = bad ? -1 : j;
    pl.c_hi = c.hi;
    pl.c_lo = c.lo;
    split(s_L[j], pl.lt_hi, pl.lt_lo);
    if (j < K) {
      split(s_L[K + 1 + j] - s_L[j], pl.d_hi, pl.d_lo);
    } else {
      pl.d_hi = 0.0f;
      pl.d_lo = 0.0f;
    }
    pl.pad = 0.0f;
    P.plan[b] = pl;
    if (bad && P.residual_mass != nullptr) P.residual_mass[b] = -1.0f;
    raise_error(P.err_flags, s_err);
  }
}

}  // namespace

// ---------------------------------------------------------------- pass 1

template <class T>
__global__ __launch_bounds__(kThreads) void chain_stats_kernel(ChainParams P) {
  __shared__ float s_redf[kWaves];
  __shared__ double s_redd[kWaves];
  __shared__ int s_flag;
  constexpr int VEC = T::kVec;
  constexpr int U = kStatsUnroll;

  const int R = 2 * P.K + 1;
  const int64_t blk = blockIdx.x;
  const int seg = static_cast<int>(blk % P.nseg);
  const int64_t rowid = blk / P.nseg;
  const int r = static_cast<int>(rowid % R);
  const int b = static_cast<int>(rowid / R);
  const int tid = threadIdx.x;

  const void* row = chain_row<T>(P, b, r);
  const Scale c = exponent_scale(temperature_of(P.temperature, b));

  // Split the row into an unaligned head, 16-byte vectors, and a tail.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  const int head = min(static_cast<int>(((16u - (addr & 15u)) & 15u) / T::kBytes), P.V);
  const int64_t nvec = (P.V - head) / VEC;
  const int tail = static_cast<int>((P.V - head) - nvec * VEC);
  const int64_t v0 = static_cast<int64_t>(seg) * P.seg_vecs;
  const int64_t v1 = min(nvec, v0 + P.seg_vecs);
  const uint4* body = reinterpret_cast<const uint4*>(static_cast<const char*>(row) + head * T::kBytes);

  Running st{-INFINITY, 0.0f};
  if (seg == 0 && tid < head) running_add1(st, load_elem<T>(row, tid), c);

  for (int64_t base = v0 + tid; base < v1; base += static_cast<int64_t>(kThreads) * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t vi = base + static_cast<int64_t>(u) * kThreads;
      raw[u] = (vi < v1) ? body[vi] : make_uint4(0u, 0u, 0u, 0u);
    }
    float x[U * VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unpack<T>(raw[u], &x[u * VEC]);
      const int64_t vi = base + static_cast<int64_t>(u) * kThreads;
      if (vi >= v1) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) x[u * VEC + i] = -INFINITY;
      }
    }
    running_add(st, x, c);
  }

  if (seg == P.nseg - 1 && tid < tail) running_add1(st, load_elem<T>(row, head + nvec * VEC + tid), c);

  // Block combine: max of the references fl(mx*c_hi), then the fp64 sum of
  // the rescaled sums.
  const float mc = (st.mx == -INFINITY) ? -INFINITY : st.mx * c.hi;
  const float MC = block_max(mc, s_redf);
  double sd = 0.0;
  if (mc != -INFINITY) sd = static_cast<double>(st.s) * exp2(static_cast<double>(mc) - static_cast<double>(MC));
  const double S = block_sum(sd, s_redd);
  if (tid == 0) {
    publish(&P.part_m[blk], tag_float(MC));
    publish(&P.part_s[blk], tag_nonneg_double(S));
  }

  if (!arrive_and_check_last(&P.cnt_a[b], static_cast<uint32_t>(R) * P.nseg, &s_flag)) return;
  chain_decide<T>(P, b, c);
  // Leave the workspace as it was found (all zero): the partials are consumed.
  __syncthreads();
  const int64_t base = static_cast<int64_t>(b) * R * P.nseg;
  for (int64_t i = tid; i < static_cast<int64_t>(R) * P.nseg; i += kThreads) {
    clear_slot(&P.part_m[base + i]);
    clear_slot(&P.part_s[base + i]);
  }
  reset_counter(&P.cnt_a[b]);
}

// ---------------------------------------------------------------- pass 2

namespace {

// The kSampleEPT logits of one thread in a tile, -inf beyond V.
template <class T>
__device__ __forceinline__ void load_ept(const void* row, int64_t e0, int V, float (&x)[kSampleEPT]) {
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0u;
  if (aligned && e0 + kSampleEPT <= V) {
    const char* p = static_cast<const char*>(row) + e0 * T::kBytes;
#pragma unroll
    for (int v = 0; v < kSampleEPT / T::kVec; ++v) unpack<T>(load_vec(p + 16 * v), &x[v * T::kVec]);
  } else {
#pragma unroll
    for (int i = 0; i < kSampleEPT; ++i) x[i] = (e0 + i < V) ? load_elem<T>(row, e0 + i) : -INFINITY;
  }
}

struct SampleRows {
  const void* t;  // target row j
  const void* d;  // draft row j, or nullptr when drawing from p only
  Scale c;
  float neg_lt_hi, neg_lt_lo;  // -L_t
  float neg_d_hi, neg_d_lo;    // -(L_d - L_t)
};

// Weights of this thread's kSampleEPT tokens in tile `tile`, and their running
// fp32 sum (the same operations in the same order wherever it is called).
//   bonus / p only:  w = p_t(v) = 2^(x_t c - L_t)
//   residual:        w = p_t(v) * max(0, 1 - 2^((x_d - x_t) c - (L_d - L_t)))
//                      = max(0, p_t(v) - p_d(v))
// The ratio form keeps the exponent small exactly where p_t and p_d nearly
// cancel, and any rounding common to all weights cancels in the draw.
template <class T>
__device__ __forceinline__ float tile_weights(const SampleRows& S, int64_t tile, int V, float (&w)[kSampleEPT]) {
  const int64_t e0 = tile * kSampleTile + static_cast<int64_t>(threadIdx.x) * kSampleEPT;
  float xt[kSampleEPT];
  load_ept<T>(S.t, e0, V, xt);
  float pt[kSampleEPT];
#pragma unroll
  for (int i = 0; i < kSampleEPT; ++i) pt[i] = fast_exp2(scaled_arg(xt[i], S.c, S.neg_lt_hi) + S.neg_lt_lo);
  if (S.d != nullptr) {
    float xd[kSampleEPT];
    load_ept<T>(S.d, e0, V, xd);
#pragma unroll
    for (int i = 0; i < kSampleEPT; ++i) {
      const float dx = xd[i] - xt[i];
      const float ratio = fast_exp2(scaled_arg(dx, S.c, S.neg_d_hi) + S.neg_d_lo);
      w[i] = pt[i] * fmaxf(1.0f - ratio, 0.0f);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSampleEPT; ++i) w[i] = pt[i];
  }
  float run = 0.0f;
#pragma unroll
  for (int i = 0; i < kSampleEPT; ++i) run += w[i];
  return run;
}

template <class T>
__device__ __forceinline__ SampleRows sample_rows(const ChainParams& P, int b, const SeqPlan& pl, bool p_only) {
  SampleRows S;
  S.t = chain_row<T>(P, b, pl.j);
  S.d = (pl.j < P.K && !p_only) ? chain_row<T>(P, b, P.K + 1 + pl.j) : nullptr;
  S.c = Scale{pl.c_hi, pl.c_lo};
  S.neg_lt_hi = -pl.lt_hi;
  S.neg_lt_lo = -pl.lt_lo;
  S.neg_d_hi = -pl.d_hi;
  S.neg_d_lo = -pl.d_lo;
  return S;
}

// Rescan tile `tile` of the sampling row: the first token (ascending id) with
// a positive weight whose cumulative weight within the tile exceeds
// `target`; if rounding leaves none, the last token with a positive weight.
template <class T>
__device__ int draw_in_tile(const SampleRows& Sr, int tile, double target, int V, double* s_scan, int* s_redi) {
  float w[kSampleEPT];
  const float x = tile_weights<T>(Sr, tile, V, w);
  double tot;
  const double excl = block_exclusive_scan(static_cast<double>(x), s_scan, &tot);
  int first = INT_MAX;
  int lastpos = -1;
  float run = 0.0f;
#pragma unroll
  for (int i = 0; i < kSampleEPT; ++i) {
    run += w[i];
    const int idx = static_cast<int>(threadIdx.x) * kSampleEPT + i;
    if (w[i] > 0.0f) {
      if (first == INT_MAX && excl + static_cast<double>(run) > target) first = idx;
      lastpos = idx;
    }
  }
  // lowest crossing index in the tile, else the last positive weight
  const int first_all = -block_max_int(first == INT_MAX ? INT_MIN + 1 : -first, s_redi);
  const int last_all = block_max_int(lastpos, s_redi);
  const int e = (first_all >= 0 && first_all < kSampleTile) ? first_all : last_all;
  return (e >= 0) ? static_cast<int>(static_cast<int64_t>(tile) * kSampleTile + e) : -1;
}

// Draw the token: called by the last sampling block of sequence b, once every
// block of the sequence has published its tile totals.
template <class T>
__device__ void chain_draw(const ChainParams& P, int b, const SeqPlan& pl) {
  __shared__ double s_scan[kWaves];
  __shared__ int s_redi[kWaves];
  __shared__ double s_S, s_target;
  __shared__ int s_tile;
  __shared__ uint32_t s_err;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  uint64_t* ts = P.tile_sum + static_cast<int64_t>(b) * P.ntiles;
  const double u = static_cast<double>(P.uniforms[static_cast<int64_t>(b) * (P.K + 1) + P.K]);
  if (tid == 0) s_err = 0u;
  __syncthreads();

  // (1) total weight and the tile holding u * total (wave 0, fp64, tile order).
  if (tid < kWave) {
    uint32_t err = 0u;
    double carry = 0.0;
    int last_pos = -1;
    for (int base = 0; base < P.ntiles; base += kWave) {
      const int t = base + lane;
      const double v = (t < P.ntiles) ? untag_nonneg_double(await_slot(&ts[t], &err)) : 0.0;
      double inc = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const double n = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += n;
      }
      const uint64_t pos = __ballot(t < P.ntiles && v > 0.0);
      if (pos != 0ull) last_pos = base + 63 - __clzll(static_cast<long long>(pos));
      carry += __shfl(inc, kWave - 1, kWave);
    }
    const double total = carry;
    const double target = u * total;
    int found = -1;
    double prefix = 0.0;
    carry = 0.0;
    for (int base = 0; base < P.ntiles && found < 0; base += kWave) {
      const int t = base + lane;
      const double v = (t < P.ntiles) ? untag_nonneg_double(await_slot(&ts[t], &err)) : 0.0;
      double inc = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const double n = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += n;
      }
      double excl = __shfl_up(inc, 1, kWave);
      if (lane == 0) excl = 0.0;
      const uint64_t hit = __ballot(t < P.ntiles && v > 0.0 && carry + inc > target);
      if (hit != 0ull) {
        const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        found = base + l;
        prefix = carry + __shfl(excl, l, kWave);
      }
      carry += __shfl(inc, kWave - 1, kWave);
    }
    if (err != 0u) atomicOr(&s_err, err);
    if (tid == 0) {
      s_S = total;
      if (found >= 0) {
        s_tile = found;
        s_target = target - prefix;
      } else {  // rounding at the top end: the last tile with weight
        s_tile = last_pos;
        s_target = INFINITY;
      }
    }
  }
  __syncthreads();
  const double S_res = s_S;
  bool p_only = false;

  if (!(S_res > 0.0) && pl.j < P.K) {
    // A rejected position whose residual vanished in fp32: draw from p_j.
    // Two passes over the row's tiles by this block (a rare path).
    p_only = true;
    const SampleRows Sp = sample_rows<T>(P, b, pl, true);
    double total = 0.0;
    int last_pos = -1;
    for (int t = 0; t < P.ntiles; ++t) {
      float w[kSampleEPT];
      double tot;
      block_exclusive_scan(static_cast<double>(tile_weights<T>(Sp, t, P.V, w)), s_scan, &tot);
      total += tot;
      if (tot > 0.0) last_pos = t;
    }
    const double target = u * total;
    double prefix = 0.0;
    int found = -1;
    for (int t = 0; t < P.ntiles && found < 0; ++t) {
      float w[kSampleEPT];
      double tot;
      block_exclusive_scan(static_cast<double>(tile_weights<T>(Sp, t, P.V, w)), s_scan, &tot);
      if (tot > 0.0 && prefix + tot > target) found = t;
      else prefix += tot;
    }
    if (tid == 0) {
      s_tile = found >= 0 ? found : last_pos;
      s_target = found >= 0 ? target - prefix : INFINITY;
    }
    __syncthreads();
  }

  // (2) rescan the chosen tile.
  const int tile = s_tile;
  const double target = s_target;
  int token = -1;
  if (tile >= 0) token = draw_in_tile<T>(sample_rows<T>(P, b, pl, p_only), tile, target, P.V, s_scan, s_redi);
  if (tid == 0) {
    P.out_tokens[static_cast<int64_t>(b) * (P.K + 1) + pl.j] = token;
    if (P.residual_mass != nullptr) P.residual_mass[b] = (pl.j < P.K) ? static_cast<float>(S_res) : -1.0f;
    raise_error(P.err_flags, s_err);
  }
}

}  // namespace

template <class T>
__global__ __launch_bounds__(kThreads) void chain_sample_kernel(ChainParams P) {
  __shared__ double s_scan[kWaves];
  __shared__ int s_flag;
  const int b = blockIdx.x / P.nblk_b;
  const int blk = blockIdx.x % P.nblk_b;
  const SeqPlan pl = P.plan[b];

  if (pl.j >= 0) {  // an invalid row has nothing to draw: its outputs are already -1
    const SampleRows S = sample_rows<T>(P, b, pl, false);
    const int t0 = blk * P.tiles_per_block;
    const int t1 = min(P.ntiles, t0 + P.tiles_per_block);
    for (int t = t0; t < t1; ++t) {
      float w[kSampleEPT];
      const float x = tile_weights<T>(S, t, P.V, w);
      double tot;
      block_exclusive_scan(static_cast<double>(x), s_scan, &tot);
      if (threadIdx.x == 0) publish(&P.tile_sum[static_cast<int64_t>(b) * P.ntiles + t], tag_nonneg_double(tot));
    }
  }

  if (!arrive_and_check_last(&P.cnt_b[b], static_cast<uint32_t>(P.nblk_b), &s_flag)) return;
  if (pl.j >= 0) chain_draw<T>(P, b, pl);
  // Leave the workspace all zero for the next call, whatever its shape.
  __syncthreads();
  if (pl.j >= 0)
    for (int t = threadIdx.x; t < P.ntiles; t += kThreads) clear_slot(&P.tile_sum[static_cast<int64_t>(b) * P.ntiles + t]);
  if (threadIdx.x == 0) P.plan[b] = SeqPlan{};
  reset_counter(&P.cnt_b[b]);
}

// ---------------------------------------------------------------- launcher

template <class T>
static hipError_t launch_chain_t(const ChainParams& p, hipStream_t stream) {
  const int64_t R = 2 * static_cast<int64_t>(p.K) + 1;
  const int64_t grid_a = static_cast<int64_t>(p.B) * R * p.nseg;
  const int64_t grid_b = static_cast<int64_t>(p.B) * p.nblk_b;
  if (grid_a > INT32_MAX || grid_b > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(chain_stats_kernel<T>, dim3(static_cast<uint32_t>(grid_a)), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chain_sample_kernel<T>, dim3(static_cast<uint32_t>(grid_b)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chain(const ChainParams& p, sv_dtype dtype, hipStream_t stream) {
  return dtype == SV_DTYPE_BF16 ? launch_chain_t<BF16>(p, stream) : launch_chain_t<F32>(p, stream);
}

}  // namespace sv
