// Chain verification kernels (modified rejection sampling over K proposals).
//
// Pass 1 — statistics. Streams every logit row of the call once (the K+1
// target rows and K draft rows of each sequence) with coalesced 16-byte loads.
// Each thread keeps the running maximum m of its logits and the sum of
// 2^(x*c - m*c), c = log2(e)/T (one pass: a batch of 32 values is reduced to
// its maximum first, the sum is rescaled once per batch, then the batch's
// exponentials are added). Each block combines its threads in fp64 and stores
// one (reference, sum) pair per row piece. Two layouts:
//   chain_stats_flat_kernel: rows on 16-byte boundaries (the usual case); the
//     flattened vector space of all rows is cut into equal ranges, one per
//     block, so every block streams the same number of bytes;
//   chain_stats_rows_kernel: any row alignment; one block per (row, segment).
//
// Pass 2 — chain_decide_kernel, one workgroup per sequence: combines the
// pieces of the sequence's 2K+1 rows into their log-normalisers
// L = log2 sum_v 2^(x_v c) (fp64), forms p_k(x_k) and q_k(x_k) in fp64,
// alpha_k = min(1, p/q), accepts while u_k < alpha_k and takes j = the first
// rejection with a wave ballot; writes the accepted prefix and a sampling plan.
//   [Topologies] "Speculative Decoding & Draft Model Topologies", section 2
//   (acceptance-probability equation, timeline figure steps 2-3);
//   [In Production] "Speculative Decoding in Production", section 2.
//
// Pass 3 — chain_sample_kernel, one workgroup per (sequence, group of tiles):
//   1. re-reads its tiles of row j (target, and draft when j < K), forms the
//      weights max(0, p_j - q_j) (or p_K for the bonus draw) and publishes
//      each tile's total;
//   2. the last workgroup of the sequence scans the tile totals, finds the
//      tile holding u_K * total, rescans it with a block-wide prefix sum and
//      picks the first token whose cumulative weight exceeds it.
//      [Topologies] section 2 (residual equation, step 4); [At Scale]
//      "Speculative Decoding at Scale", section 1; [Draft-and-Verify]
//      "Speculative Decoding for LLM Inference", "The draft-and-verify loop"
//      (the bonus token when every proposal is kept).
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
  // Rescale the running sum to the new maximum (branch-free: a factor of 1
  // when the maximum did not move, 0 while nothing finite had been seen).
  const float m_new = fmaxf(st.mx, bm);
  const float scale = (st.mx == -INFINITY) ? 0.0f : fast_exp2(st.mx * c.hi - m_new * c.hi);
  st.mx = m_new;
  const float neg_m = neg_reference(m_new, c);
  // four partial sums, pairwise inside each group of 8
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < N; g += 8) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (g + i < N) ? fast_exp2(scaled_arg(x[g + i], c, neg_m)) : 0.0f;
    acc[(g / 8) & 3] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }
  st.s = st.s * scale + ((acc[0] + acc[1]) + (acc[2] + acc[3]));
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

// Block-wide combine of the threads' running states into (reference, sum):
// the largest fl(mx*c_hi), and the fp64 sum of each thread's sum rescaled to it.
__device__ __forceinline__ void block_combine(const Running& st, Scale c, float* s_redf, double* s_redd, float* MC,
                                              double* S) {
  const float mc = (st.mx == -INFINITY) ? -INFINITY : st.mx * c.hi;
  *MC = block_max(mc, s_redf);
  double sd = 0.0;
  if (mc != -INFINITY) sd = static_cast<double>(st.s * fast_exp2(mc - *MC));
  *S = block_sum(sd, s_redd);
}

// 16 bytes of -inf logits (a padding vector contributes exactly 0).
template <class T>
__device__ __forceinline__ uint4 neg_inf_vec();
template <>
__device__ __forceinline__ uint4 neg_inf_vec<BF16>() {
  return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
}
template <>
__device__ __forceinline__ uint4 neg_inf_vec<F32>() {
  return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
}

template <class T>
__device__ __forceinline__ void add_batch(Running& st, const uint4 (&raw)[kStatsUnroll], Scale c) {
  float x[kStatsUnroll * T::kVec];
#pragma unroll
  for (int u = 0; u < kStatsUnroll; ++u) unpack<T>(raw[u], &x[u * T::kVec]);
  running_add(st, x, c);
}

// One thread's share of the vectors [p0, p1) of a row: full batches of
// kStatsUnroll vectors per thread without any masking, then one ragged batch
// whose missing vectors are replaced by -inf.
template <class T>
__device__ __forceinline__ void flat_piece_stats(const uint4* body, int64_t p0, int64_t p1, Scale c, Running& st) {
  constexpr int U = kStatsUnroll;
  constexpr int64_t STEP = static_cast<int64_t>(kThreads) * U;
  const int64_t nfull = (p1 - p0) / STEP;
  const uint4* ptr = body + p0 + threadIdx.x;
#pragma unroll 1
  for (int64_t i = 0; i < nfull; ++i, ptr += STEP) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = ptr[u * kThreads];
    add_batch<T>(st, raw, c);
  }
  const int64_t rest = (p1 - p0) - nfull * STEP;  // vectors in the ragged batch
  if (rest > 0) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = static_cast<int64_t>(u) * kThreads + threadIdx.x;
      raw[u] = (k < rest) ? ptr[u * kThreads] : neg_inf_vec<T>();
    }
    add_batch<T>(st, raw, c);
  }
}


}  // namespace

// ---------------------------------------------------------------- pass 1

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void chain_stats_rows_kernel(ChainParams P) {
  __shared__ float s_redf[kWaves];
  __shared__ double s_redd[kWaves];
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
      raw[u] = (vi < v1) ? body[vi] : neg_inf_vec<T>();
    }
    add_batch<T>(st, raw, c);
  }
  if (seg == P.nseg - 1 && tid < tail) running_add1(st, load_elem<T>(row, head + nvec * VEC + tid), c);

  float MC;
  double S;
  block_combine(st, c, s_redf, s_redd, &MC, &S);
  if (tid == 0) {
    publish(&P.part_m[blk], tag_float(MC));
    publish(&P.part_s[blk], tag_nonneg_double(S));
  }
}

namespace {

// The flattened layout: chunk g covers the vectors [g*per, (g+1)*per) of the
// concatenation of all rows, streamed as one piece per row it touches; each
// piece's (reference, sum) goes to slot g * fl_kmax + (row - first row).
template <class T>
__device__ __forceinline__ void stats_chunk(const ChainParams& P, int64_t g) {
  __shared__ float s_redf[kWaves];
  __shared__ double s_redd[kWaves];
  const int R = 2 * P.K + 1;
  const int64_t nvec = P.fl_nvec;
  const int64_t per = P.fl_per;
  const int64_t total = static_cast<int64_t>(P.B) * R * nvec;
  const int64_t lo = g * per;
  const int64_t hi = min(total, lo + per);
  const int64_t row_lo = lo / nvec;
  const int64_t row_hi = (hi - 1) / nvec;
  for (int64_t row = row_lo; row <= row_hi; ++row) {
    const int b = static_cast<int>(row / R);
    const int r = static_cast<int>(row % R);
    const int64_t p0 = max(lo, row * nvec) - row * nvec;
    const int64_t p1 = min(hi, (row + 1) * nvec) - row * nvec;
    const uint4* body = static_cast<const uint4*>(chain_row<T>(P, b, r));
    const Scale c = exponent_scale(temperature_of(P.temperature, b));
    Running st{-INFINITY, 0.0f};
    flat_piece_stats<T>(body, p0, p1, c, st);
    float MC;
    double S;
    block_combine(st, c, s_redf, s_redd, &MC, &S);
    if (threadIdx.x == 0) {
      const int64_t slot = g * P.fl_kmax + (row - row_lo);
      publish(&P.part_m[slot], tag_float(MC));
      publish(&P.part_s[slot], tag_nonneg_double(S));
    }
  }
}

}  // namespace

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void chain_stats_flat_kernel(ChainParams P) {
  stats_chunk<T>(P, blockIdx.x);
}

// ---------------------------------------------------------------- pass 2

namespace {

// a / b for non-negative 64-bit values, in 32-bit arithmetic when both fit
// (a hardware-friendly path for every realistic size).
__device__ __forceinline__ int64_t div_nonneg(int64_t a, int64_t b) {
  if (((a | b) >> 32) == 0) return static_cast<int64_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(b));
  return a / b;
}

// Slot index of piece `p` of global row `grow`, or -1 past its last piece.
__device__ __forceinline__ int64_t piece_slot(const ChainParams& P, int64_t grow, int p) {
  if (P.fl_blocks > 0) {
    const int64_t nvec = P.fl_nvec, per = P.fl_per;
    const int64_t gg = div_nonneg(grow * nvec, per) + p;
    if (gg > div_nonneg((grow + 1) * nvec - 1, per)) return -1;
    return gg * P.fl_kmax + (grow - div_nonneg(gg * per, nvec));
  }
  return p < P.nseg ? grow * P.nseg + p : -1;
}

// The sampling plan travels as kPlanWords tagged 32-bit payloads (each word
// is (1 << 32) | payload, never zero), so a reader can wait for each word.
__device__ __forceinline__ void publish_plan(const ChainParams& P, int b, const SeqPlan& pl) {
  uint32_t w[kPlanWords];
  static_assert(sizeof(SeqPlan) == 4 * kPlanWords, "plan layout");
  __builtin_memcpy(w, &pl, sizeof(SeqPlan));
  for (int i = 0; i < kPlanWords; ++i) publish(&P.plan_w[static_cast<int64_t>(b) * kPlanWords + i], (1ull << 32) | w[i]);
}

__device__ __forceinline__ SeqPlan await_plan(const ChainParams& P, int b, uint32_t* err) {
  uint64_t v[kPlanWords];
  await_run(P.plan_w + static_cast<int64_t>(b) * kPlanWords, v, err, P.abort);
  uint32_t w[kPlanWords];
#pragma unroll
  for (int i = 0; i < kPlanWords; ++i) w[i] = static_cast<uint32_t>(v[i]);
  SeqPlan pl;
  __builtin_memcpy(&pl, w, sizeof(SeqPlan));
  return pl;
}

// Largest number of statistics pieces of any row (host and device agree).
__device__ __forceinline__ int max_pieces(const ChainParams& P) {
  if (P.fl_blocks > 0) return static_cast<int>(div_nonneg(P.fl_nvec + P.fl_per - 2, P.fl_per)) + 1;
  return P.nseg;
}

}  // namespace

// The decision of one sequence: the rows' log-normalisers (one wave
// per row, rows spread over the waves), the drafted tokens' logits gathered
// by the last wave meanwhile, then p_k(x_k), q_k(x_k) in fp64, alpha_k =
// min(1, p/q), acceptance while u_k < alpha_k and j = the first rejection
// (wave ballot). Writes accept_len, the accepted prefix of out_tokens,
// p_draft / q_draft, the error bits, and the sampling plan.
namespace {

template <class T>
__device__ void decide_seq(const ChainParams& P, int b) {
  __shared__ double s_L[2 * SV_MAX_K + 1];
  __shared__ float s_lt[kWave], s_ld[kWave], s_u[kWave];
  __shared__ int s_x[kWave];
  __shared__ uint32_t s_err;
  __shared__ int s_j;
  const int K = P.K;
  const int R = 2 * K + 1;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const Scale c = exponent_scale(temperature_of(P.temperature, b));
  if (tid == 0) {
    s_err = 0u;
    s_j = K;
  }
  __syncthreads();

  uint32_t err = 0u;
  if (wave_id() == kWaves - 1) {  // gathers
    const int k = lane;
    if (k < K) {
      const int x = P.tokens[static_cast<int64_t>(b) * K + k];
      s_x[k] = x;
      s_u[k] = P.uniforms[static_cast<int64_t>(b) * (K + 1) + k];
      if (x < 0 || x >= P.V) {
        err |= SV_ERRF_TOKEN;
      } else {
        s_lt[k] = load_elem<T>(chain_row<T>(P, b, k), x);
        s_ld[k] = load_elem<T>(chain_row<T>(P, b, K + 1 + k), x);
      }
    }
  }
  // Rows' log-normalisers: a group of G lanes per row (G a power of two that
  // covers the row's pieces, up to a wave), all pieces loaded in one round.
  // Group max of the references M, each lane rescales its sum by 2^(m - M) in
  // fp64, group sum Z, L = M + log2 Z. The consumed pieces are set to zero.
  {
    const int pmax = max_pieces(P);
    int G = 1;
    while (G < pmax && G < kWave) G <<= 1;
    const int rows_per_round = kThreads / G;
    for (int r0 = 0; r0 < R; r0 += rows_per_round) {
      const int r = r0 + tid / G;
      const int gl = tid % G;
      const bool row_ok = r < R;
      const int64_t grow = static_cast<int64_t>(b) * R + r;
      float mf = -INFINITY;  // reference of the folded sum zf (pieces beyond four per lane)
      double zf = 0.0;
      float ms[4];
      double ss[4];
      int64_t sl[4];
      int n = 0;
      // pieces gl, gl+G, ... of this row (one round when G >= pieces): the
      // first four of each lane are loaded together, any further ones folded
      // in one at a time
      uint64_t rm[4], rs[4];
      for (int p = gl; row_ok && p < pmax; p += G) {
        const int64_t s = piece_slot(P, grow, p);
        if (s < 0) break;
        if (n < 4) {
          sl[n] = s;
          rm[n] = peek(&P.part_m[s]);
          rs[n] = peek(&P.part_s[s]);
          ++n;
        } else {
          const float mm = untag_float(await_slot(&P.part_m[s], &err, P.abort));
          const double sv = untag_nonneg_double(await_slot(&P.part_s[s], &err, P.abort));
          if (mm != -INFINITY) {
            if (mm > mf) {
              zf = (mf == -INFINITY ? 0.0 : zf * exp2(static_cast<double>(mf) - static_cast<double>(mm))) + sv;
              mf = mm;
            } else {
              zf += sv * exp2(static_cast<double>(mm) - static_cast<double>(mf));
            }
          }
          clear_slot(&P.part_m[s]);
          clear_slot(&P.part_s[s]);
        }
      }
      for (int i = 0; i < n; ++i) {
        if (rm[i] == 0ull) rm[i] = await_slot(&P.part_m[sl[i]], &err, P.abort);
        if (rs[i] == 0ull) rs[i] = await_slot(&P.part_s[sl[i]], &err, P.abort);
        ms[i] = untag_float(rm[i]);
        ss[i] = untag_nonneg_double(rs[i]);
      }
      float M = mf;
      for (int i = 0; i < n; ++i) M = fmaxf(M, ms[i]);
      for (int o = 1; o < G; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
      double zl = (mf == -INFINITY) ? 0.0 : zf * exp2(static_cast<double>(mf) - static_cast<double>(M));
      for (int i = 0; i < n; ++i) {
        if (ms[i] != -INFINITY) zl += ss[i] * exp2(static_cast<double>(ms[i]) - static_cast<double>(M));
        clear_slot(&P.part_m[sl[i]]);  // consumed: leave the workspace zero
        clear_slot(&P.part_s[sl[i]]);
      }
      for (int o = 1; o < G; o <<= 1) zl += __shfl_xor(zl, o, kWave);
      if (row_ok && gl == 0) {
        if (!(zl > 0.0) || !isfinite(zl) || !isfinite(M)) err |= SV_ERRF_NONFINITE;
        s_L[r] = static_cast<double>(M) + log2(zl);
      }
    }
  }
  if (err != 0u) atomicOr(&s_err, err);
  __syncthreads();

  const double c64 = static_cast<double>(c.hi) + static_cast<double>(c.lo);
  if (tid < kWave) {
    const int k = tid;
    uint32_t e = 0u;
    bool reject = false;
    const float Tv = temperature_of(P.temperature, b);
    if (!(Tv > 0.0f) || !isfinite(Tv)) e |= SV_ERRF_TEMPERATURE;
    if (k < K) {
      const int x = s_x[k];
      float pf = NAN, qf = NAN;
      if (x >= 0 && x < P.V) {
        const double p = exp2(static_cast<double>(s_lt[k]) * c64 - s_L[k]);
        const double q = exp2(static_cast<double>(s_ld[k]) * c64 - s_L[K + 1 + k]);
        const double alpha = (p > 0.0) ? ((q > 0.0) ? fmin(1.0, p / q) : 1.0) : 0.0;
        reject = !(static_cast<double>(s_u[k]) < alpha);
        pf = static_cast<float>(p);
        qf = static_cast<float>(q);
      }
      if (P.p_draft != nullptr) P.p_draft[static_cast<int64_t>(b) * K + k] = pf;
      if (P.q_draft != nullptr) P.q_draft[static_cast<int64_t>(b) * K + k] = qf;
    }
    if (e != 0u) atomicOr(&s_err, e);
    const uint64_t rej = __ballot(reject);
    if (tid == 0) s_j = (rej != 0ull) ? (__ffsll(static_cast<unsigned long long>(rej)) - 1) : K;
  }
  __syncthreads();

  const bool bad = s_err != 0u;
  const int j = s_j;
  for (int i = tid; i <= K; i += kThreads) {
    if (i == j && !bad) continue;  // the drawn token: written by the sampling pass
    P.out_tokens[static_cast<int64_t>(b) * (K + 1) + i] = (bad || i > j) ? -1 : s_x[i];
  }
  if (tid == 0) {
    P.accept_len[b] = bad ? -1 : j;
    if (bad && P.residual_mass != nullptr) P.residual_mass[b] = -1.0f;
    raise_error(P.err_flags, s_err);
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
    publish_plan(P, b, pl);
  }
  __syncthreads();
}

}  // namespace

// The decision, one block per sequence (the three-kernel schedule).
template <class T>
__global__ __launch_bounds__(kThreads) void chain_decide_kernel(ChainParams P) {
  decide_seq<T>(P, blockIdx.x);
}

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

// One thread's kSampleEPT logits of a tile, for the target row and (when
// sampling from the residual) the draft row.
struct TileData {
  float xt[kSampleEPT];
  float xd[kSampleEPT];
};

template <class T>
__device__ __forceinline__ void tile_load(const SampleRows& S, int64_t tile, int V, TileData& d) {
  const int64_t e0 = tile * kSampleTile + static_cast<int64_t>(threadIdx.x) * kSampleEPT;
  load_ept<T>(S.t, e0, V, d.xt);
  if (S.d != nullptr) load_ept<T>(S.d, e0, V, d.xd);
}

// Weights of this thread's kSampleEPT tokens, and their running fp32 sum (the
// same operations in the same order wherever it is called).
//   bonus / p only:  w = p_t(v) = 2^(x_t c - L_t)
//   residual:        w = p_t(v) * max(0, 1 - 2^((x_d - x_t) c - (L_d - L_t)))
//                      = max(0, p_t(v) - p_d(v))
// The ratio form keeps the exponent small exactly where p_t and p_d nearly
// cancel, and any rounding common to all weights cancels in the draw.
__device__ __forceinline__ float tile_compute(const SampleRows& S, const TileData& d, float (&w)[kSampleEPT]) {
  float pt[kSampleEPT];
#pragma unroll
  for (int i = 0; i < kSampleEPT; ++i) pt[i] = fast_exp2(scaled_arg(d.xt[i], S.c, S.neg_lt_hi) + S.neg_lt_lo);
  if (S.d != nullptr) {
#pragma unroll
    for (int i = 0; i < kSampleEPT; ++i) {
      const float dx = d.xd[i] - d.xt[i];
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
__device__ __forceinline__ float tile_weights(const SampleRows& S, int64_t tile, int V, float (&w)[kSampleEPT]) {
  TileData d;
  tile_load<T>(S, tile, V, d);
  return tile_compute(S, d, w);
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
  //     With at most 64 tiles the totals stay in registers between the passes.
  if (tid < kWave) {
    uint32_t err = 0u;
    const bool one_chunk = P.ntiles <= kWave;
    double v0 = (one_chunk && lane < P.ntiles) ? untag_nonneg_double(await_slot(&ts[lane], &err, P.abort)) : 0.0;
    double carry = 0.0;
    int last_pos = -1;
    for (int base = 0; base < P.ntiles; base += kWave) {
      const int t = base + lane;
      const double v = one_chunk ? v0 : ((t < P.ntiles) ? untag_nonneg_double(await_slot(&ts[t], &err, P.abort)) : 0.0);
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
      const double v = one_chunk ? v0 : ((t < P.ntiles) ? untag_nonneg_double(await_slot(&ts[t], &err, P.abort)) : 0.0);
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

// One sampling work item: tiles [4 blk, 4 blk + 4) of sequence b's row pair.
template <class T>
__device__ void sample_item(const ChainParams& P, int b, int blk) {
  constexpr int TPB = kSampleTilesPerBlock;
  __shared__ double s_red[TPB][kWaves];
  __shared__ int s_flag;
  __shared__ uint32_t s_perr;
  uint32_t perr = 0u;
  const SeqPlan pl = await_plan(P, b, &perr);
  if (threadIdx.x == 0) s_perr = perr;

  if (pl.j >= 0) {  // an invalid row has nothing to draw: its outputs are -1
    const SampleRows S = sample_rows<T>(P, b, pl, false);
    const int t0 = blk * TPB;
    TileData d[TPB];
#pragma unroll
    for (int i = 0; i < TPB; ++i)  // every load of the item in flight at once
      if (t0 + i < P.ntiles) tile_load<T>(S, t0 + i, P.V, d[i]);
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
      float w[kSampleEPT];
      const double part = (t0 + i < P.ntiles) ? wave_sum(static_cast<double>(tile_compute(S, d[i], w))) : 0.0;
      if (lane_id() == 0) s_red[i][wave_id()] = part;
    }
    __syncthreads();
    if (threadIdx.x < TPB && t0 + static_cast<int>(threadIdx.x) < P.ntiles) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += s_red[threadIdx.x][w];
      publish(&P.tile_sum[static_cast<int64_t>(b) * P.ntiles + t0 + threadIdx.x], tag_nonneg_double(tot));
    }
  }

  if (!arrive_and_check_last(&P.cnt[b], static_cast<uint32_t>(P.nblk_b), &s_flag)) return;
  if (pl.j >= 0) chain_draw<T>(P, b, pl);
  // Leave the workspace all zero for the next call, whatever its shape.
  __syncthreads();
  if (pl.j >= 0)
    for (int t = threadIdx.x; t < P.ntiles; t += kThreads) clear_slot(&P.tile_sum[static_cast<int64_t>(b) * P.ntiles + t]);
  if (threadIdx.x < kPlanWords) clear_slot(&P.plan_w[static_cast<int64_t>(b) * kPlanWords + threadIdx.x]);
  if (threadIdx.x == 0) raise_error(P.err_flags, s_perr);
  reset_counter(&P.cnt[b]);
  __syncthreads();
}

}  // namespace

template <class T>
__global__ __launch_bounds__(kThreads) void chain_sample_kernel(ChainParams P) {
  sample_item<T>(P, blockIdx.x / P.nblk_b, blockIdx.x % P.nblk_b);
}

// ---------------------------------------------------------------- launcher

template <class T>
static hipError_t launch_chain_t(const ChainParams& p, hipStream_t stream) {
  const int64_t R = 2 * static_cast<int64_t>(p.K) + 1;
  const int64_t grid_a = p.fl_blocks > 0 ? p.fl_blocks : static_cast<int64_t>(p.B) * R * p.nseg;
  const int64_t grid_b = static_cast<int64_t>(p.B) * p.nblk_b;
  if (grid_a > INT32_MAX || grid_b > INT32_MAX) return hipErrorInvalidConfiguration;
  if (p.fl_blocks > 0)
    hipLaunchKernelGGL(chain_stats_flat_kernel<T>, dim3(static_cast<uint32_t>(grid_a)), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(chain_stats_rows_kernel<T>, dim3(static_cast<uint32_t>(grid_a)), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chain_decide_kernel<T>, dim3(static_cast<uint32_t>(p.B)), dim3(kThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chain_sample_kernel<T>, dim3(static_cast<uint32_t>(grid_b)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chain(const ChainParams& p, sv_dtype dtype, hipStream_t stream) {
  return dtype == SV_DTYPE_BF16 ? launch_chain_t<BF16>(p, stream) : launch_chain_t<F32>(p, stream);
}

}  // namespace sv
