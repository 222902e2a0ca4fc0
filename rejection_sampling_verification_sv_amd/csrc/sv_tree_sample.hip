// Sampling (stochastic) verification of a candidate tree: lossless
// speculative sampling over a tree whose children at each node were drawn
// independently from the draft's distribution at that node ([Topologies]
// "Speculative Decoding & Draft Model Topologies", section 4 figure: every
// node checked in one target pass, the longest accepted path kept;
// [In Production] "Speculative Decoding in Production", section 4: a tree of
// competing branches after SpecInfer; section 2 and [Topologies] section 2:
// the per-token acceptance probability min(1, p/q) and the residual
// max(0, p - q) normalised). The pages give no rule for several candidates at
// one position; the rule taken is multi-step speculative sampling, as in the
// SpecInfer paper they cite: the children of the current node are tried in
// ascending node index against the current distribution P (first the
// target's p at the node), a rejection replacing P by
// max(0, P - q) / sum(max(0, P - q)) (unchanged if that sum is 0); an
// accepted child becomes the current node; where every child is rejected, or
// at a leaf, one token is drawn from P by the inverse CDF (ascending token id,
// the final uniform).
//
// Pass 1 — tree_stats_kernel over the target rows and the draft rows of the
// call: every row cut into nrec equal chunks, one workgroup streaming each
// with the chain's one-pass statistics (per-thread online maximum and sum,
// fp64 block combine) into one (reference, sum) record; one read of every
// logit.
//
// Pass 2 — tree_sample_walk_kernel, one 1024-thread workgroup per sequence,
// all threads following the same walk (every decision is computed by every
// thread from the same shared values):
//   up front, one round trip: every node's token, uniform and two logits at
//   its parent's position, and every position's target and draft
//   log-normalisers from their records (fp64), into LDS;
//   at each node: its children by one ballot per wave over the parent array
//   (one node per thread);
//   each child's test in fp64: P_r(x) = max(0, P_{r-1}(x) - q(x)) / Z_r
//   applied r times to p(x), alpha = min(1, P_r(x) / q(x));
//   each rejection: one block-wide pass over the row pair forming
//   max(0, P_r - q) per token in fp32 (per-run totals kept in LDS) and
//   Z_{r+1} = their sum in fp64;
//   the final draw: the run holding u * total by a scan of the per-run
//   totals, then a one-wave rescan of that run.
#include <float.h>
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_stream.h"

namespace sv {

namespace {

constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / kWave;

// The distributions of the walk at one position. With p = 2^(x_t c - L_t)
// and q = 2^(x_d c - L_d) the target and draft distributions there, the
// distribution after r rejections is P_r = max(0, p - T_r q) / C_r, where
// T_0 = 0, C_0 = 1, T_{k+1} = T_k + C_k and C_{k+1} = C_k Z_{k+1}, Z_{k+1}
// the total of the residual max(0, P_k - q): by induction, max(0, P_k - q)
// = max(0, p - (T_k + C_k) q) / C_k. So every level is one difference of two
// exponentials, p / C_r and U q with U = T_r / C_r (U_{k+1} = (U_k + 1) /
// Z_{k+1}), the constants folded into the exponent offsets:
//   P_r(v)              = max(0, 2^(x_t c - L_t - log2 C_r) - 2^(x_d c - L_d + log2 U_r))
//   max(0, P_r - q)(v)  = the same with U_r + 1 in place of U_r.
// WalkRows holds those offsets (negated, as hi + lo fp32 pairs).
struct WalkRows {
  Scale c;
  float nlt_hi, nlt_lo, nld_hi, nld_lo;
};

__device__ __forceinline__ void split_neg(double v, float& hi, float& lo) {
  hi = static_cast<float>(-v);
  lo = static_cast<float>(-v - static_cast<double>(hi));
}

// Offsets for target log-normaliser Lt, draft Ld, the factor C and the
// draft factor Uq (U, or U + 1 for a residual); Uq = 0 leaves the draft term
// out. The logarithms of the factors are taken as log2_fast (about 1e-7
// absolute, the order of the fp32 weights' own rounding).
__device__ __forceinline__ WalkRows walk_rows(Scale c, double Lt, double Ld, double C, double Uq) {
  WalkRows w;
  w.c = c;
  split_neg(C == 1.0 ? Lt : Lt + log2_fast(C), w.nlt_hi, w.nlt_lo);
  if (Uq > 0.0) {
    split_neg(Uq == 1.0 ? Ld : Ld - log2_fast(Uq), w.nld_hi, w.nld_lo);
  } else {
    w.nld_hi = -INFINITY;
    w.nld_lo = 0.0f;
  }
  return w;
}

// Weight of one token in fp32: max(0, p' - q') with the offsets of w, or p'
// alone when there is no draft term (kQ false).
template <bool kQ>
__device__ __forceinline__ float walk_weight(float xt, float xd, const WalkRows& w) {
  const float p = fast_exp2(scaled_arg(xt, w.c, w.nlt_hi) + w.nlt_lo);
  if constexpr (!kQ) return p;
  const float q = fast_exp2(scaled_arg(xd, w.c, w.nld_hi) + w.nld_lo);
  return fmaxf(p - q, 0.0f);
}

// This lane's vectors of run g of a row (vectors g * kRunVecs + lane + 64 i),
// -inf past the end of the row.
template <class T>
__device__ __forceinline__ void walk_load(const uint4* row, int64_t g, int64_t nvec, uint4 (&a)[kRunLaneVecs]) {
  const int64_t v0 = g * kRunVecs + lane_id();
#pragma unroll
  for (int i = 0; i < kRunLaneVecs; ++i) {
    const int64_t v = v0 + static_cast<int64_t>(i) * kWave;
    a[i] = (v < nvec) ? row[v] : neg_inf_vec<T>();
  }
}

template <class T, bool kQ>
__device__ __forceinline__ float walk_run_sum(const uint4 (&at)[kRunLaneVecs], const uint4 (&ad)[kRunLaneVecs],
                                              const WalkRows& w) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kRunLaneVecs; ++i) {
    float xt[T::kVec], xd[T::kVec] = {};
    unpack<T>(at[i], xt);
    if constexpr (kQ) unpack<T>(ad[i], xd);
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) s += walk_weight<kQ>(xt[e], xd[e], w);
  }
  return s;
}

// One pass of the workgroup over runs [lo, hi) of the row pair: s_run[g] =
// the fp32 total of the weights of run g (wave w takes runs lo + w,
// lo + w + 16, ..., the next run's loads in flight while the current one is
// reduced), and with pub, the same total published for the sequence's other
// workgroups as walk_exchange reads it (tagged with the pass number). No
// barrier.
__device__ __forceinline__ uint64_t pass_word(uint32_t pass, float s) {
  return (static_cast<uint64_t>(pass) << 32) | static_cast<uint64_t>(__float_as_uint(s));
}

template <class T, bool kQ>
__device__ void walk_pass_q(const uint4* rt, const uint4* rd, int64_t nvec, int lo, int hi, const WalkRows& w,
                            double* s_run, uint64_t* pub, uint32_t pass) {
  const int g0 = lo + wave_id();
  if (g0 >= hi) return;
  int g = g0;
  uint4 at[kRunLaneVecs], ad[kRunLaneVecs] = {};
  walk_load<T>(rt, g, nvec, at);
  if constexpr (kQ) walk_load<T>(rd, g, nvec, ad);
  for (;;) {
    const int gn = g + kWalkWaves;
    uint4 bt[kRunLaneVecs], bd[kRunLaneVecs] = {};
    if (gn < hi) {
      walk_load<T>(rt, gn, nvec, bt);
      if constexpr (kQ) walk_load<T>(rd, gn, nvec, bd);
    }
    const float s = wave_sum_dpp(walk_run_sum<T, kQ>(at, ad, w));
    if (lane_id() == 0) {
      s_run[g] = static_cast<double>(s);
      if (pub != nullptr) publish(&pub[g], pass_word(pass, s));
    }
    if (gn >= hi) break;
    g = gn;
#pragma unroll
    for (int i = 0; i < kRunLaneVecs; ++i) {
      at[i] = bt[i];
      ad[i] = bd[i];
    }
  }
}

// One pass over the workgroup's runs of the distribution or residual that w
// describes (with the draft term when q is set).
template <class T>
__device__ void walk_pass(const uint4* rt, const uint4* rd, int64_t nvec, int lo, int hi, const WalkRows& w, bool q,
                          double* s_run, uint64_t* pub, uint32_t pass) {
  if (q)
    walk_pass_q<T, true>(rt, rd, nvec, lo, hi, w, s_run, pub, pass);
  else
    walk_pass_q<T, false>(rt, rd, nvec, lo, hi, w, s_run, pub, pass);
}

// Wait until *slot holds the totals of pass `pass` (its upper half) and
// return it; bounded like await_slot (kErrInternal and 0 on expiry or abort).
__device__ __forceinline__ uint64_t await_pass(uint64_t* slot, uint32_t pass, uint32_t* err, uint64_t* abort) {
  uint64_t v = peek(slot);
  if (static_cast<uint32_t>(v >> 32) == pass) return v;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(2);
    v = peek(slot);
    if (static_cast<uint32_t>(v >> 32) == pass) return v;
    if (peek(abort) != 0ull) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      publish(abort, 1ull);
      break;
    }
  }
  *err |= kErrInternal;
  return 0ull;
}

// The exchange slots of pass `pass` of sequence b (pass k uses buffer
// k % 2).
__device__ __forceinline__ uint64_t* pass_slots(const TreeSampleParams& P, int b, uint32_t pass) {
  return P.slots + (static_cast<int64_t>(b) * 2 + (pass & 1u)) * P.nrun;
}

// Exchange of one pass among the G workgroups of a sequence: each
// workgroup's run totals [lo, hi) went out tagged with the pass number
// (never 0) as its pass formed them; the others' are read back into s_run,
// so every workgroup then holds the totals of all runs, the same values as
// one workgroup computing them all. A workgroup publishes pass k + 2 (into
// the buffer of pass k) only after it has read every workgroup's pass
// k + 1, which each published after reading pass k.
__device__ void walk_exchange(const TreeSampleParams& P, int b, uint32_t pass, int lo, int hi, double* s_run,
                              uint32_t* s_err) {
  uint64_t* slots = pass_slots(P, b, pass);
  const int tid = static_cast<int>(threadIdx.x);
  uint32_t err = 0u;
  for (int g = tid; g < P.nrun; g += kWalkThreads) {
    if (g >= lo && g < hi) continue;
    const uint64_t v = await_pass(&slots[g], pass, &err, P.abort);
    s_run[g] = static_cast<double>(__uint_as_float(static_cast<uint32_t>(v)));
  }
  if (err != 0u) atomicOr(s_err, err);
}

// The lowest child of `node` above node `after` (children follow their
// parent, so next_child(node, node) is the first), or -1: 64 nodes per
// ballot. Every wave gets the same answer.
__device__ __forceinline__ int next_child(const int* s_par, int N, int node, int after) {
  for (int base = after + 1; base < N; base += kWave) {
    const int u = base + lane_id();
    const uint64_t m = __ballot(u < N && s_par[u] == node);
    if (m != 0ull) return base + __ffsll(static_cast<unsigned long long>(m)) - 1;
  }
  return -1;
}

// Step one of the final draw, by any wave (every wave gets the same
// answer): the run whose inclusive total first exceeds u * (sum of the run
// totals), with the remainder inside it, or the last run with weight and an
// infinite remainder if rounding leaves none; run -1 if no run has weight.
// Rounds of 64 runs, fp64 DPP scans; up to kLocRounds rounds keep their
// scans in registers for the search, more scan again.
constexpr int kLocRounds = 4;

struct RunPick {
  int g;
  double tk;
};

__device__ RunPick walk_locate(int nrun, const double* s_run, double u) {
  const int lane = lane_id();
  int found = -1, last_pos = -1;
  double prefix = 0.0;
  if (nrun <= kLocRounds * kWave) {
    double v[kLocRounds], inc[kLocRounds], rsum[kLocRounds];
    double carry = 0.0;
#pragma unroll
    for (int k = 0; k < kLocRounds; ++k) {
      const int t = k * kWave + lane;
      v[k] = (t < nrun) ? s_run[t] : 0.0;
      inc[k] = wave_scan_dpp(v[k]);
      rsum[k] = readlane_f64(inc[k], kWave - 1);
      carry += rsum[k];
    }
    const double target = u * carry;
    carry = 0.0;
#pragma unroll
    for (int k = 0; k < kLocRounds; ++k) {
      const uint64_t pos = __ballot(v[k] > 0.0);
      if (pos != 0ull) last_pos = k * kWave + 63 - __clzll(static_cast<long long>(pos));
      const uint64_t hit = __ballot(v[k] > 0.0 && carry + inc[k] > target);
      if (found < 0 && hit != 0ull) {
        const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        found = k * kWave + l;
        prefix = carry + readlane_f64(wave_exclusive_from(inc[k]), l);
      }
      carry += rsum[k];
    }
    const int g = found >= 0 ? found : last_pos;
    return RunPick{g, found >= 0 ? target - prefix : INFINITY};
  }
  double carry = 0.0;
  for (int base = 0; base < nrun; base += kWave)
    carry += readlane_f64(wave_scan_dpp(base + lane < nrun ? s_run[base + lane] : 0.0), kWave - 1);
  const double target = u * carry;
  carry = 0.0;
  for (int base = 0; base < nrun && found < 0; base += kWave) {
    const double v = base + lane < nrun ? s_run[base + lane] : 0.0;
    const double inc = wave_scan_dpp(v);
    const uint64_t pos = __ballot(v > 0.0);
    if (pos != 0ull) last_pos = base + 63 - __clzll(static_cast<long long>(pos));
    const uint64_t hit = __ballot(v > 0.0 && carry + inc > target);
    if (hit != 0ull) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      found = base + l;
      prefix = carry + readlane_f64(wave_exclusive_from(inc), l);
    }
    carry += readlane_f64(inc, kWave - 1);
  }
  const int g = found >= 0 ? found : last_pos;
  return RunPick{g, found >= 0 ? target - prefix : INFINITY};
}

// Step two, by one wave (of the workgroup whose runs include g, which read
// them in its last pass): run g rescanned in ascending token order (lane l
// holds its vectors kRunLaneVecs * l ..) with the first token whose
// cumulative weight exceeds the remainder tk (the last token with weight if
// none).
template <class T, bool kQ>
__device__ int walk_rescan_q(const uint4* rt, const uint4* rd, int64_t nvec, int g, double tk, const WalkRows& w) {
  const int lane = lane_id();
  // lane l: vectors g * kRunVecs + kRunLaneVecs * l + i, its tokens in ascending order
  const int64_t vb = static_cast<int64_t>(g) * kRunVecs + kRunLaneVecs * lane;
  constexpr int NE = kRunLaneVecs * T::kVec;
  float wv[NE];
  float lane_tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kRunLaneVecs; ++i) {
    const uint4 qt = (vb + i < nvec) ? rt[vb + i] : neg_inf_vec<T>();
    float xt[T::kVec], xd[T::kVec] = {};
    unpack<T>(qt, xt);
    if constexpr (kQ) unpack<T>((vb + i < nvec) ? rd[vb + i] : neg_inf_vec<T>(), xd);
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
      wv[i * T::kVec + e] = walk_weight<kQ>(xt[e], xd[e], w);
      lane_tot += wv[i * T::kVec + e];
    }
  }
  const double excl = wave_exclusive_from(wave_scan_dpp(static_cast<double>(lane_tot)));
  int first = -1, last = -1;
  float run = 0.0f;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    run += wv[e];
    if (wv[e] > 0.0f) {
      if (first < 0 && excl + static_cast<double>(run) > tk) first = e;
      last = e;
    }
  }
  const uint64_t hit = __ballot(first >= 0);
  const uint64_t any = __ballot(last >= 0);
  int sel = -1, e = 0;
  if (hit != 0ull) {
    sel = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    e = __builtin_amdgcn_readlane(first, sel);
  } else if (any != 0ull) {
    sel = 63 - __clzll(static_cast<long long>(any));
    e = __builtin_amdgcn_readlane(last, sel);
  }
  if (sel < 0) return -1;
  return static_cast<int>((static_cast<int64_t>(g) * kRunVecs + kRunLaneVecs * sel) * T::kVec + e);
}

template <class T>
__device__ int walk_rescan(const uint4* rt, const uint4* rd, int64_t nvec, int g, double tk, const WalkRows& w,
                           bool q) {
  return q ? walk_rescan_q<T, true>(rt, rd, nvec, g, tk, w) : walk_rescan_q<T, false>(rt, rd, nvec, g, tk, w);
}

}  // namespace

// Pass 1: workgroup c of row r streams the vectors [c nvec / nrec,
// (c + 1) nvec / nrec) of the row (target rows 0 .. B(N+1)-1, then the draft
// rows) and writes its record: the largest fl(x * c_hi) over the chunk and
// the fp64 sum of 2^(x c - reference), rounded to fp32.
template <class T>
__global__ __launch_bounds__(kStatsTPB) __attribute__((amdgpu_waves_per_eu(SV_STATS_WAVES, SV_STATS_WAVES))) void tree_stats_kernel(TreeSampleParams P) {
  constexpr int NW = kStatsTPB / kWave;
  __shared__ float s_redf[NW];
  __shared__ double s_redd[NW];
  const uint32_t nrec = static_cast<uint32_t>(P.nrec);
  const uint32_t r = blockIdx.x / nrec;
  const int64_t ch = static_cast<int64_t>(blockIdx.x - r * nrec);
  const int64_t p0 = div_nonneg(ch * P.nvec, nrec);
  const int64_t p1 = div_nonneg((ch + 1) * P.nvec, nrec);
  const int64_t R1 = static_cast<int64_t>(P.B) * (P.N + 1);
  const int64_t rr = (static_cast<int64_t>(r) < R1) ? static_cast<int64_t>(r) : static_cast<int64_t>(r) - R1;
  const char* base = static_cast<const char*>(static_cast<int64_t>(r) < R1 ? P.target : P.draft);
  const uint4* row = reinterpret_cast<const uint4*>(base + rr * P.nvec * 16);
  LazyScale sc{P.temperature, static_cast<int>(rr / (P.N + 1)), false, Scale{}};
  Running st{-INFINITY, 0.0f, 0.0f};
  flat_piece_stats<T, kStatsTPB>(row, p0, p1, sc, st);
  float MC;
  double S;
  block_combine<NW>(st, sc.get(), s_redf, s_redd, &MC, &S);
  if (threadIdx.x == 0) P.rec[static_cast<int64_t>(r) * nrec + ch] = tag_run(MC, static_cast<float>(S));
}

template <class T>
__global__ __launch_bounds__(kWalkThreads) void tree_sample_walk_kernel(TreeSampleParams P) {
  __shared__ int s_par[SV_MAX_TREE_NODES];
  __shared__ float s_lt[SV_MAX_TREE_NODES];  // node v's target and draft logits at its parent's position
  __shared__ float s_ld[SV_MAX_TREE_NODES];
  __shared__ float s_u[SV_MAX_TREE_NODES];   // node v's uniform
  __shared__ int s_path[SV_MAX_TREE_NODES];
  __shared__ double s_run2[2][kMaxWalkRuns];  // run totals, passes alternating between the two
  __shared__ double s_L[2 * (SV_MAX_TREE_NODES + 1)];  // log-normalisers: target rows, then draft rows, by position
  __shared__ int s_token;
  __shared__ int s_drawn;
  __shared__ uint32_t s_err;
  __shared__ int s_role;

  const int tid = static_cast<int>(threadIdx.x);
  // Role: sequence b, slice gi of G. With G > 1 the roles go by a ticket
  // taken when the workgroup starts, so the workgroups of a sequence start
  // one after another: a workgroup waits only for siblings that are running
  // or next in line for a compute unit, never for one stuck behind it.
  const int G = P.G;
  int b = static_cast<int>(blockIdx.x), gi = 0;
  if (G > 1) {
    if (tid == 0)
      s_role = static_cast<int>(__hip_atomic_fetch_add(&P.cnt[P.B], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    if (s_role < 0 || s_role >= P.B * G) {
      // a ticket counter not left at zero (a workspace not re-zeroed after an
      // expired wait): no role; flag it, release any waiting sibling, leave
      __shared__ int s_flag0;
      if (tid == 0) {
        raise_error(P.err_flags, kErrInternal);
        publish(P.abort, 1ull);
      }
      arrive_and_check_last(&P.cnt[P.B + 1], static_cast<uint32_t>(P.B * G), &s_flag0);
      return;
    }
    b = s_role / G;
    gi = s_role - b * G;
  }
  // this workgroup's runs of every pass
  const int lo = static_cast<int>(static_cast<int64_t>(gi) * P.nrun / G);
  const int hi = static_cast<int>(static_cast<int64_t>(gi + 1) * P.nrun / G);
  uint32_t pass = 0u;
  const int lane = lane_id();
  const int wv = wave_id();
  const int N = P.N;
  const int64_t N1 = N + 1;
  const float Tv = temperature_of(P.temperature, b);
  const Scale c = exponent_scale(Tv);
  const double c64 = static_cast<double>(c.hi) + static_cast<double>(c.lo);
  const char* tbase = static_cast<const char*>(P.target);
  const char* dbase = static_cast<const char*>(P.draft);
  const int64_t row_bytes = static_cast<int64_t>(P.V) * T::kBytes;

  if (tid == 0) {
    s_err = (!(Tv > 0.0f) || !isfinite(Tv)) ? static_cast<uint32_t>(SV_ERRF_TEMPERATURE) : 0u;
    s_token = -1;
    s_drawn = -1;
  }
  __syncthreads();
  // thread v owns node v (N <= kWalkThreads): its parent, token and uniform,
  // and its two logits at its parent's position (the position its test is
  // taken at), all loaded once, up front
  if (tid < N) {
    const int par = P.parents[tid];
    const int x = P.tokens[static_cast<int64_t>(b) * N + tid];
    s_par[tid] = par;
    s_u[tid] = P.uniforms[static_cast<int64_t>(b) * N1 + tid];
    const bool par_ok = par == -1 || (par >= 0 && par < tid);
    const bool x_ok = x >= 0 && x < P.V;
    if (!par_ok) atomicOr(&s_err, static_cast<uint32_t>(SV_ERRF_PARENT));
    if (!x_ok) atomicOr(&s_err, static_cast<uint32_t>(SV_ERRF_TOKEN));
    float lt = 0.0f, ld = 0.0f;
    if (par_ok && x_ok) {
      const int64_t row = static_cast<int64_t>(b) * N1 + (par + 1);
      lt = load_elem<T>(tbase + row * row_bytes, x);
      ld = load_elem<T>(dbase + row * row_bytes, x);
    }
    s_lt[tid] = lt;
    s_ld[tid] = ld;
  }
  // every position's log-normalisers L = M + log2 Z of its target and draft
  // rows from their records (M the largest reference, Z the fp64 sum of
  // sum * 2^(ref - M) in record order; NaN for a row without finite
  // statistics), one row per thread
  for (int q = tid; q < 2 * static_cast<int>(N1); q += kWalkThreads) {
    const int64_t pos = q < N1 ? q : q - N1;
    const int64_t rec_row = (q < N1 ? 0 : static_cast<int64_t>(P.B) * N1) + static_cast<int64_t>(b) * N1 + pos;
    const uint64_t* rec = P.rec + rec_row * P.nrec;
    uint32_t e = 0u;
    float m = -INFINITY;
    for (int g = 0; g < P.nrec; ++g) {
      const uint64_t v = rec[g];
      if (v == 0ull) e |= kErrInternal;
      m = fmaxf(m, run_ref(v));
    }
    double z = 0.0;
    for (int g = 0; g < P.nrec; ++g) {
      const uint64_t v = rec[g];
      const float ref = run_ref(v);
      const float sm = run_sum(v);
      if (sm != sm) z += static_cast<double>(sm);
      else if (ref != -INFINITY && sm > 0.0f) z += static_cast<double>(sm) * ref_factor(ref, m);
    }
    if (e != 0u) atomicOr(&s_err, e);
    const bool fin = (z > 0.0) && isfinite(z) && isfinite(m);
    s_L[q] = fin ? static_cast<double>(m) + log2_fast(z) : NAN;
  }
  __syncthreads();

  int depth = 0;
  if (s_err == 0u) {  // block-uniform from here: every thread takes the same decisions
    int node = -1, pos = 0;
    int buf = 0;  // s_run2 buffer of the next pass
    for (;;) {
      const int64_t rowt = static_cast<int64_t>(b) * N1 + pos;
      const uint4* rt = reinterpret_cast<const uint4*>(tbase + rowt * row_bytes);
      const uint4* rd = reinterpret_cast<const uint4*>(dbase + (rowt)*row_bytes);
      const double Lt = s_L[pos], Ld = s_L[N1 + pos];
      if (!isfinite(Lt) || !isfinite(Ld)) {
        if (tid == 0) s_err |= SV_ERRF_NONFINITE;
        break;
      }
      // P_r at this position as (C_r, U_r), P_0 = p (see WalkRows), with
      // iC = 1 / C_r
      double C = 1.0, iC = 1.0, U = 0.0;
      bool taken = false, resid_totals = false;
      WalkRows wl{};  // the offsets of the last pass (its residual)
      double* run = s_run2[buf];
      for (int kid = next_child(s_par, N, node, node); kid >= 0; kid = next_child(s_par, N, node, kid)) {
        const double ap = static_cast<double>(s_lt[kid]) * c64 - Lt;
        const double aq = static_cast<double>(s_ld[kid]) * c64 - Ld;
        const double q = exp2_split(aq);
        // P_r(x) = max(0, p(x) / C_r - U_r q(x))
        const double pc = exp2_split(ap) * iC;
        const double val = (U > 0.0) ? fmax(pc - U * q, 0.0) : pc;
        // u < alpha = min(1, P_r(x) / q(x)) (1 where q vanishes, 0 where P_r
        // does), tested as u q < P_r(x): no division
        const double uk = static_cast<double>(s_u[kid]);
        if (val > 0.0 && uk < 1.0 && (q > 0.0 ? uk * q < val : true)) {
          node = kid;
          pos = node + 1;
          if (tid == 0) s_path[depth] = node;
          ++depth;
          taken = true;
          break;
        }
        // rejected: the residual max(0, P_r - q), per run and in total. A
        // pass writes the buffer the previous pass did not, so a wave may
        // start it while others still sum the previous one.
        run = s_run2[buf];
        buf ^= 1;
        ++pass;
        wl = walk_rows(c, Lt, Ld, C, U + 1.0);
        walk_pass<T>(rt, rd, P.nvec, lo, hi, wl, true, run, G > 1 ? pass_slots(P, b, pass) : nullptr, pass);
        __syncthreads();
        if (G > 1) {
          walk_exchange(P, b, pass, lo, hi, run, &s_err);
          __syncthreads();
        }
        // every wave sums the run totals itself, in the same order, and
        // moves on to P_{r+1} = max(0, P_r - q) / Z
        double z = 0.0;
        for (int g = lane; g < P.nrun; g += kWave) z += run[g];
        const double Zr = wave_sum_f64_dpp(z);
        if (Zr >= static_cast<double>(FLT_MIN)) {
          const double iZ = 1.0 / Zr;
          U = (U + 1.0) * iZ;
          C *= Zr;
          iC *= iZ;
          resid_totals = true;
        } else {
          resid_totals = false;  // a residual of no (representable) mass: P unchanged
        }
      }
      if (taken) continue;
      if (s_err != 0u) break;  // an expired exchange wait
      // no child accepted (or a leaf): draw from P_r at this position
      const double u = static_cast<double>(P.uniforms[static_cast<int64_t>(b) * N1 + N]);
      // The run is located by every wave (the same answer everywhere); the
      // workgroup whose runs include it (it read them in its last pass) draws.
      if (resid_totals) {  // run holds the totals of the last residual, proportional to P_r
        if (wv == 0) {
          const RunPick pick = walk_locate(P.nrun, run, u);
          if (lane == 0) s_drawn = pick.g;
          if (pick.g >= lo && pick.g < hi) {
            const int t = walk_rescan<T>(rt, rd, P.nvec, pick.g, pick.tk, wl, true);
            if (lane == 0) s_token = t;
          }
        }
      } else {
        run = s_run2[buf];
        ++pass;
        const WalkRows w = walk_rows(c, Lt, Ld, C, U);
        walk_pass<T>(rt, rd, P.nvec, lo, hi, w, U > 0.0, run, G > 1 ? pass_slots(P, b, pass) : nullptr, pass);
        __syncthreads();
        if (G > 1) {
          walk_exchange(P, b, pass, lo, hi, run, &s_err);
          __syncthreads();
        }
        if (wv == 0) {
          const RunPick pick = walk_locate(P.nrun, run, u);
          if (lane == 0) s_drawn = pick.g;
          if (pick.g >= lo && pick.g < hi) {
            const int t = walk_rescan<T>(rt, rd, P.nvec, pick.g, pick.tk, w, U > 0.0);
            if (lane == 0) s_token = t;
          }
        }
      }
      break;
    }
  }
  __syncthreads();
  const int drawn_run = s_drawn;  // the run the token is drawn from (-1: none, or the walk ended early)
  // no token with weight in a distribution that passed the normaliser checks
  // would take every weight underflowing: reported as a zero normaliser
  const uint32_t err =
      s_err | ((s_err == 0u && drawn_run < 0) ? static_cast<uint32_t>(SV_ERRF_NONFINITE) : 0u);
  const bool bad = err != 0u;
  // the drawn token by the workgroup that drew it (by workgroup 0 when there
  // is none), the rest of the sequence's outputs by workgroup 0
  const bool draws = drawn_run >= 0 ? (drawn_run >= lo && drawn_run < hi) : (gi == 0);
  if (draws && tid == 0) P.next_token[b] = bad ? -1 : s_token;
  if (gi == 0) {
    if (tid == 0) {
      P.accept_len[b] = bad ? -1 : depth;
      raise_error(P.err_flags, err);
    }
    for (int i = tid; i < N; i += kWalkThreads)
      P.path_nodes[static_cast<int64_t>(b) * N + i] = (!bad && i < depth) ? s_path[i] : -1;
  } else if (tid == 0) {
    raise_error(P.err_flags, s_err);  // an expired wait of this workgroup
  }
  // Every record of the sequence's rows (and every exchange slot) has been
  // read once all its workgroups are here: the last one leaves them zero.
  if (G > 1) {
    __shared__ int s_flag;
    if (arrive_and_check_last(&P.cnt[b], static_cast<uint32_t>(G), &s_flag)) {
      const int64_t per = N1 * P.nrec;
      uint64_t* rec_t = P.rec + static_cast<int64_t>(b) * per;
      uint64_t* rec_d = P.rec + (static_cast<int64_t>(P.B) + b) * per;
      for (int64_t i = tid; i < per; i += kWalkThreads) {
        rec_t[i] = 0ull;
        rec_d[i] = 0ull;
      }
      for (int i = tid; i < 2 * P.nrun; i += kWalkThreads) clear_slot(&P.slots[static_cast<int64_t>(b) * 2 * P.nrun + i]);
      reset_counter(&P.cnt[b]);
    }
    // the last workgroup of the launch returns the ticket counter to zero
    if (arrive_and_check_last(&P.cnt[P.B + 1], static_cast<uint32_t>(P.B * G), &s_flag) && tid == 0) {
      __hip_atomic_store(&P.cnt[P.B], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&P.cnt[P.B + 1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    const int64_t per = N1 * P.nrec;
    uint64_t* rec_t = P.rec + static_cast<int64_t>(b) * per;
    uint64_t* rec_d = P.rec + (static_cast<int64_t>(P.B) + b) * per;
    for (int64_t i = tid; i < per; i += kWalkThreads) {
      rec_t[i] = 0ull;
      rec_d[i] = 0ull;
    }
  }
}

hipError_t launch_tree_sample(const TreeSampleParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream) {
  const uint32_t grid_a = static_cast<uint32_t>(2LL * p.B * (p.N + 1) * p.nrec);  // checked on the host
  if (dtype == SV_DTYPE_BF16)
    launch_stream_pass(tree_stats_kernel<BF16>, dim3(grid_a), dim3(kStatsTPB), stream, ev, p);
  else
    launch_stream_pass(tree_stats_kernel<F32>, dim3(grid_a), dim3(kStatsTPB), stream, ev, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t grid = static_cast<uint32_t>(p.B) * static_cast<uint32_t>(p.G);
  if (dtype == SV_DTYPE_BF16)
    hipLaunchKernelGGL(tree_sample_walk_kernel<BF16>, dim3(grid), dim3(kWalkThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(tree_sample_walk_kernel<F32>, dim3(grid), dim3(kWalkThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
