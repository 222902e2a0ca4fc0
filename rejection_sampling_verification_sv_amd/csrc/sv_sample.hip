// Draft-side sampling in one pass over the logits (rows on 16-byte
// boundaries): the drafter's step x ~ q(x), q = softmax(logits / T), by the
// inverse CDF over ascending token id with one caller-supplied uniform per
// row ([In Production] "Speculative Decoding in Production", section 2: the
// draft model samples each candidate; [Draft-and-Verify] "Speculative
// Decoding for LLM Inference", "The draft-and-verify loop").
//
// Pass 1 — sample_stream_kernel. Every row is cut into runs of kRunVecs
// 16-byte vectors (the row's last run may be short). One wave streams a whole
// run with non-temporal loads (lane l holds its vectors l, l + 64, ...) and
// reduces it to one record:
// ref = fl(max * c_hi) over the run, sum = sum over the run of
// 2^(x c - ref) in fp32. A workgroup takes a chunk of consecutive runs, its
// waves taking every fourth one; two runs' loads are in flight per wave.
// Only wave-level reductions: no LDS and no barrier in the stream.
//
// Pass 2 — sample_draw_kernel, one wave per row. It reads the row's records,
// forms in fp64 M = max ref, Z = sum of sum * 2^(ref - M), and the inclusive
// scan of the runs' weights in run order; the run holding u * Z is the first
// whose inclusive weight exceeds it (rounding at the top end: the last run
// with weight). It re-reads that one run, recomputes its weights with the
// same fp32 operations as pass 1, scans them and picks the first token whose
// cumulative weight exceeds the remainder (rounding: the last token with
// weight). It then returns the row's records to zero.
#include <hip/hip_ext.h>
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

__device__ __forceinline__ const uint4* sample_row(const SampleParams& P, int64_t r, int eb) {
  return reinterpret_cast<const uint4*>(static_cast<const char*>(P.logits) + r * P.V * eb);
}

// This lane's vectors of run g (vectors g * kRunVecs + lane + i * 64), -inf
// past the end of the row.
template <class T>
__device__ __forceinline__ void load_run(const uint4* row, int64_t g, int64_t nvec, uint4 (&a)[kRunLaneVecs]) {
  const int64_t v0 = g * kRunVecs + lane_id();
#pragma unroll
  for (int i = 0; i < kRunLaneVecs; ++i) {
    const int64_t v = v0 + static_cast<int64_t>(i) * kWave;
    a[i] = (v < nvec) ? stream_load(row + v) : neg_inf_vec<T>();
  }
  // keep the loads ahead of the reduction that follows them
  __builtin_amdgcn_sched_barrier(0);
}

// Reduce one run held by the wave to its record; lane 0 stores it.
// The logits are widened twice from the raw vectors (for the maximum, then
// for the exponentials) rather than held as floats across the wave
// reduction: the empty asm makes the second widening opaque to common
// subexpression elimination, so only the raw vectors stay live.
template <class T>
__device__ __forceinline__ void finish_run(const uint4 (&a)[kRunLaneVecs], Scale c, uint64_t* slot) {
  constexpr int NV = T::kVec;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRunLaneVecs; ++i) {
    float t[NV];
    unpack<T>(a[i], t);
#pragma unroll
    for (int e = 0; e < NV; ++e) m = fmaxf(m, t[e]);
  }
  m = wave_max_dpp(m);
  const float neg_m = neg_reference(m, c);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kRunLaneVecs; ++i) {
    uint4 raw = a[i];
    asm volatile("" : "+v"(raw.x), "+v"(raw.y), "+v"(raw.z), "+v"(raw.w));
    float t[NV];
    unpack<T>(raw, t);
    float e[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) e[k] = fast_exp2(scaled_arg(t[k], c, neg_m));
    float s4 = (e[0] + e[1]) + (e[2] + e[3]);
    if constexpr (NV == 8) s4 += (e[4] + e[5]) + (e[6] + e[7]);
    acc[i & 3] += s4;
  }
  const float s = wave_sum_dpp((acc[0] + acc[1]) + (acc[2] + acc[3]));
  // ref = fl(m * c_hi), -inf for a run of -inf logits (weight 0)
  if (lane_id() == 0) *slot = tag_run(m == -INFINITY ? -INFINITY : -neg_m, s);
}

// Weight of a record relative to the reference M, for fp64 accumulation (0
// for a missing or empty run, NaN for a NaN sum). The factor 2^(ref - M) is
// formed in fp32: the record's sum is an fp32 value, and an error of about
// one ulp in a run's weight moves every CDF boundary by far less than the
// fp32 rounding of the sums themselves.
__device__ __forceinline__ double run_weight(uint64_t v, float M) {
  const float ref = run_ref(v);
  const float s = run_sum(v);
  if (v == 0ull || ref == -INFINITY || !(s > 0.0f)) return (s != s) ? static_cast<double>(s) : 0.0;
  return static_cast<double>(s) * static_cast<double>(fast_exp2(ref - M));
}

constexpr int kRegRounds = 4;  // rounds of 64 records kept in registers by the draw

}  // namespace

// Pass 1: workgroup ch of row r streams the runs [ch * nrun / cps,
// (ch + 1) * nrun / cps) of the row (the chunks of a row differ by at most
// one run); wave w takes every fourth of them, starting at the w-th.
template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void sample_stream_kernel(
    SampleParams P) {
  const uint32_t cps = static_cast<uint32_t>(P.cps);
  const uint32_t r = blockIdx.x / cps;
  const int64_t ch = static_cast<int64_t>(blockIdx.x - r * cps);
  const int32_t c0 = static_cast<int32_t>(div_nonneg(ch * P.nrun, cps));
  const int32_t g_end = static_cast<int32_t>(div_nonneg((ch + 1) * P.nrun, cps));
  const int32_t g0 = c0 + wave_id();
  if (g0 >= g_end) return;  // no barrier follows: an idle wave may leave
  const int32_t n = (g_end - g0 + kWaves - 1) / kWaves;  // runs of this wave, >= 1
  const uint4* row = sample_row(P, r, T::kBytes);
  uint64_t* rec = P.rec + static_cast<int64_t>(r) * P.nrun;
  uint4 a[kRunLaneVecs], b[kRunLaneVecs];
  load_run<T>(row, g0, P.nvec, a);
  const Scale c = exponent_scale(temperature_of(P.temperature, static_cast<int>(r)));
  // invariant: `a` holds this wave's run i - 1
  int32_t i = 1;
#pragma unroll 1
  for (; i + 1 < n; i += 2) {
    load_run<T>(row, g0 + i * kWaves, P.nvec, b);
    finish_run<T>(a, c, rec + g0 + (i - 1) * kWaves);
    load_run<T>(row, g0 + (i + 1) * kWaves, P.nvec, a);
    finish_run<T>(b, c, rec + g0 + i * kWaves);
  }
  if (i < n) {
    load_run<T>(row, g0 + i * kWaves, P.nvec, b);
    finish_run<T>(a, c, rec + g0 + (i - 1) * kWaves);
    finish_run<T>(b, c, rec + g0 + i * kWaves);
  } else {
    finish_run<T>(a, c, rec + g0 + (i - 1) * kWaves);
  }
}

// Pass 2: one wave per row.
template <class T>
__global__ __launch_bounds__(kWave) void sample_draw_kernel(SampleParams P) {
  const int r = static_cast<int>(blockIdx.x);
  const int lane = lane_id();
  const int nr = P.nrun;
  const int rounds = (nr + kWave - 1) / kWave;
  uint64_t* rec = P.rec + static_cast<int64_t>(r) * P.nrun;
  uint32_t err = 0u;
  const float Tv = temperature_of(P.temperature, r);
  const double u = static_cast<double>(P.uniforms[r]);
  if (!(Tv > 0.0f) || !isfinite(Tv)) err |= SV_ERRF_TEMPERATURE;

  // Rows of up to kRegRounds * 64 runs (every realistic vocabulary) keep all
  // their records, weights and scans in registers; longer rows re-read their
  // records in each pass.
  const bool in_regs = rounds <= kRegRounds;
  uint64_t v[kRegRounds];
#pragma unroll
  for (int k = 0; k < kRegRounds; ++k) {
    const int g = k * kWave + lane;
    v[k] = (g < nr && (in_regs || k == 0)) ? load_ready(&rec[g], &err) : 0ull;
  }
  auto record = [&](int rd) -> uint64_t {
    const int g = rd * kWave + lane;
    return g < nr ? load_ready(&rec[g], &err) : 0ull;
  };

  // (1) the largest reference
  float M = -INFINITY;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kRegRounds; ++k)
      if (v[k] != 0ull) M = fmaxf(M, run_ref(v[k]));
  } else {
    for (int rd = 0; rd < rounds; ++rd) {
      const uint64_t x = record(rd);
      if (x != 0ull) M = fmaxf(M, run_ref(x));
    }
  }
  M = wave_max_dpp(M);

  // (2) the weights' inclusive scan in run order, and the total
  double w_k[kRegRounds], inc_k[kRegRounds], base_k[kRegRounds];
  double carry = 0.0;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kRegRounds; ++k) {
      w_k[k] = run_weight(v[k], M);
      inc_k[k] = wave_inclusive_scan(w_k[k]);
      base_k[k] = carry;
      if (k < rounds) carry += __shfl(inc_k[k], kWave - 1, kWave);
    }
  } else {
    for (int rd = 0; rd < rounds; ++rd) carry += __shfl(wave_inclusive_scan(run_weight(record(rd), M)), kWave - 1, kWave);
  }
  const double Z = carry;
  const double target = u * Z;

  // (3) the first run whose inclusive weight exceeds the target, and the last
  //     run with weight (rounding at the top end)
  int found = -1, last_pos = -1;
  double prefix = 0.0;
  float ref_found = 0.0f, ref_last = 0.0f;
  auto search = [&](int rd, uint64_t x, double w, double inc, double base) {
    const uint64_t pos = __ballot(w > 0.0);
    if (pos != 0ull) {
      const int l = 63 - __clzll(static_cast<long long>(pos));
      last_pos = rd * kWave + l;
      ref_last = __shfl(run_ref(x), l, kWave);
    }
    const uint64_t hit = __ballot(w > 0.0 && base + inc > target);
    if (hit != 0ull && found < 0) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      double excl = __shfl_up(inc, 1, kWave);
      if (lane == 0) excl = 0.0;
      found = rd * kWave + l;
      prefix = base + __shfl(excl, l, kWave);
      ref_found = __shfl(run_ref(x), l, kWave);
    }
  };
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kRegRounds; ++k)
      if (k < rounds && found < 0) search(k, v[k], w_k[k], inc_k[k], base_k[k]);
  } else {
    carry = 0.0;
    for (int rd = 0; rd < rounds && found < 0; ++rd) {
      const uint64_t x = record(rd);
      const double w = run_weight(x, M);
      const double inc = wave_inclusive_scan(w);
      search(rd, x, w, inc, carry);
      carry += __shfl(inc, kWave - 1, kWave);
    }
  }
  if (!(Z > 0.0) || !isfinite(Z) || !isfinite(M)) err |= SV_ERRF_NONFINITE;
  const bool bad = err != 0u;

  int token = -1;
  float prob = NAN;
  if (!bad && (found >= 0 || last_pos >= 0)) {
    const int g = found >= 0 ? found : last_pos;
    const float ref = found >= 0 ? ref_found : ref_last;
    // remainder of the target in the run's own units (its weights are 2^(x c - ref))
    // (divided by the same fp32 factor that scaled the run's weight)
    const double tk = found >= 0 ? (target - prefix) / static_cast<double>(fast_exp2(ref - M)) : INFINITY;
    const Scale c = exponent_scale(Tv);
    const uint4* row = sample_row(P, r, T::kBytes);
    constexpr int NE = kRunLaneVecs * T::kVec;
    // lane l holds the run's vectors 4l .. 4l + 3 (its tokens in ascending order)
    const int64_t vbase = static_cast<int64_t>(g) * kRunVecs + kRunLaneVecs * lane;
    uint4 q[kRunLaneVecs];
#pragma unroll
    for (int k = 0; k < kRunLaneVecs; ++k) q[k] = (vbase + k < P.nvec) ? row[vbase + k] : neg_inf_vec<T>();
    float x[NE], w[NE];
#pragma unroll
    for (int k = 0; k < kRunLaneVecs; ++k) unpack<T>(q[k], &x[k * T::kVec]);
    const float neg_m = -ref;
    float lane_tot = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      w[e] = fast_exp2(scaled_arg(x[e], c, neg_m));
      lane_tot += w[e];
    }
    const double inc = wave_inclusive_scan(static_cast<double>(lane_tot));
    double excl = __shfl_up(inc, 1, kWave);
    if (lane == 0) excl = 0.0;
    int first = -1, last = -1;
    float x_first = 0.0f, x_last = 0.0f, run = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      run += w[e];
      if (w[e] > 0.0f) {
        if (first < 0 && excl + static_cast<double>(run) > tk) {
          first = e;
          x_first = x[e];
        }
        last = e;
        x_last = x[e];
      }
    }
    const uint64_t hit = __ballot(first >= 0);
    const uint64_t any = __ballot(last >= 0);
    int sel_lane, sel_e;
    float xs;
    if (hit != 0ull) {
      sel_lane = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      sel_e = __shfl(first, sel_lane, kWave);
      xs = __shfl(x_first, sel_lane, kWave);
    } else if (any != 0ull) {
      sel_lane = 63 - __clzll(static_cast<long long>(any));
      sel_e = __shfl(last, sel_lane, kWave);
      xs = __shfl(x_last, sel_lane, kWave);
    } else {
      sel_lane = -1;
      sel_e = 0;
      xs = 0.0f;
    }
    if (sel_lane >= 0) {
      token = static_cast<int>((static_cast<int64_t>(g) * kRunVecs + kRunLaneVecs * sel_lane) * T::kVec + sel_e);
      // q of the drawn token in fp64: 2^(x c - L), L = M + log2 Z
      const double c64 = static_cast<double>(c.hi) + static_cast<double>(c.lo);
      prob = static_cast<float>(exp2(static_cast<double>(xs) * c64 - (static_cast<double>(M) + log2(Z))));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) err |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(err), o, kWave));
  if (lane == 0) {
    P.out_tokens[r] = (err != 0u) ? -1 : token;
    if (P.out_prob != nullptr) P.out_prob[r] = (err != 0u) ? NAN : prob;
    raise_error(P.err_flags, err);
  }
  // every record of the row has been read: leave them zero
  for (int g = lane; g < nr; g += kWave) rec[g] = 0ull;
}

template <class T>
static hipError_t launch_sample_stream_t(const SampleParams& p, const PassEvents& ev, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(p.R) * p.cps;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  // Armed events take the streaming kernel's own start and end timestamps.
  launch_stream_pass(sample_stream_kernel<T>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), stream, ev, p);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_sample_t(const SampleParams& p, const PassEvents& ev, hipStream_t stream) {
  const hipError_t e = launch_sample_stream_t<T>(p, ev, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_draw_kernel<T>, dim3(static_cast<uint32_t>(p.R)), dim3(kWave), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_sample(const SampleParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream) {
  return dtype == SV_DTYPE_BF16 ? launch_sample_t<BF16>(p, ev, stream) : launch_sample_t<F32>(p, ev, stream);
}

}  // namespace sv
