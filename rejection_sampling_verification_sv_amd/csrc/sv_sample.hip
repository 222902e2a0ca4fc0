// Draft-side sampling in one launch over the logits (rows on 16-byte
// boundaries): the drafter's step x ~ q(x), q = softmax(logits / T), by the
// inverse CDF over ascending token id with one caller-supplied uniform per
// row ([In Production] "Speculative Decoding in Production", section 2: the
// draft model samples each candidate; [Draft-and-Verify] "Speculative
// Decoding for LLM Inference", "The draft-and-verify loop").
//
// Pass 1 — sample_stream_kernel. Each row is cut into units of kUnitVecs
// 16-byte vectors; the call's units are split into ngroups contiguous
// ranges, and the waves of a group's blocks take its units in order from
// the group's counter (the next ticket requested while the current unit
// streams). A group's blocks come from every round in which the hardware
// hands blocks out: the waves of late blocks, which get less of the memory
// bandwidth while early blocks run, take fewer units instead of finishing
// last. A wave streams its unit with coalesced non-temporal 16-byte loads,
// two batches of two vectors per lane in flight (across units too), each
// lane keeping a running maximum and the sum of 2^(x c - reference)
// (c = log2(e) / T); at the end of each segment of kSegVecs vectors the
// wave combines its lanes and stores the segment's record: reference
// M_g = the largest fl(max * c_hi) of its lanes, S_g = sum over the segment
// of 2^(x c - M_g). No wave waits for another; each wave makes exactly one
// take that finds its group's units gone, and the last such take returns
// the group's counter to zero.
//
// Pass 2 — sample_draw_kernel, one wave per row: it reads the row's
// records, forms M = max M_g, the weights S_g 2^(M_g - M) and their
// inclusive scan in fp64 in token order, and finds the segment whose
// inclusive weight first exceeds u Z (Z = the total; rounding at the top
// end: the last segment with weight). It re-reads that one segment,
// recomputes its weights with the stream's fp32 operations, scans the
// lanes' totals in fp64 and picks the first token whose cumulative weight
// exceeds the remainder (rounding: the last token with weight). It returns
// the row's records to zero.
#include <hip/hip_ext.h>
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_stream.h"

namespace sv {

namespace {

__device__ __forceinline__ const uint4* sample_row(const SampleParams& P, int64_t r) {
  return reinterpret_cast<const uint4*>(static_cast<const char*>(P.logits) + r * P.nvec * 16);
}

// The wave's combine of its lanes' running states into a segment record:
// M = the largest fl(max * c_hi) (-inf for an empty or all -inf segment),
// S = the sum of each lane's sum rescaled to M (fp32 over the wave: a
// segment holds kSegVecs vectors). Lane 0 stores it.
__device__ __forceinline__ void publish_segment(const Running& st, Scale c, uint64_t* rm, uint64_t* rs) {
  const float mc = (st.mx == -INFINITY) ? -INFINITY : st.mx * c.hi;
  const float M = wave_max_dpp(mc);
  const float S = wave_sum_dpp((mc == -INFINITY) ? 0.0f : st.s * fast_exp2(mc - M));
  if (lane_id() == 0) {
    *rm = tag_float(M);
    *rs = tag_nonneg_double(static_cast<double>(S));
  }
}

// Weight of a record relative to the row's reference M, for fp64
// accumulation (0 for an empty segment, NaN for a NaN sum). The factor
// 2^(M_g - M) is formed in fp32, like the segment's own weights.
__device__ __forceinline__ double seg_weight(uint64_t m, uint64_t s, float M) {
  const float ref = untag_float(m);
  const double S = untag_nonneg_double(s);
  if (ref == -INFINITY || !(S > 0.0)) return (S != S) ? S : 0.0;
  return S * static_cast<double>(fast_exp2(ref - M));
}

constexpr int kRegRounds = 2;  // rounds of 64 records the draw keeps in registers

// OR of the error bits over the wave.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave));
  return v;
}


// Pass 2 for row r (one wave). The records were stored by the previous
// launch on the same stream: plain loads; a record still zero was never
// written (SV_ERRF_INTERNAL). Rows of up to kRegRounds * 64 records keep
// them in registers; longer rows read them again in each pass.
template <class T>
__device__ __forceinline__ void draw_row(const SampleParams& P, int r) {
  const int lane = lane_id();
  const int nr = P.nrec;
  const int rounds = (nr + kWave - 1) / kWave;
  const int64_t base = static_cast<int64_t>(r) * nr;
  uint32_t err = 0u;
  const float Tv = temperature_of(P.temperature, r);
  const double u = static_cast<double>(P.uniforms[r]);
  if (!(Tv > 0.0f) || !isfinite(Tv)) err |= SV_ERRF_TEMPERATURE;
  const Scale c = exponent_scale(Tv);  // while the records are on their way
  const bool in_regs = rounds <= kRegRounds;
  auto fetch = [&](int rd, uint64_t& m, uint64_t& s) {
    const int g = rd * kWave + lane;
    m = (g < nr) ? load_ready(&P.rec_m[base + g], &err) : 0ull;
    s = (g < nr) ? load_ready(&P.rec_s[base + g], &err) : 0ull;
  };
  uint64_t vm[kRegRounds], vs[kRegRounds];
#pragma unroll
  for (int k = 0; k < kRegRounds; ++k) {
    vm[k] = vs[k] = 0ull;
    if (in_regs && k < rounds) fetch(k, vm[k], vs[k]);
  }

  // (1) the largest reference
  float M = -INFINITY;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kRegRounds; ++k)
      if (vm[k] != 0ull) M = fmaxf(M, untag_float(vm[k]));
  } else {
    for (int rd = 0; rd < rounds; ++rd) {
      uint64_t m, s;
      fetch(rd, m, s);
      if (m != 0ull) M = fmaxf(M, untag_float(m));
    }
  }
  M = wave_max_dpp(M);

  // (2) the weights' inclusive scan in token order, and the total
  double w_k[kRegRounds], inc_k[kRegRounds], base_k[kRegRounds];
  double carry = 0.0;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kRegRounds; ++k) {
      w_k[k] = inc_k[k] = 0.0;
      base_k[k] = carry;
      if (k < rounds) {
        w_k[k] = (vm[k] != 0ull) ? seg_weight(vm[k], vs[k], M) : 0.0;
        inc_k[k] = wave_scan_dpp(w_k[k]);
        carry += readlane_f64(inc_k[k], kWave - 1);
      }
    }
  } else {
    for (int rd = 0; rd < rounds; ++rd) {
      uint64_t m, s;
      fetch(rd, m, s);
      carry += readlane_f64(wave_scan_dpp(m != 0ull ? seg_weight(m, s, M) : 0.0), kWave - 1);
    }
  }
  const double Z = carry;
  const double target = u * Z;

  // (3) the first segment whose inclusive weight exceeds the target, and
  //     the last segment with weight (rounding at the top end)
  int found = -1, last_pos = -1;
  double prefix = 0.0;
  float ref_found = 0.0f, ref_last = 0.0f;
  auto search = [&](int rd, uint64_t m, double w, double inc, double b0) {
    const uint64_t pos = __ballot(w > 0.0);
    if (pos != 0ull) {
      const int l = 63 - __clzll(static_cast<long long>(pos));
      last_pos = rd * kWave + l;
      ref_last = readlane_f32(untag_float(m), l);
    }
    const uint64_t hit = __ballot(w > 0.0 && b0 + inc > target);
    if (hit != 0ull && found < 0) {
      const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      found = rd * kWave + l;
      prefix = b0 + readlane_f64(wave_exclusive_from(inc), l);
      ref_found = readlane_f32(untag_float(m), l);
    }
  };
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kRegRounds; ++k)
      if (k < rounds && found < 0) search(k, vm[k], w_k[k], inc_k[k], base_k[k]);
  } else {
    carry = 0.0;
    for (int rd = 0; rd < rounds && found < 0; ++rd) {
      uint64_t m, s;
      fetch(rd, m, s);
      const double w = (m != 0ull) ? seg_weight(m, s, M) : 0.0;
      const double inc = wave_scan_dpp(w);
      search(rd, m, w, inc, carry);
      carry += readlane_f64(inc, kWave - 1);
    }
  }
  if (!(Z > 0.0) || !isfinite(Z) || !isfinite(M)) err |= SV_ERRF_NONFINITE;
  err = wave_or(err);

  int token = -1;
  float prob = NAN;
  const int g = (err != 0u) ? -1 : (found >= 0 ? found : last_pos);
  if (g >= 0) {
    const float ref = found >= 0 ? ref_found : ref_last;
    // the remainder in the segment's own units (its weights are
    // 2^(x c - M_g)), divided by the same fp32 factor that scaled its weight
    const float factor = fast_exp2(ref - M);
    const double tk = found >= 0 ? (target - prefix) / static_cast<double>(factor) : INFINITY;
    // segment g covers the row's vectors [g kSegVecs, (g + 1) kSegVecs);
    // lane l holds its vectors kSegLaneVecs l .. + kSegLaneVecs - 1 (tokens
    // ascending)
    const int64_t v0 = static_cast<int64_t>(g) * kSegVecs;
    const int64_t v1 = min(P.nvec, v0 + kSegVecs);
    const uint4* row = sample_row(P, r);
    const int64_t vl = v0 + static_cast<int64_t>(lane) * kSegLaneVecs;
    uint4 q[kSegLaneVecs];
#pragma unroll
    for (int k = 0; k < kSegLaneVecs; ++k) q[k] = (vl + k < v1) ? row[vl + k] : neg_inf_vec<T>();
    const float neg_m = -ref;
    // the lane's weights, formed twice from the raw vectors (the same
    // operations give the same values) rather than held across the scan
    float tot = 0.0f;
#pragma unroll
    for (int k = 0; k < kSegLaneVecs; ++k) {
      float x[T::kVec];
      unpack<T>(q[k], x);
#pragma unroll
      for (int e = 0; e < T::kVec; ++e) tot += fast_exp2(scaled_arg(x[e], c, neg_m));
    }
    const double excl = wave_exclusive_from(wave_scan_dpp(static_cast<double>(tot)));
    int first = -1, last = -1;
    float w_first = 0.0f, w_last = 0.0f, run = 0.0f;
#pragma unroll
    for (int k = 0; k < kSegLaneVecs; ++k) {
      uint4 raw = q[k];
      asm volatile("" : "+v"(raw.x), "+v"(raw.y), "+v"(raw.z), "+v"(raw.w));
      float x[T::kVec];
      unpack<T>(raw, x);
#pragma unroll
      for (int e = 0; e < T::kVec; ++e) {
        const float wv = fast_exp2(scaled_arg(x[e], c, neg_m));
        run += wv;
        if (wv > 0.0f) {
          if (first < 0 && excl + static_cast<double>(run) > tk) {
            first = k * T::kVec + e;
            w_first = wv;
          }
          last = k * T::kVec + e;
          w_last = wv;
        }
      }
    }
    const uint64_t hit = __ballot(first >= 0);
    const uint64_t any = __ballot(last >= 0);
    int sel_lane = -1, sel_e = 0;
    float ws = 0.0f;
    if (hit != 0ull) {
      sel_lane = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      sel_e = __builtin_amdgcn_readlane(first, sel_lane);
      ws = readlane_f32(w_first, sel_lane);
    } else if (any != 0ull) {
      sel_lane = 63 - __clzll(static_cast<long long>(any));
      sel_e = __builtin_amdgcn_readlane(last, sel_lane);
      ws = readlane_f32(w_last, sel_lane);
    }
    if (sel_lane >= 0) {
      token = static_cast<int>((v0 + static_cast<int64_t>(sel_lane) * kSegLaneVecs) * T::kVec + sel_e);
      // q of the drawn token: its weight 2^(x c - M_g) times 2^(M_g - M), over Z
      prob = static_cast<float>(static_cast<double>(ws) * static_cast<double>(factor) / Z);
    }
  }
  if (lane == 0) {
    P.out_tokens[r] = (err != 0u) ? -1 : token;
    if (P.out_prob != nullptr) P.out_prob[r] = (err != 0u) ? NAN : prob;
    raise_error(P.err_flags, err);
  }
  // every record of the row has been read: leave them zero
  for (int k = lane; k < nr; k += kWave) {
    P.rec_m[base + k] = 0ull;
    P.rec_s[base + k] = 0ull;
  }
}

}  // namespace

// A unit of the call: row r, unit j of the row, its vectors
// [j kUnitVecs, min(nvec, (j + 1) kUnitVecs)).
struct Unit {
  int32_t r;
  int32_t j;
  int32_t n;      // vectors
  int32_t nb;     // batches (the last may be ragged)
  int32_t nfull;  // full batches
};

// One wave's share of its group's units (the group's units are u0 .. u0 +
// nk - 1): wave i of the group's waves_k waves starts with unit i, and the
// group's counter `take` hands out units waves_k, waves_k + 1, ... in
// order. Two batches of kStreamU vectors per lane are in flight at any
// time, also across units; the next ticket is requested when the current
// unit starts.
template <class T>
__device__ __forceinline__ void stream_units(const SampleParams& P, uint32_t* take, int64_t u0, uint32_t nk,
                                             uint32_t waves_k, uint32_t i) {
  constexpr int U = kStreamU;
  constexpr int STEP = kWave * U;        // vectors per batch
  constexpr int BPS = kSegVecs / STEP;   // batches per segment
  const int lane = lane_id();
  // lane 0's fetch-add (waited for where the value is used), as a unit index
  auto grab = [&]() -> uint32_t {
    uint32_t t = 0u;
    if (lane == 0) t = __hip_atomic_fetch_add(take, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + waves_k;
    return t;
  };
  // The wave's one take that found the units gone: the group's last such
  // take returns the counter to zero (nobody takes from it afterwards). The
  // counter sees max(nk - waves_k, 0) takes that found a unit and waves_k
  // that did not.
  const uint32_t last_take = (nk > waves_k ? nk : waves_k) + waves_k - 1u;
  auto closing_take = [&](uint32_t t) {
    if (t == last_take && lane == 0) __hip_atomic_store(take, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // (wave-uniform values, kept in scalar registers: the division runs on
  // the vector unit)
  auto unit_of = [&](uint32_t t) {
    const int64_t u = u0 + t;
    Unit x;
    x.r = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(div_nonneg(u, P.upr)));
    x.j = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(u - static_cast<int64_t>(x.r) * P.upr));
    const int64_t v0 = static_cast<int64_t>(x.j) * kUnitVecs;
    x.n = static_cast<int32_t>(min(static_cast<int64_t>(kUnitVecs), P.nvec - v0));
    x.nb = (x.n + STEP - 1) / STEP;
    x.nfull = x.n / STEP;
    return x;
  };
  auto load = [&](const Unit& x, int32_t i, uint4 (&raw)[U]) {
    const uint4* src = sample_row(P, x.r) + static_cast<int64_t>(x.j) * kUnitVecs;
    if (i < x.nfull) {
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = stream_load(src + i * STEP + u * kWave + lane);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = i * STEP + u * kWave + lane;
        raw[u] = (k < x.n) ? stream_load(src + k) : neg_inf_vec<T>();
      }
    }
    // keep the loads ahead of the reduction that follows them
    __builtin_amdgcn_sched_barrier(0);
  };

  if (i >= nk) {  // no unit of its own: the wave's one (failing) take
    closing_take(__builtin_amdgcn_readfirstlane(grab()));
    return;
  }
  const uint32_t t = i;
  uint32_t pend = grab();  // the next ticket, in flight
  Unit cur = unit_of(t), nxt = cur;
  uint4 a[U], b[U];
  load(cur, 0, a);
  int32_t c_row = cur.r;
  Scale c = exponent_scale(temperature_of(P.temperature, cur.r));
  Running st{-INFINITY, 0.0f, 0.0f};
  int32_t bi = 0;    // batch of `cur` held in the buffer being reduced
  bool more = true;  // a batch follows the one being reduced

  // reduce the batch in `x` (batch bi of cur) while the next one (if any)
  // goes into `y`
  auto step = [&](uint4 (&x)[U], uint4 (&y)[U]) {
    const bool last_batch = bi + 1 == cur.nb;
    bool next_unit = false;
    if (!last_batch) {
      load(cur, bi + 1, y);
    } else {
      const uint32_t tn = __builtin_amdgcn_readfirstlane(pend);
      if (tn < nk) {
        nxt = unit_of(tn);
        load(nxt, 0, y);
        pend = grab();
        next_unit = true;
      } else {
        closing_take(tn);
        more = false;
      }
    }
    add_batch<T, U, false>(st, x, c);
    if ((bi + 1) % BPS == 0 || last_batch) {
      const int64_t rec = static_cast<int64_t>(cur.r) * P.nrec + static_cast<int64_t>(cur.j) * kSegsPerUnit + bi / BPS;
      publish_segment(st, c, P.rec_m + rec, P.rec_s + rec);
      st = Running{-INFINITY, 0.0f, 0.0f};
    }
    if (!last_batch) {
      ++bi;
      return;
    }
    // the unit is done: empty records for its segments past the row's end
    if (lane == 0)
      for (int s = bi / BPS + 1; s < kSegsPerUnit; ++s) {
        const int64_t rec = static_cast<int64_t>(cur.r) * P.nrec + static_cast<int64_t>(cur.j) * kSegsPerUnit + s;
        P.rec_m[rec] = tag_float(-INFINITY);
        P.rec_s[rec] = tag_nonneg_double(0.0);
      }
    if (next_unit) {
      cur = nxt;
      bi = 0;
      if (cur.r != c_row) {
        c_row = cur.r;
        c = exponent_scale(temperature_of(P.temperature, cur.r));
      }
    }
  };
#pragma unroll 1
  while (more) {
    step(a, b);
    if (!more) break;
    step(b, a);
  }
}

// Pass 1: block b streams for group b % ngroups; every wave takes units of
// the group's range on its own (no barrier, no wave waits for another).
template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void sample_stream_kernel(
    SampleParams P) {
  const uint32_t G = static_cast<uint32_t>(P.ngroups);
  const uint32_t k = blockIdx.x % G;
  const int64_t total = static_cast<int64_t>(P.R) * P.upr;
  const int64_t u0 = div_nonneg(static_cast<int64_t>(k) * total, G);
  const int64_t u1 = div_nonneg(static_cast<int64_t>(k + 1) * total, G);
  // this wave's place among the group's waves: blocks k, k + G, ... in order
  const uint32_t i = (blockIdx.x / G) * kWaves + static_cast<uint32_t>(wave_id());
  stream_units<T>(P, P.take + static_cast<int64_t>(k) * kCtrStride, u0, static_cast<uint32_t>(u1 - u0),
                  static_cast<uint32_t>(P.wpg) * kWaves, i);
}

// Pass 2: one wave per row.
template <class T>
__global__ __launch_bounds__(kWave) void sample_draw_kernel(SampleParams P) {
  draw_row<T>(P, static_cast<int>(blockIdx.x));
}

template <class T>
static hipError_t launch_sample_t(const SampleParams& p, const PassEvents& ev, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(p.ngroups) * p.wpg;
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  // Armed events take the streaming kernel's own start and end timestamps.
  launch_stream_pass(sample_stream_kernel<T>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), stream, ev, p);
  hipLaunchKernelGGL(sample_draw_kernel<T>, dim3(static_cast<uint32_t>(p.R)), dim3(kWave), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_sample(const SampleParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream) {
  return dtype == SV_DTYPE_BF16 ? launch_sample_t<BF16>(p, ev, stream) : launch_sample_t<F32>(p, ev, stream);
}

}  // namespace sv
