// The one-pass statistics stream shared by the chain kernels and the
// sampling-tree kernels: each thread keeps the running maximum of its logits
// and the sum of 2^(x c - reference) over them (online rescaling per batch of
// 16-byte vectors), and a workgroup combines its threads in fp64 into one
// (reference, sum) pair per piece of a row.
#pragma once

#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

// Running (max, sum) of one thread. `mx` is the largest raw logit seen and
// `s` = sum of 2^a over the logits seen, a = x*c - fl(mx*c_hi). With the
// entropy requested (kEnt) it also keeps `a` = sum of 2^a * a (<= 0 up to
// rounding): for p = 2^a / s, the entropy is ln 2 * (log2 s - A / s). When the
// reference rises by d, every a falls by d: s -> 2^-d s, A -> 2^-d (A - d s).
// Arguments are clamped at -256 before the product (2^a is already 0 there),
// so -inf logits add 0, not 0 * -inf.
struct Running {
  float mx;
  float s;
  float a;
};

constexpr float kArgFloor = -256.0f;

template <int N, bool kEnt = false>
__device__ __forceinline__ void running_add(Running& st, const float (&x)[N], Scale c) {
  float bm = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
  // Rescale the running sum to the new maximum (branch-free: a factor of 1
  // when the maximum did not move, 0 while nothing finite had been seen).
  const float m_new = fmaxf(st.mx, bm);
  const float scale = (st.mx == -INFINITY) ? 0.0f : fast_exp2(st.mx * c.hi - m_new * c.hi);
  if constexpr (kEnt) st.a = (st.mx == -INFINITY) ? 0.0f : scale * (st.a - (m_new * c.hi - st.mx * c.hi) * st.s);
  st.mx = m_new;
  const float neg_m = neg_reference(m_new, c);
  // four partial sums, pairwise inside each group of 8
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float acca[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < N; g += 8) {
    float e[8], ea[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float arg = (g + i < N) ? scaled_arg(x[g + i], c, neg_m) : -INFINITY;
      e[i] = (g + i < N) ? fast_exp2(arg) : 0.0f;
      if constexpr (kEnt) ea[i] = e[i] * fmaxf(arg, kArgFloor);
    }
    acc[(g / 8) & 3] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    if constexpr (kEnt) acca[(g / 8) & 3] += ((ea[0] + ea[1]) + (ea[2] + ea[3])) + ((ea[4] + ea[5]) + (ea[6] + ea[7]));
  }
  st.s = st.s * scale + ((acc[0] + acc[1]) + (acc[2] + acc[3]));
  if constexpr (kEnt) st.a += (acca[0] + acca[1]) + (acca[2] + acca[3]);
}

template <bool kEnt = false>
__device__ __forceinline__ void running_add1(Running& st, float x, Scale c) {
  if (x > st.mx) {
    if constexpr (kEnt)
      st.a = (st.mx == -INFINITY) ? 0.0f
                                  : fast_exp2(st.mx * c.hi - x * c.hi) * (st.a - (x * c.hi - st.mx * c.hi) * st.s);
    st.s = (st.mx == -INFINITY) ? 0.0f : st.s * fast_exp2(st.mx * c.hi - x * c.hi);
    st.mx = x;
  }
  const float arg = scaled_arg(x, c, neg_reference(st.mx, c));
  const float e = fast_exp2(arg);
  st.s += e;
  if constexpr (kEnt) st.a += e * fmaxf(arg, kArgFloor);
}

__device__ __forceinline__ void split(double v, float& hi, float& lo) {
  hi = static_cast<float>(v);
  lo = static_cast<float>(v - static_cast<double>(hi));
}

// Block-wide combine of the threads' running states into (reference, sum):
// the largest fl(mx*c_hi), and the fp64 sum of each thread's sum rescaled to it
// (with kEnt also the fp64 sum of each thread's A rescaled to it, into *A).
template <int NW = kWaves, bool kEnt = false>
__device__ __forceinline__ void block_combine(const Running& st, Scale c, float* s_redf, double* s_redd, float* MC,
                                              double* S, double* A = nullptr) {
  const float mc = (st.mx == -INFINITY) ? -INFINITY : st.mx * c.hi;
  *MC = block_max<NW>(mc, s_redf);
  double sd = 0.0, ad = 0.0;
  if (mc != -INFINITY) {
    const float f = fast_exp2(mc - *MC);
    sd = static_cast<double>(st.s * f);
    if constexpr (kEnt)
      ad = static_cast<double>(f) * (static_cast<double>(st.a) -
                                     (static_cast<double>(*MC) - static_cast<double>(mc)) * static_cast<double>(st.s));
  }
  *S = block_sum<NW>(sd, s_redd);
  if constexpr (kEnt) *A = block_sum<NW>(ad, s_redd);
}

template <class T, int U = kStatsUnroll, bool kEnt = false>
__device__ __forceinline__ void add_batch(Running& st, const uint4 (&raw)[U], Scale c) {
  if constexpr (kEnt && T::kVec == 8) {
    // bf16 with the entropy: the same operations in the same order as
    // running_add (one group of 8 per vector), so the same (reference, sum);
    // A as one fma chain
    float t[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack<T>(raw[u], t[u]);
    float bm = -INFINITY, bl = INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bm = fmaxf(bm, t[u][i]);
        bl = fminf(bl, t[u][i]);
      }
    const float m_new = fmaxf(st.mx, bm);
    const float scale = (st.mx == -INFINITY) ? 0.0f : fast_exp2(st.mx * c.hi - m_new * c.hi);
    st.a = (st.mx == -INFINITY) ? 0.0f : scale * (st.a - (m_new * c.hi - st.mx * c.hi) * st.s);
    st.mx = m_new;
    const float neg_m = neg_reference(m_new, c);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float acca = st.a;
    // Arguments below kArgFloor have 2^a = 0, so the clamp changes nothing
    // but the product 0 * -inf of a masked logit: a batch without -inf
    // (the usual case) sums A unclamped
    if (bl != -INFINITY) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float arg = scaled_arg(t[u][i], c, neg_m);
          e[i] = fast_exp2(arg);
          acca = fmaf(e[i], arg, acca);
        }
        acc[u & 3] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float arg = scaled_arg(t[u][i], c, neg_m);
          e[i] = fast_exp2(arg);
          acca = fmaf(e[i], fmaxf(arg, kArgFloor), acca);
        }
        acc[u & 3] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      }
    }
    st.s = st.s * scale + ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    // A is made here, batch by batch: otherwise the compiler sinks the fma
    // chain into the next batch's rescale, which drops A when no finite
    // logit has been seen, and keeps this batch's 16 arguments and
    // exponentials live across the next batch's loads (82 VGPRs, not 57)
    asm volatile("" : "+v"(acca));
    st.a = acca;
  } else {
    float x[U * T::kVec];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack<T>(raw[u], &x[u * T::kVec]);
    running_add<U * T::kVec, kEnt>(st, x, c);
  }
}

// The exponent scale of a sequence, computed on first use: the statistics
// pass issues its first loads before it waits for the temperature.
struct LazyScale {
  const float* temperature;
  int b;
  bool ready;
  Scale c;
  __device__ __forceinline__ const Scale& get() {
    if (!ready) {
      c = exponent_scale(temperature_of(temperature, b));
      ready = true;
    }
    return c;
  }
};

// One thread's share of the vectors [p0, p1) of a row: full batches of
// kStreamU vectors per thread without any masking, then one ragged batch
// whose missing vectors are replaced by -inf. Two batch buffers alternate, so
// one batch's loads are always in flight while the other is reduced, and the
// first loads go out before anything (the temperature) is waited for.
template <class T, int U, int TPB>
__device__ __forceinline__ void load_batch(const uint4* ptr, uint4 (&raw)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) raw[u] = stream_load(ptr + u * TPB);
  // keep the loads ahead of the reduction that follows them (the scheduler
  // would otherwise sink them below the wait for the other buffer)
  __builtin_amdgcn_sched_barrier(0);
}

template <class T, int TPB, bool kEnt = false, int U = kStreamU>
__device__ __forceinline__ void flat_piece_stats(const uint4* body, int64_t p0, int64_t p1, LazyScale& sc,
                                                 Running& st) {
  constexpr int STEP = TPB * U;
  const int32_t nfull = static_cast<int32_t>((p1 - p0) / STEP);
  const uint4* ptr = body + p0 + threadIdx.x;
  if (nfull > 0) {
    uint4 a[U], b[U];
    load_batch<T, U, TPB>(ptr, a);
    const Scale c = sc.get();
    // invariant: `a` holds batch i - 1, which starts at ptr
    int32_t i = 1;
#pragma unroll 1
    for (; i + 1 < nfull; i += 2) {
      load_batch<T, U, TPB>(ptr + STEP, b);
      add_batch<T, U, kEnt>(st, a, c);
      load_batch<T, U, TPB>(ptr + 2 * STEP, a);
      add_batch<T, U, kEnt>(st, b, c);
      ptr += 2 * STEP;
    }
    if (i < nfull) {  // one batch left to load
      load_batch<T, U, TPB>(ptr + STEP, b);
      add_batch<T, U, kEnt>(st, a, c);
      add_batch<T, U, kEnt>(st, b, c);
      ptr += 2 * STEP;
    } else {
      add_batch<T, U, kEnt>(st, a, c);
      ptr += STEP;
    }
  }
  const int64_t rest = (p1 - p0) - static_cast<int64_t>(nfull) * STEP;  // vectors in the ragged batch
  if (rest > 0) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = static_cast<int64_t>(u) * TPB + threadIdx.x;
      raw[u] = (k < rest) ? stream_load(ptr + u * TPB) : neg_inf_vec<T>();
    }
    add_batch<T, U, kEnt>(st, raw, sc.get());
  }
}

}  // namespace

}  // namespace sv
