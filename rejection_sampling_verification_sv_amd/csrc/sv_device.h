// Device-side building blocks shared by the specverify kernels (gfx950, wave64).
//
// - 16-byte vector loads of logits and their conversion to fp32 (bf16 is the
//   upper half of a binary32, so widening is a shift or a mask);
// - wave64 reductions through cross-lane shuffles and block (256-thread)
//   reductions / exclusive scans through LDS, in a fixed order so that the
//   same inputs always give bit-identical results;
// - the "last workgroup to arrive" hand-off: every workgroup of a sequence
//   publishes its partial result, bumps the sequence's counter, and the one
//   that brings the counter to its total finishes the sequence (atomic
//   slots, see below: no fences, so no L2 write-back per workgroup).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;             // threads per workgroup (4 wave64s)
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;

// Logit element types. kVec = elements per 16-byte load.
struct BF16 {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
};
struct F32 {
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

template <class T>
__device__ __forceinline__ float load_elem(const void* row, int64_t i);

template <>
__device__ __forceinline__ float load_elem<BF16>(const void* row, int64_t i) {
  return bf16_bits_to_float(static_cast<const uint16_t*>(row)[i]);
}
template <>
__device__ __forceinline__ float load_elem<F32>(const void* row, int64_t i) {
  return static_cast<const float*>(row)[i];
}

// Widen one 16-byte vector into T::kVec floats, in ascending element order.
template <class T>
__device__ __forceinline__ void unpack(const uint4& v, float* out);

template <>
__device__ __forceinline__ void unpack<BF16>(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<F32>(const uint4& v, float* out) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}

// 16 bytes of -inf logits (padding that never wins a maximum and weighs 0).
// A 16-byte load of logits that are read once: a non-temporal load, so the
// stream does not displace what the caches hold (measured faster than a
// plain load on every streaming pass here).
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

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

// v_exp_f32: 2^x (about 1 ulp; inputs below -126 give 0 or a denormal).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- temperature scale

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

// ---------------------------------------------------------------- fp64 results from fp32 transcendentals

// 2^(lo - hi) for two fp32 references lo <= hi, as an fp64 factor: v_exp_f32
// of the fp32 difference. A factor multiplies an fp32 partial sum, so its
// error of about one fp32 ulp is of the order of that sum's own rounding.
__device__ __forceinline__ double ref_factor(float lo, float hi) { return static_cast<double>(fast_exp2(lo - hi)); }

// 2^a for an fp64 argument: a power of two times v_exp_f32 of the fraction in
// [-1/2, 1/2] (relative error about one fp32 ulp; the software fp64 exp2 is
// several times longer on this path, which every sampling workgroup runs).
__device__ __forceinline__ double exp2_split(double a) {
  if (!(a > -1100.0)) return (a != a) ? a : 0.0;  // NaN stays NaN; far below the fp64 range: 0
  if (a > 1100.0) return INFINITY;
  const double n = rint(a);
  return ldexp(static_cast<double>(fast_exp2(static_cast<float>(a - n))), static_cast<int>(n));
}

// log2 z for a finite z > 0: the fp64 exponent plus v_log_f32 of the
// mantissa in [1/2, 1) (absolute error about 1e-7; a row's log-normaliser
// needs no more, its sums being fp32-rounded).
__device__ __forceinline__ double log2_fast(double z) {
  int e;
  const double m = frexp(z, &e);
  return static_cast<double>(e) + static_cast<double>(__builtin_amdgcn_logf(static_cast<float>(m)));
}

// ---------------------------------------------------------------- wave64 reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum over the wave in lane order (fp64).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double n = __shfl_up(v, o, kWave);
    if ((threadIdx.x & (kWave - 1)) >= o) v += n;
  }
  return v;
}

// Wave-uniform maximum / sum through DPP row permutes (xor 1, xor 2, half-row
// mirror, row mirror: every lane of a 16-lane row then holds the row's
// result) and the four rows' results read from lanes 0, 16, 32, 48, combined
// in a fixed order. Much shorter latency than the shuffle forms (each step of
// those is an LDS permute); the same inputs give bit-identical results.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_read(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_move<0xb1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_move<0x4e>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_move<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_move<0x140>(v));  // row_mirror
  return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xb1>(v);
  v += dpp_move<0x4e>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

// fp64 lane moves through DPP (both 32-bit halves with the same control;
// lanes the control leaves without a source read 0).
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), kCtrl, kRowMask, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), kCtrl, kRowMask, 0xf, true);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                          __builtin_amdgcn_readlane(__double2loint(v), lane));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Inclusive fp64 prefix sum over the wave in lane order: steps of 1, 2, 4
// and 8 lanes within each row of 16, then each row adds the totals of the
// rows before it (row_bcast 15 and 31). DPP moves instead of LDS permutes.
__device__ __forceinline__ double wave_scan_dpp(double v) {
  v += dpp_f64<0x111>(v);        // row_shr:1
  v += dpp_f64<0x112>(v);        // row_shr:2
  v += dpp_f64<0x114>(v);        // row_shr:4
  v += dpp_f64<0x118>(v);        // row_shr:8
  v += dpp_f64<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}
// The exclusive prefix from the inclusive one: the previous lane's value
// (wave_shr:1; lane 0 reads 0).
__device__ __forceinline__ double wave_exclusive_from(double inc) { return dpp_f64<0x138>(inc); }
// fp64 sum over the wave in a fixed order (the tree of wave_sum_dpp: xor 1,
// xor 2, half-row mirror, row mirror, then the four rows' sums from lanes 0,
// 16, 32 and 48); every lane gets the result.
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_f64<0xb1>(v);
  v += dpp_f64<0x4e>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---------------------------------------------------------------- block (256) reductions
// `scratch` must hold kWaves elements; every thread of the block must call.

// NW = waves in the block (kWaves for the usual 256 threads).
template <int NW = kWaves>
__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, scratch[w]);
  __syncthreads();
  return r;
}

template <int NW = kWaves>
__device__ __forceinline__ double block_sum(double v, double* scratch) {
  v = wave_sum(v);
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += scratch[w];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_max_int(int v, int* scratch) {
  v = wave_max_int(v);
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = max(r, scratch[w]);
  __syncthreads();
  return r;
}

// Exclusive prefix sum over the block in thread order (fp64). Returns the
// exclusive prefix of this thread; *total gets the block total, computed as
// (exclusive prefix of the last thread) + (its value) so that a caller can
// reproduce it exactly from the same inputs.
__device__ __forceinline__ double block_exclusive_scan(double v, double* scratch, double* total) {
  const int lane = lane_id();
  double inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  double excl_in_wave = __shfl_up(inc, 1, kWave);
  if (lane == 0) excl_in_wave = 0.0;
  if (lane == kWave - 1) scratch[wave_id()] = inc;
  __syncthreads();
  double wave_prefix = 0.0;
  for (int w = 0; w < wave_id(); ++w) wave_prefix += scratch[w];
  const double excl = wave_prefix + excl_in_wave;
  __syncthreads();
  // The last thread publishes the total in the same terms a caller uses:
  // its exclusive prefix plus its own value.
  if (threadIdx.x == kThreads - 1) scratch[0] = excl + v;
  __syncthreads();
  *total = scratch[0];
  __syncthreads();
  return excl;
}

// ---------------------------------------------------------------- last-arriver hand-off
//
// Blocks of one sequence publish partial results into 64-bit slots of the
// workspace and bump the sequence's counter; the block whose increment brings
// the counter to its total combines the slots. No cache write-back or
// invalidate is needed (an agent-scope fence costs an L2 write-back per block
// on this part): each slot is written by ONE agent-scope atomic store whose
// value is never all-zero bits, and the last block reads each slot with
// agent-scope atomic loads until it is non-zero. Every store it waits for
// has already been issued (or belongs to work held by a running block), so
// the wait ends; it is still bounded in wall time and reports
// SV_ERRF_INTERNAL if it ever expires. The reader sets slots back to zero
// after use.

constexpr uint64_t kWaitTicks = 10000000ull;  // 100 ms of the 100 MHz real-time counter
constexpr uint32_t kErrInternal = 0x10u;      // SV_ERRF_INTERNAL

__device__ __forceinline__ void publish(uint64_t* slot, uint64_t v) {
  __hip_atomic_store(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t peek(const uint64_t* slot) {
  return __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *slot is non-zero and return it. Bounded: after kWaitTicks of
// wall time, or as soon as *abort is set by another expired wait, give up,
// set *abort, flag kErrInternal and return 0 (so a failure drains the launch
// quickly instead of spinning).
// kSleep sets the pause between polls (s_sleep units of 64 cycles).
template <int kSleep = 2>
__device__ __forceinline__ uint64_t await_slot(uint64_t* slot, uint32_t* err, uint64_t* abort) {
  uint64_t v = peek(slot);
  if (v != 0ull) return v;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(kSleep);
    v = peek(slot);
    if (v != 0ull) return v;
    if (peek(abort) != 0ull) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      publish(abort, 1ull);
      break;
    }
  }
  *err |= kErrInternal;
  return 0ull;
}

// A slot written by an earlier launch on the same stream: the kernel boundary
// makes it visible, so a plain (cacheable) load suffices. A zero means it was
// never written, which is reported as kErrInternal.
__device__ __forceinline__ uint64_t load_ready(const uint64_t* slot, uint32_t* err) {
  const uint64_t v = *slot;
  if (v == 0ull) *err |= kErrInternal;
  return v;
}

__device__ __forceinline__ void clear_slot(uint64_t* slot) { publish(slot, 0ull); }

// Tagged encodings (a written slot is never zero).
__device__ __forceinline__ uint64_t tag_float(float f) {
  return (1ull << 32) | static_cast<uint64_t>(__float_as_uint(f));
}
__device__ __forceinline__ float untag_float(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v)); }
// a non-negative double with its sign bit set (so 0.0 is stored as -0.0)
__device__ __forceinline__ uint64_t tag_nonneg_double(double d) {
  return static_cast<uint64_t>(__double_as_longlong(d)) | (1ull << 63);
}
__device__ __forceinline__ double untag_nonneg_double(uint64_t v) {
  return __longlong_as_double(static_cast<long long>(v & ~(1ull << 63)));
}
// any double, stored as the complement of its bits: zero only for the
// all-ones pattern, a NaN that no arithmetic here produces (a NaN it makes
// or passes on from fp32 inputs has zero low mantissa bits)
__device__ __forceinline__ uint64_t tag_any_double(double d) {
  return ~static_cast<uint64_t>(__double_as_longlong(d));
}
__device__ __forceinline__ double untag_any_double(uint64_t v) { return __longlong_as_double(static_cast<long long>(~v)); }

// Every thread of the block calls this after thread 0 has published the
// block's slots. Returns true in exactly one block per counter round (the
// last to arrive), which then resets the counter for the next launch.
__device__ __forceinline__ bool arrive_and_check_last(uint32_t* counter, uint32_t total, int* s_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (prev + 1u == total) ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

__device__ __forceinline__ void reset_counter(uint32_t* counter) {
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void raise_error(int32_t* err_flags, uint32_t bits) {
  if (err_flags != nullptr && bits != 0u)
    __hip_atomic_fetch_or(err_flags, static_cast<int32_t>(bits), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
