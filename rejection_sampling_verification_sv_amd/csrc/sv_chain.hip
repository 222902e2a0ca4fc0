// Chain verification kernels (modified rejection sampling over K proposals).
//
// Pass 1 — chain_stats_chunk_kernel (or chain_stats_segment_kernel). Streams
// every logit row of the call once (the K+1 target rows and K draft rows of
// each sequence) with coalesced 16-byte non-temporal loads: the logits are
// read once, and loads that do not allocate in the caches stream faster.
// Each thread keeps the running maximum m of its logits and the sum of
// 2^(x*c - m*c), c = log2(e)/T (one pass: a batch of values is reduced to its
// maximum first, the sum is rescaled once per batch, then the batch's
// exponentials are added; two batch buffers alternate so that one batch is
// always in flight). Each block combines its threads in fp64 and publishes
// one (reference, sum) pair per row piece. Work items:
//   chunked layout (rows on 16-byte boundaries, the usual case): each
//     sequence's rows, laid end to end, are cut into equal chunks, so every
//     block streams the same number of bytes;
//   segments layout (any row alignment): one item per (row, segment).
// The piece holding a drafted token also publishes that token's logit.
//
// Pass 2 — chain_sample_kernel, nblk_b workgroups per sequence (workgroup
// g of sequence b is block g * B + b):
//   1. each workgroup makes the sequence's decision for itself (the same
//      inputs and operations, so the same plan everywhere; no workgroup
//      waits for another): combines the pieces of the sequence's 2K+1 rows
//      into their log-normalisers L = log2 sum_v 2^(x_v c) (fp64), forms
//      p_k(x_k) and q_k(x_k) in fp64, alpha_k = min(1, p/q), accepts while
//      u_k < alpha_k and takes j = the first rejection with a wave ballot;
//      workgroup 0 writes the accepted prefix;
//      [Topologies] "Speculative Decoding & Draft Model Topologies", section 2
//      (acceptance-probability equation, timeline figure steps 2-3);
//      [In Production] "Speculative Decoding in Production", section 2.
//   2. workgroup g re-reads tiles [g * TPB, g * TPB + TPB) of row j (target, and
//      draft when j < K), forms the weights max(0, p_j - q_j) (or p_K for the
//      bonus draw) and publishes each tile's total;
//   3. the last workgroup of the sequence scans the tile totals, finds the
//      tile holding u_K * total, rescans it with a block-wide prefix sum and
//      picks the first token whose cumulative weight exceeds it.
//      [Topologies] section 2 (residual equation, step 4); [At Scale]
//      "Speculative Decoding at Scale", section 1; [Draft-and-Verify]
//      "Speculative Decoding for LLM Inference", "The draft-and-verify loop"
//      (the bonus token when every proposal is kept).
#include <hip/hip_ext.h>
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_stream.h"

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

}  // namespace

// ---------------------------------------------------------------- pass 1

namespace {

// The drafted token verified on row r of sequence b (target row k or draft
// row K+1+k carry token k; the bonus row K carries none): -1 if none.
__device__ __forceinline__ int row_token(const ChainParams& P, int b, int r) {
  const int k = r < P.K ? r : r - P.K - 1;
  return (r == P.K) ? -1 : P.tokens[static_cast<int64_t>(b) * P.K + k];
}

// Publish the logit of row r at its drafted token x (a valid id) for the
// decision, which then needs no dependent gather of its own.
template <class T>
__device__ __forceinline__ void publish_gather(const ChainParams& P, int b, int r, const void* row, int x) {
  publish(&P.gat[static_cast<int64_t>(b) * (2 * P.K + 1) + r], tag_float(load_elem<T>(row, x)));
}

// Segments layout: segment `seg` of row r of sequence b (any alignment), its
// (reference, sum) to slot (b * (2K+1) + r) * nseg + seg.
template <class T, bool kEnt>
__device__ void stats_segment(const ChainParams& P, int b, int r, int seg) {
  __shared__ float s_redf[kWaves];
  __shared__ double s_redd[kWaves];
  constexpr int VEC = T::kVec;
  constexpr int U = kStatsUnroll;
  const int R = 2 * P.K + 1;
  const int tid = threadIdx.x;

  const void* row = chain_row<T>(P, b, r);
  const Scale c = exponent_scale(temperature_of(P.temperature, b));

  // Split the row into an unaligned head, 16-byte vectors, and a tail.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  const int head = min(static_cast<int>(((16u - (addr & 15u)) & 15u) / T::kBytes), P.V);
  const int64_t nvec = (P.V - head) / VEC;
  const int tail = static_cast<int>((P.V - head) - nvec * VEC);
  const int64_t v0 = static_cast<int64_t>(seg) * P.L.seg_vecs;
  const int64_t v1 = min(nvec, v0 + P.L.seg_vecs);
  const uint4* body = reinterpret_cast<const uint4*>(static_cast<const char*>(row) + head * T::kBytes);

  const int x = (seg == 0 && tid == 0) ? row_token(P, b, r) : -1;
  Running st{-INFINITY, 0.0f, 0.0f};
  if (seg == 0 && tid < head) running_add1<kEnt>(st, load_elem<T>(row, tid), c);
  for (int64_t base = v0 + tid; base < v1; base += static_cast<int64_t>(kThreads) * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t vi = base + static_cast<int64_t>(u) * kThreads;
      raw[u] = (vi < v1) ? stream_load(body + vi) : neg_inf_vec<T>();
    }
    add_batch<T, U, kEnt>(st, raw, c);
  }
  if (seg == P.L.nseg - 1 && tid < tail) running_add1<kEnt>(st, load_elem<T>(row, head + nvec * VEC + tid), c);

  float MC;
  double S, A = 0.0;
  block_combine<kWaves, kEnt>(st, c, s_redf, s_redd, &MC, &S, &A);
  if (tid == 0) {
    const int64_t slot = (static_cast<int64_t>(b) * R + r) * P.L.nseg + seg;
    publish(&P.part_m[slot], tag_float(MC));
    publish(&P.part_s[slot], tag_nonneg_double(S));
    if constexpr (kEnt) publish(&P.part_a[slot], tag_any_double(A));
    if (x >= 0 && x < P.V) publish_gather<T>(P, b, r, row, x);
  }
}

// Chunked layout: chunk `ch` of sequence b covers the vectors
// [ch * per, (ch + 1) * per) of the sequence's 2K+1 rows laid end to end,
// streamed as one piece per row it touches; the piece of row r goes to slot
// (b * cps + ch) * kmax + (r - first row of the chunk).
template <class T, int TPB, bool kEnt>
__device__ void stats_chunk(const ChainParams& P, int b, int ch) {
  constexpr int NW = TPB / kWave;
  __shared__ float s_redf[NW];
  __shared__ double s_redd[NW];
  const int R = 2 * P.K + 1;
  const int64_t nvec = P.L.nvec;
  const int64_t lo = static_cast<int64_t>(ch) * P.L.per;
  const int64_t hi = min(static_cast<int64_t>(R) * nvec, lo + P.L.per);
  const int r_lo = static_cast<int>(div_nonneg(lo, nvec));
  const int r_hi = static_cast<int>(div_nonneg(hi - 1, nvec));
  LazyScale sc{P.temperature, b, false, Scale{0.0f, 0.0f}};
  for (int r = r_lo; r <= r_hi; ++r) {
    const int64_t p0 = max(lo, r * nvec) - r * nvec;
    const int64_t p1 = min(hi, (r + 1) * nvec) - r * nvec;
    const uint4* body = static_cast<const uint4*>(chain_row<T>(P, b, r));
    const int x = row_token(P, b, r);  // a uniform (scalar) load, consumed after the piece
    Running st{-INFINITY, 0.0f, 0.0f};
    flat_piece_stats<T, TPB, kEnt, kEnt ? kStreamUEnt : kStreamU>(body, p0, p1, sc, st);
    float MC;
    double S, A = 0.0;
    block_combine<NW, kEnt>(st, sc.get(), s_redf, s_redd, &MC, &S, &A);
    if (threadIdx.x == 0) {
      const int64_t slot = (static_cast<int64_t>(b) * P.L.cps + ch) * P.L.kmax + (r - r_lo);
      publish(&P.part_m[slot], tag_float(MC));
      publish(&P.part_s[slot], tag_nonneg_double(S));
      if constexpr (kEnt) publish(&P.part_a[slot], tag_any_double(A));
      // the piece holding the drafted token publishes its logit
      if (x >= 0 && x < P.V && x / T::kVec >= p0 && x / T::kVec < p1) publish_gather<T>(P, b, r, body, x);
    }
  }
}

// The small call's statistics chunk: stats_chunk's row pieces, batches of
// kStreamU vectors per thread and operations in the same order (so the same
// slots, bit for bit), with every load of the chunk issued before the first
// batch is reduced: one round trip instead of one per batch. Plain loads, so
// the rows stay in L2 for the row pair the sampling reads again. At most two
// row pieces and kMaxB batches; returns false, with nothing loaded, for a
// chunk that needs more (the caller streams it with stats_chunk).
template <class T, int TPB, int kMaxB>
__device__ bool stats_chunk_prefetched(const ChainParams& P, int b, int ch) {
  constexpr int NW = TPB / kWave;
  constexpr int U = kStreamU;
  constexpr int STEP = TPB * U;
  __shared__ float s_redf[NW];
  __shared__ double s_redd[NW];
  const int R = 2 * P.K + 1;
  const int64_t nvec = P.L.nvec;
  const int64_t lo = static_cast<int64_t>(ch) * P.L.per;
  const int64_t hi = min(static_cast<int64_t>(R) * nvec, lo + P.L.per);
  const int r_lo = static_cast<int>(div_nonneg(lo, nvec));
  const int r_hi = static_cast<int>(div_nonneg(hi - 1, nvec));
  if (r_hi - r_lo > 1) return false;
  // piece 0: row r_lo, vectors [a0, a1); piece 1 (r_hi > r_lo): row r_hi, [0, b1)
  const int64_t a0 = lo - r_lo * nvec;
  const int64_t a1 = min(hi, (r_lo + 1) * nvec) - r_lo * nvec;
  const int64_t b1 = (r_hi > r_lo) ? hi - r_hi * nvec : 0;
  const int nb0 = static_cast<int>((a1 - a0 + STEP - 1) / STEP);
  const int nb1 = static_cast<int>((b1 + STEP - 1) / STEP);
  if (nb0 + nb1 > kMaxB) return false;
  const uint4* body0 = static_cast<const uint4*>(chain_row<T>(P, b, r_lo));
  const uint4* body1 = static_cast<const uint4*>(chain_row<T>(P, b, r_hi));
  const int x0 = row_token(P, b, r_lo);
  const int x1 = row_token(P, b, r_hi);
  uint4 raw[kMaxB][U];
#pragma unroll
  for (int q = 0; q < kMaxB; ++q) {
    const bool second = q >= nb0;
    const int64_t start = second ? 0 : a0;
    const int64_t end = second ? b1 : a1;
    const uint4* body = second ? body1 : body0;
    const int64_t k0 = static_cast<int64_t>(second ? q - nb0 : q) * STEP + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = k0 + u * TPB;
      raw[q][u] = (q < nb0 + nb1 && start + k < end) ? body[start + k] : neg_inf_vec<T>();
    }
  }
  const Scale c = exponent_scale(temperature_of(P.temperature, b));
#pragma unroll
  for (int piece = 0; piece < 2; ++piece) {
    if (piece == 1 && r_hi == r_lo) break;
    Running st{-INFINITY, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < kMaxB; ++q)
      if ((piece == 0 && q < nb0) || (piece == 1 && q >= nb0 && q < nb0 + nb1)) add_batch<T, U, false>(st, raw[q], c);
    float MC;
    double S;
    block_combine<NW, false>(st, c, s_redf, s_redd, &MC, &S);
    if (threadIdx.x == 0) {
      const int r = piece == 0 ? r_lo : r_hi;
      const int64_t p0 = piece == 0 ? a0 : 0;
      const int64_t p1 = piece == 0 ? a1 : b1;
      const int x = piece == 0 ? x0 : x1;
      const int64_t slot = (static_cast<int64_t>(b) * P.L.cps + ch) * P.L.kmax + (r - r_lo);
      publish(&P.part_m[slot], tag_float(MC));
      publish(&P.part_s[slot], tag_nonneg_double(S));
      if (x >= 0 && x < P.V && x / T::kVec >= p0 && x / T::kVec < p1)
        publish_gather<T>(P, b, r, piece == 0 ? body0 : body1, x);
    }
  }
  return true;
}

// ---------------------------------------------------------------- pass 2

// The decision of sequence b, made by wave 0 of every sampling workgroup of
// the sequence (the same inputs and operations give every one the same
// plan, so no workgroup waits for another). All of its loads are issued
// before any of them is used: one round trip. The rows' log-normalisers come
// from the statistics pieces (G lanes per row, G the largest power of two
// that fits all 2K+1 rows in one wave or covers a row's pieces; rounds of up
// to four pieces per lane): group max of the references M, each lane
// rescales its sums by 2^(m - M) in fp64, group sum Z, L = M + log2 Z. Lane
// k < K holds drafted token k, its uniform and the logits pass 1 published
// for it; p_k(x_k), q_k(x_k) in fp64, alpha_k = min(1, p/q), acceptance while
// u_k < alpha_k, j = the first rejection (ballot). Leaves the sampling plan in
// *s_plan; the `writer` also writes accept_len, the accepted prefix of
// out_tokens, p_draft / q_draft and the error bits.
// Issue the loads of pieces p0, p0 + G, p0 + 2G, p0 + 3G of row r (r < 0:
// none) and return how many exist; every lane issues all eight loads (the
// missing ones read any_slot and are dropped), so they are in flight together.
template <bool kEnt>
__device__ __forceinline__ int issue_pieces(const ChainParams& P, int b, int r, int p0, int G, int pmax,
                                            int64_t any_slot, uint64_t (&rm)[4], uint64_t (&rs)[4],
                                            uint64_t (&ra)[4]) {
  int64_t sl[4];
  int n = 0;
  if (P.L.cps > 0 && r >= 0) {
    // chunked: row r's pieces are chunks ch0 .. chl; only the first one can
    // start in an earlier row (three divisions per lane, not three per piece)
    const PieceLayout& L = P.L;
    const int64_t ch0 = div_nonneg(r * L.nvec, L.per);
    const int64_t chl = div_nonneg((r + 1) * L.nvec - 1, L.per);
    const int64_t first_row0 = div_nonneg(ch0 * L.per, L.nvec);
    const int64_t base = static_cast<int64_t>(b) * L.cps;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + i * G;
      const int64_t ch = ch0 + p;
      sl[i] = (ch <= chl) ? (base + ch) * L.kmax + (p == 0 ? r - first_row0 : 0) : -1;
      if (sl[i] >= 0 && n == i) n = i + 1;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sl[i] = (r >= 0 && p0 + i * G < pmax) ? piece_slot(P.L, b, r, p0 + i * G) : -1;
      if (sl[i] >= 0 && n == i) n = i + 1;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t a = i < n ? sl[i] : any_slot;
    rm[i] = P.part_m[a];
    rs[i] = P.part_s[a];
    ra[i] = kEnt ? P.part_a[a] : 0ull;
  }
  return n;
}

// OR of the error bits (SV_ERRF_*, bits 0..4) over the wave: one ballot per
// bit instead of a chain of shuffles.
__device__ __forceinline__ uint32_t wave_or_err(uint32_t v) {
  static_assert((SV_ERRF_TOKEN | SV_ERRF_TEMPERATURE | SV_ERRF_PARENT | SV_ERRF_NONFINITE | SV_ERRF_INTERNAL) == 0x1f,
                "error bits are bits 0..4");
  uint32_t r = 0u;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit)
    if (__ballot((v >> bit) & 1u) != 0ull) r |= 1u << bit;
  return r;
}

// One step of a reduction over aligned groups of 2o lanes (o a power of
// two), after which every lane of each half of a group holds the same value:
// the value of a lane in the other half. DPP moves within a row of 16 lanes
// (quad permutes, then the half-row and row mirrors), an LDS permute beyond.
__device__ __forceinline__ float other_half(float v, int o) {
  switch (o) {
    case 1: return dpp_move<0xb1>(v);
    case 2: return dpp_move<0x4e>(v);
    case 4: return dpp_move<0x141>(v);
    case 8: return dpp_move<0x140>(v);
    default: return __shfl_xor(v, o, kWave);
  }
}
__device__ __forceinline__ double other_half(double v, int o) {
  switch (o) {
    case 1: return dpp_f64<0xb1>(v);
    case 2: return dpp_f64<0x4e>(v);
    case 4: return dpp_f64<0x141>(v);
    case 8: return dpp_f64<0x140>(v);
    default: return __shfl_xor(v, o, kWave);
  }
}

// The decision of sequence b once its rows' log-normalisers are in s_L
// (wave 0; lane k < K holds drafted token k, its uniform and the two
// gathered logits): p_k(x_k), q_k(x_k) in fp64, alpha_k = min(1, p/q),
// acceptance while u_k < alpha_k, j = the first rejection (ballot). Leaves
// the sampling plan in *s_plan; the `writer` also writes accept_len, the
// accepted prefix of out_tokens, p_draft / q_draft and the error bits.
template <class T>
__device__ __forceinline__ void decide_tail(const ChainParams& P, int b, SeqPlan* s_plan, bool writer,
                                            const double* s_L, int x, float u, uint64_t vt, uint64_t vd,
                                            uint32_t err, float Tv, Scale c) {
  const int K = P.K;
  const int lane = lane_id();
  // s_L is written by the group leaders and read by other lanes of this wave.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  float lt = 0.0f, ld = 0.0f;
  if (lane < K) {
    if (x < 0 || x >= P.V) {
      err |= SV_ERRF_TOKEN;
    } else {
      if (vt == 0ull || vd == 0ull) err |= kErrInternal;
      lt = untag_float(vt);
      ld = untag_float(vd);
    }
  }
  if (!(Tv > 0.0f) || !isfinite(Tv)) err |= SV_ERRF_TEMPERATURE;
  const double c64 = static_cast<double>(c.hi) + static_cast<double>(c.lo);
  bool reject = false;
  if (lane < K) {
    float pf = NAN, qf = NAN;
    if (x >= 0 && x < P.V) {
      // p = 2^ap, q = 2^aq; alpha = min(1, p / q) = 2^min(0, ap - aq)
      const double ap = static_cast<double>(lt) * c64 - s_L[lane];
      const double aq = static_cast<double>(ld) * c64 - s_L[K + 1 + lane];
      const double p = exp2_split(ap);
      const double q = exp2_split(aq);
      const double alpha = (p > 0.0) ? ((q > 0.0) ? ((ap >= aq) ? 1.0 : exp2_split(ap - aq)) : 1.0) : 0.0;
      reject = !(static_cast<double>(u) < alpha);
      pf = static_cast<float>(p);
      qf = static_cast<float>(q);
    }
    if (writer && P.p_draft != nullptr) P.p_draft[static_cast<int64_t>(b) * K + lane] = pf;
    if (writer && P.q_draft != nullptr) P.q_draft[static_cast<int64_t>(b) * K + lane] = qf;
  }
  const uint64_t rej = __ballot(reject);
  const int j = (rej != 0ull) ? (__ffsll(static_cast<unsigned long long>(rej)) - 1) : K;
  err = wave_or_err(err);
  const bool bad = err != 0u;

  // Lane i writes out_tokens[i] (K + 1 <= 64): its own token up to j, -1 after;
  // the drawn token at j is written by the sampling pass.
  if (writer && lane <= K && !(lane == j && !bad))
    P.out_tokens[static_cast<int64_t>(b) * (K + 1) + lane] = (bad || lane > j) ? -1 : x;
  if (lane == 0) {
    if (writer) {
      if (P.accept_len != nullptr) P.accept_len[b] = bad ? -1 : j;
      if (bad && P.residual_mass != nullptr) P.residual_mass[b] = -1.0f;
      if (bad && P.drawn_prob != nullptr) P.drawn_prob[b] = NAN;
      raise_error(P.err_flags, err);
    }
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
    pl.pad = 0u;
    *s_plan = pl;
  }
}

template <class T, bool kEnt>
__device__ void decide_wave(const ChainParams& P, int b, SeqPlan* s_plan, bool writer) {
  __shared__ double s_L[2 * SV_MAX_K + 1];
  const int K = P.K;
  const int R = 2 * K + 1;
  const int lane = lane_id();
  uint32_t err = 0u;

  const int pmax = max_pieces(P.L);
  int G = 1;
  while (G < pmax && R * 2 * G <= kWave) G <<= 1;
  const int64_t any_slot = static_cast<int64_t>(b) * slots_per_seq(P.L);  // a valid address

  // The loads of the usual case all go out before any is used: the first
  // round of this lane's statistics pieces (every piece when the rows fit
  // one wave and have at most 4 G pieces), then the drafted tokens' inputs.
  uint64_t rm0[4], rs0[4], ra0[4];
  const int n0 = issue_pieces<kEnt>(P, b, lane / G < R ? lane / G : -1, lane % G, G, pmax, any_slot, rm0, rs0, ra0);
  const float Tv = temperature_of(P.temperature, b);
  int x = -1;
  float u = 0.0f;
  uint64_t vt = 0ull, vd = 0ull;
  if (K > 0) {  // every lane loads (lanes past K repeat lane K - 1's values and drop them)
    const int k = min(lane, K - 1);
    x = P.tokens[static_cast<int64_t>(b) * K + k];
    u = P.uniforms[static_cast<int64_t>(b) * (K + 1) + k];
    vt = P.gat[static_cast<int64_t>(b) * R + k];
    vd = P.gat[static_cast<int64_t>(b) * R + K + 1 + k];
    if (lane >= K) x = -1;
  }

  for (int r0 = 0; r0 < R; r0 += kWave / G) {
    const int r = r0 + lane / G;
    const int gl = lane % G;
    const bool row_ok = r < R;
    // this lane's pieces p = gl, gl + G, ...: rounds of up to four loads in
    // flight, each round folded into (mf, zf) = (reference, fp64 sum)
    // (and with the entropy requested, af = the fp64 sum of 2^a * a at the
    // reference mf: a piece moved to a reference higher by d contributes
    // 2^-d (A - d S))
    constexpr bool ent = kEnt;
    float mf = -INFINITY;
    double zf = 0.0, af = 0.0;
    bool more = row_ok;
    for (int p0 = gl; more; p0 += 4 * G) {
      uint64_t rm[4], rs[4], ra[4];
      int n;
      if (r0 == 0 && p0 == gl) {
        n = n0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rm[i] = rm0[i];
          rs[i] = rs0[i];
          ra[i] = ra0[i];
        }
      } else {
        n = issue_pieces<kEnt>(P, b, r, p0, G, pmax, any_slot, rm, rs, ra);
      }
      more = (n == 4);
      for (int i = 0; i < n; ++i) {
        if (rm[i] == 0ull || rs[i] == 0ull || (ent && ra[i] == 0ull)) err |= kErrInternal;
        const float mm = untag_float(rm[i]);
        const double sv = untag_nonneg_double(rs[i]);
        const double av = untag_any_double(ra[i]);
        if (mm == -INFINITY) continue;
        if (mm > mf) {
          const double d = static_cast<double>(mm) - static_cast<double>(mf);
          const double f = (mf == -INFINITY) ? 0.0 : ref_factor(mf, mm);
          if constexpr (ent) af = (mf == -INFINITY ? 0.0 : f * (af - d * zf)) + av;
          zf = zf * f + sv;
          mf = mm;
        } else {
          const double d = static_cast<double>(mf) - static_cast<double>(mm);
          const double f = ref_factor(mm, mf);
          zf += sv * f;
          if constexpr (ent) af += f * (av - d * sv);
        }
      }
    }
    float M = mf;
    for (int o = 1; o < G; o <<= 1) M = fmaxf(M, other_half(M, o));
    const double dl = static_cast<double>(M) - static_cast<double>(mf);
    const double fl = (mf == -INFINITY) ? 0.0 : ref_factor(mf, M);
    double zl = zf * fl;
    for (int o = 1; o < G; o <<= 1) zl += other_half(zl, o);
    double al = 0.0;
    if constexpr (ent) {
      al = (mf == -INFINITY) ? 0.0 : fl * (af - dl * zf);
      for (int o = 1; o < G; o <<= 1) al += other_half(al, o);
    }
    if (row_ok && gl == 0) {
      const bool fin = (zl > 0.0) && isfinite(zl) && isfinite(M);
      if (!fin) err |= SV_ERRF_NONFINITE;
      const double lz = fin ? log2_fast(zl) : log2(zl);
      s_L[r] = static_cast<double>(M) + lz;
      // H = ln 2 * (log2 Z - A / Z); NaN for a row without finite statistics
      if (ent && writer)
        P.entropy[static_cast<int64_t>(b) * R + r] =
            (fin && Tv > 0.0f && isfinite(Tv)) ? static_cast<float>(0.6931471805599453 * (lz - al / zl)) : NAN;
    }
  }
  decide_tail<T>(P, b, s_plan, writer, s_L, x, u, vt, vd, err, Tv, exponent_scale(Tv));
}

// Lanes per row of the decision's statistics combine: the largest power of
// two G (at most one past the row's piece count) with 2K+1 rows of 2G lanes
// fitting a wave, as decide_wave takes it.
__device__ __forceinline__ int decision_lanes(int R, int pmax) {
  int G = 1;
  while (G < pmax && R * 2 * G <= kWave) G <<= 1;
  return G;
}

// One-launch call: the decision of sequence b (wave 0) from statistics
// written by running workgroups of the same launch. The host takes the
// one-launch call only when every piece of every row is in the first round
// of decide_wave (at most 4 pieces per lane, 2K+1 rows of G lanes in one
// wave, chunk indices within 32 bits), and this function makes exactly
// decide_wave's operations in the same order on that round, so the
// normalisers, and every output, are bit-identical to the two-launch call.
// Every slot is read with an agent-scope load, all issued together; a slot
// still zero (its store not visible yet) makes the wave return false before
// anything is written, for the caller to read again.
// The inputs of sequence b's decision that do not come from the statistics
// (wave 0; lane k < K gets drafted token k and its uniform): loaded, and the
// temperature's scale formed, once before the statistics are polled.
struct DecideIn {
  int x;
  float u;
  float Tv;
  Scale c;
};

__device__ __forceinline__ DecideIn decide_inputs(const ChainParams& P, int b) {
  DecideIn in;
  in.Tv = temperature_of(P.temperature, b);
  in.x = -1;
  in.u = 0.0f;
  const int K = P.K;
  if (K > 0) {  // every lane loads (lanes past K repeat lane K - 1's values and drop them)
    const int lane = lane_id();
    const int k = min(lane, K - 1);
    in.x = P.tokens[static_cast<int64_t>(b) * K + k];
    in.u = P.uniforms[static_cast<int64_t>(b) * (K + 1) + k];
    if (lane >= K) in.x = -1;
  }
  in.c = exponent_scale(in.Tv);
  return in;
}

template <class T, bool kEnt = false>
__device__ __forceinline__ bool decide_live_wave(const ChainParams& P, int b, SeqPlan* s_plan, bool writer,
                                                 const DecideIn& in) {
  __shared__ double s_L[2 * SV_MAX_K + 1];
  const int K = P.K;
  const int R = 2 * K + 1;
  const int lane = lane_id();
  const PieceLayout& L = P.L;
  const int G = decision_lanes(R, max_pieces(L));
  const int r = lane / G;
  const int gl = lane % G;
  const bool row_ok = r < R;
  uint32_t err = 0u;

  // this lane's pieces gl + i G of row r: chunks ch0 + gl + i G up to chl
  const uint32_t nv = static_cast<uint32_t>(L.nvec), pr = static_cast<uint32_t>(L.per);
  const uint32_t rr = row_ok ? static_cast<uint32_t>(r) : 0u;
  const uint32_t ch0 = rr * nv / pr;
  const uint32_t chl = ((rr + 1u) * nv - 1u) / pr;
  const uint32_t first_row0 = ch0 * pr / nv;
  const int64_t base = static_cast<int64_t>(b) * L.cps;
  const int64_t any_slot = base * L.kmax;  // a valid address
  uint64_t rm[4], rs[4], ra[4];
  bool has[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = static_cast<uint32_t>(gl + i * G);
    const uint32_t ch = ch0 + p;
    has[i] = row_ok && ch <= chl;
    const int64_t sl = has[i] ? (base + ch) * L.kmax + (p == 0u ? rr - first_row0 : 0u) : any_slot;
    rm[i] = peek(&P.part_m[sl]);
    rs[i] = peek(&P.part_s[sl]);
    ra[i] = kEnt ? peek(&P.part_a[sl]) : 0ull;
  }
  const float Tv = in.Tv;
  const int x = in.x;
  uint64_t vt = 0ull, vd = 0ull;
  if (K > 0) {
    const int k = min(lane, K - 1);
    vt = peek(&P.gat[static_cast<int64_t>(b) * R + k]);
    vd = peek(&P.gat[static_cast<int64_t>(b) * R + K + 1 + k]);
  }
  bool missing = lane < K && x >= 0 && x < P.V && (vt == 0ull || vd == 0ull);
#pragma unroll
  for (int i = 0; i < 4; ++i) missing |= has[i] && (rm[i] == 0ull || rs[i] == 0ull || (kEnt && ra[i] == 0ull));
  if (__ballot(missing) != 0ull) return false;

  // decide_wave's combine of one round: running reference mf, fp64 sum zf
  // (and af, the fp64 sum of 2^a * a at the reference mf)
  float mf = -INFINITY;
  double zf = 0.0, af = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!has[i]) continue;
    const float mm = untag_float(rm[i]);
    const double sv = untag_nonneg_double(rs[i]);
    const double av = untag_any_double(ra[i]);
    if (mm == -INFINITY) continue;
    if (mm > mf) {
      const double d = static_cast<double>(mm) - static_cast<double>(mf);
      const double f = (mf == -INFINITY) ? 0.0 : ref_factor(mf, mm);
      if constexpr (kEnt) af = (mf == -INFINITY ? 0.0 : f * (af - d * zf)) + av;
      zf = zf * f + sv;
      mf = mm;
    } else {
      const double d = static_cast<double>(mf) - static_cast<double>(mm);
      const double f = ref_factor(mm, mf);
      zf += sv * f;
      if constexpr (kEnt) af += f * (av - d * sv);
    }
  }
  float M = mf;
  for (int o = 1; o < G; o <<= 1) M = fmaxf(M, other_half(M, o));
  const double dl = static_cast<double>(M) - static_cast<double>(mf);
  const double fl = (mf == -INFINITY) ? 0.0 : ref_factor(mf, M);
  double zl = zf * fl;
  for (int o = 1; o < G; o <<= 1) zl += other_half(zl, o);
  double al = 0.0;
  if constexpr (kEnt) {
    al = (mf == -INFINITY) ? 0.0 : fl * (af - dl * zf);
    for (int o = 1; o < G; o <<= 1) al += other_half(al, o);
  }
  if (row_ok && gl == 0) {
    const bool fin = (zl > 0.0) && isfinite(zl) && isfinite(M);
    if (!fin) err |= SV_ERRF_NONFINITE;
    const double lz = fin ? log2_fast(zl) : log2(zl);
    s_L[r] = static_cast<double>(M) + lz;
    // H = ln 2 * (log2 Z - A / Z), as decide_wave
    if (kEnt && writer)
      P.entropy[static_cast<int64_t>(b) * R + r] =
          (fin && Tv > 0.0f && isfinite(Tv)) ? static_cast<float>(0.6931471805599453 * (lz - al / zl)) : NAN;
  }
  decide_tail<T>(P, b, s_plan, writer, s_L, x, in.u, vt, vd, err, Tv, in.c);
  return true;
}

// One-launch call: wave 0 of a sampling workgroup of sequence b waits until
// every statistics chunk of b has been counted (P.done[b] reaches the chunks
// per sequence), then makes the decision, reading the slots again while a
// store is not yet visible. Every chunk it waits for was handed out by the
// sequence's ticket queue before this sampling role, to a workgroup that is
// running and waits for nothing, so the wait ends; it is still bounded
// like await_slot. Returns false on expiry or on an abort raised elsewhere.
template <class T, bool kEnt = false>
__device__ bool decide_live(const ChainParams& P, int b, SeqPlan* s_plan, bool writer) {
  const uint32_t need = static_cast<uint32_t>(P.L.cps);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const DecideIn in = decide_inputs(P, b);
  uint32_t* done = P.done + static_cast<int64_t>(b) * kCtrStride;
  // Once at most SV_EAGER_CHUNKS chunks are uncounted, the slots themselves
  // are read on every poll: the decision goes ahead as soon as every slot is
  // visible, whether or not the last counts have landed (the workgroup that
  // returns the counter to zero waits for them, see sample_finish).
  uint32_t d = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (d + static_cast<uint32_t>(SV_EAGER_CHUNKS) < need) {
    if (peek(P.abort) != 0ull) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      publish(P.abort, 1ull);
      return false;
    }
    __builtin_amdgcn_s_sleep(SV_POLL_SLEEP);
    d = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (SV_TAIL_PRIO > 0) __builtin_amdgcn_s_setprio(SV_TAIL_PRIO);
  while (!decide_live_wave<T, kEnt>(P, b, s_plan, writer, in)) {
    if (peek(P.abort) != 0ull) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      publish(P.abort, 1ull);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

template <class T>
struct SampleTiles;
template <>
struct SampleTiles<BF16> {
  static constexpr int kPerBlock = kSampleTilesBF16;
};
template <>
struct SampleTiles<F32> {
  static constexpr int kPerBlock = kSampleTilesF32;
};

// 16-byte vectors holding one thread's kSampleEPT logits of a tile.
template <class T>
constexpr int kEptVecs = kSampleEPT / T::kVec;

// Logits [e0, e0 + T::kVec) of a row packed as one raw 16-byte vector, -inf
// beyond V (element loads: for rows off a 16-byte boundary and the tail).
template <class T>
__device__ __forceinline__ uint4 pack_elems(const void* row, int64_t e0, int V);
template <>
__device__ __forceinline__ uint4 pack_elems<BF16>(const void* row, int64_t e0, int V) {
  const uint16_t* p = static_cast<const uint16_t*>(row);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (e0 + 2 * i < V) ? p[e0 + 2 * i] : 0xff80u;
    const uint32_t hi = (e0 + 2 * i + 1 < V) ? p[e0 + 2 * i + 1] : 0xff80u;
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ uint4 pack_elems<F32>(const void* row, int64_t e0, int V) {
  const uint32_t* p = static_cast<const uint32_t*>(row);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (e0 + i < V) ? p[e0 + i] : 0xff800000u;
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One thread's kSampleEPT logits of a tile starting at element e0.
template <class T>
__device__ __forceinline__ void load_raw(const void* row, int64_t e0, int V, uint4 (&r)[kEptVecs<T>]) {
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0u;
  if (aligned && e0 + kSampleEPT <= V) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(row) + e0 * T::kBytes);
#pragma unroll
    for (int v = 0; v < kEptVecs<T>; ++v) r[v] = p[v];
  } else {
#pragma unroll
    for (int v = 0; v < kEptVecs<T>; ++v) r[v] = pack_elems<T>(row, e0 + v * T::kVec, V);
  }
}

struct SampleRows {
  const void* t;  // target row j
  const void* d;  // draft row j, or nullptr when drawing from p only
  Scale c;
  float neg_lt_hi, neg_lt_lo;  // -L_t
  float neg_d_hi, neg_d_lo;    // -(L_d - L_t)
};

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

// Weights of this thread's kSampleEPT tokens, and their running fp32 sum (the
// same operations in the same order wherever it is called).
//   bonus / p only:  w = p_t(v) = 2^(x_t c - L_t)
//   residual:        w = p_t(v) * max(0, 1 - 2^((x_d - x_t) c - (L_d - L_t)))
//                      = max(0, p_t(v) - p_d(v))
// The ratio form keeps the exponent small exactly where p_t and p_d nearly
// cancel, and any rounding common to all weights cancels in the draw.
template <class T>
__device__ __forceinline__ float tile_compute(const SampleRows& S, const uint4 (&rt)[kEptVecs<T>],
                                              const uint4 (&rd)[kEptVecs<T>], float (&w)[kSampleEPT]) {
  float xt[kSampleEPT];
#pragma unroll
  for (int v = 0; v < kEptVecs<T>; ++v) unpack<T>(rt[v], &xt[v * T::kVec]);
#pragma unroll
  for (int i = 0; i < kSampleEPT; ++i) w[i] = fast_exp2(scaled_arg(xt[i], S.c, S.neg_lt_hi) + S.neg_lt_lo);
  if (S.d != nullptr) {
    float xd[kSampleEPT];
#pragma unroll
    for (int v = 0; v < kEptVecs<T>; ++v) unpack<T>(rd[v], &xd[v * T::kVec]);
#pragma unroll
    for (int i = 0; i < kSampleEPT; ++i) {
      const float ratio = fast_exp2(scaled_arg(xd[i] - xt[i], S.c, S.neg_d_hi) + S.neg_d_lo);
      w[i] = w[i] * fmaxf(1.0f - ratio, 0.0f);
    }
  }
  float run = 0.0f;
#pragma unroll
  for (int i = 0; i < kSampleEPT; ++i) run += w[i];
  return run;
}

template <class T>
__device__ __forceinline__ float tile_weights(const SampleRows& S, int64_t tile, int V, float (&w)[kSampleEPT]) {
  const int64_t e0 = tile * kSampleTile + static_cast<int64_t>(threadIdx.x) * kSampleEPT;
  uint4 rt[kEptVecs<T>], rd[kEptVecs<T>] = {};
  load_raw<T>(S.t, e0, V, rt);
  if (S.d != nullptr) load_raw<T>(S.d, e0, V, rd);
  return tile_compute<T>(S, rt, rd, w);
}

// Rescan tile `tile` of the sampling row: the first token (ascending id) with
// a positive weight whose cumulative weight within the tile exceeds
// `target`; if rounding leaves none, the last token with a positive weight.
__device__ int draw_in_weights(int tile, const float (&w)[kSampleEPT], float x, double target, double* s_scan,
                               int* s_redi);

template <class T>
__device__ int draw_in_tile(const SampleRows& Sr, int tile, double target, int V, double* s_scan, int* s_redi) {
  float w[kSampleEPT];
  const float x = tile_weights<T>(Sr, tile, V, w);
  return draw_in_weights(tile, w, x, target, s_scan, s_redi);
}

// The rescan of draw_in_tile on weights already formed (w, and x their
// running sum, as tile_compute returns them). Each thread's exclusive prefix
// within the tile is the fp64 DPP scan of its wave plus the totals of the
// waves before it (one barrier); each wave's first crossing and last
// positive weight come from two ballots, and a second barrier lets every
// thread take the block's: the lowest crossing index, else the last
// positive weight. s_scan holds kWaves values and s_redi 2 kWaves; a caller
// that uses them again afterwards needs a barrier first.
__device__ int draw_in_weights(int tile, const float (&w)[kSampleEPT], float x, double target, double* s_scan,
                               int* s_redi) {
  const int lane = lane_id();
  const int wv = wave_id();
  const double inc = wave_scan_dpp(static_cast<double>(x));
  if (lane == kWave - 1) s_scan[wv] = inc;
  __syncthreads();
  double wave_prefix = 0.0;
  for (int k = 0; k < wv; ++k) wave_prefix += s_scan[k];
  const double excl = wave_prefix + wave_exclusive_from(inc);
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
  // indices grow with the lane and the wave: the wave's lowest crossing is
  // its lowest lane's, its last positive weight its highest lane's
  const uint64_t fb = __ballot(first != INT_MAX);
  const uint64_t lb = __ballot(lastpos >= 0);
  const int wf = (fb != 0ull) ? __builtin_amdgcn_readlane(first, __ffsll(static_cast<unsigned long long>(fb)) - 1)
                              : INT_MAX;
  const int wl = (lb != 0ull) ? __builtin_amdgcn_readlane(lastpos, 63 - __clzll(static_cast<long long>(lb))) : -1;
  if (lane == 0) {
    s_redi[wv] = wf;
    s_redi[kWaves + wv] = wl;
  }
  __syncthreads();
  int first_all = INT_MAX, last_all = -1;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    first_all = min(first_all, s_redi[k]);
    last_all = max(last_all, s_redi[kWaves + k]);
  }
  const int e = (first_all >= 0 && first_all < kSampleTile) ? first_all : last_all;
  return (e >= 0) ? static_cast<int>(static_cast<int64_t>(tile) * kSampleTile + e) : -1;
}

// Step one of the draw, by wave 0 once every tile total of sequence b is
// published (read with await_slot): the total weight S (fp64, tile order)
// and the tile holding u_K * S, with the target left inside it, into the
// caller's shared variables. Up to 64 tiles (the usual case) take one
// inclusive scan; more tiles are scanned in rounds of 64, twice (total
// first, then the search). No tile crossing the target (rounding at the top
// end): the last tile with weight, target +inf; none with weight: tile -1.
// pre: with up to 64 tiles, lane t's slot as the caller already read it
// (0: not read, or not visible then; read again here).
__device__ void locate_tile(const ChainParams& P, int b, double* s_S, int* s_tile, double* s_target,
                            uint32_t* s_err, uint64_t pre = 0ull) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  uint64_t* ts = P.tile_sum + static_cast<int64_t>(b) * P.ntiles;
  const double u = static_cast<double>(P.uniforms[static_cast<int64_t>(b) * (P.K + 1) + P.K]);
  if (tid < kWave) {
    uint32_t err = 0u;
    double total, target, prefix = 0.0;
    int found = -1, last_pos = -1;
    if (P.ntiles <= kWave) {
      const double v =
          (lane < P.ntiles) ? untag_nonneg_double(pre != 0ull ? pre : await_slot(&ts[lane], &err, P.abort)) : 0.0;
      const double inc = wave_scan_dpp(v);
      const double excl = wave_exclusive_from(inc);
      const uint64_t pos = __ballot(lane < P.ntiles && v > 0.0);
      if (pos != 0ull) last_pos = 63 - __clzll(static_cast<long long>(pos));
      total = readlane_f64(inc, kWave - 1);
      target = u * total;
      const uint64_t hit = __ballot(lane < P.ntiles && v > 0.0 && inc > target);
      if (hit != 0ull) {
        found = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        prefix = readlane_f64(excl, found);
      }
    } else {
      double carry = 0.0;
      for (int base = 0; base < P.ntiles; base += kWave) {
        const int t = base + lane;
        const double v = (t < P.ntiles) ? untag_nonneg_double(await_slot(&ts[t], &err, P.abort)) : 0.0;
        const double inc = wave_scan_dpp(v);
        const uint64_t pos = __ballot(t < P.ntiles && v > 0.0);
        if (pos != 0ull) last_pos = base + 63 - __clzll(static_cast<long long>(pos));
        carry += readlane_f64(inc, kWave - 1);
      }
      total = carry;
      target = u * total;
      carry = 0.0;
      for (int base = 0; base < P.ntiles && found < 0; base += kWave) {
        const int t = base + lane;
        const double v = (t < P.ntiles) ? untag_nonneg_double(peek(&ts[t])) : 0.0;  // seen above
        const double inc = wave_scan_dpp(v);
        const double excl = wave_exclusive_from(inc);
        const uint64_t hit = __ballot(t < P.ntiles && v > 0.0 && carry + inc > target);
        if (hit != 0ull) {
          const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
          found = base + l;
          prefix = carry + readlane_f64(excl, l);
        }
        carry += readlane_f64(inc, kWave - 1);
      }
    }
    if (err != 0u) atomicOr(s_err, err);
    if (tid == 0) {
      *s_S = total;
      if (found >= 0) {
        *s_tile = found;
        *s_target = target - prefix;
      } else {  // rounding at the top end: the last tile with weight
        *s_tile = last_pos;
        *s_target = INFINITY;
      }
    }
  }
}

// Draw the token: called by the last resolving workgroup of sequence b, once
// every workgroup of the sequence has published its tile totals (pre: as
// locate_tile takes it).
template <class T>
__device__ __forceinline__ void chain_draw(const ChainParams& P, int b, const SeqPlan& pl, uint64_t pre = 0ull) {
  __shared__ double s_scan[kWaves];
  __shared__ int s_redi[2 * kWaves];
  __shared__ double s_S, s_target;
  __shared__ int s_tile;
  __shared__ uint32_t s_err;
  const int tid = threadIdx.x;
  const double u = static_cast<double>(P.uniforms[static_cast<int64_t>(b) * (P.K + 1) + P.K]);
  if (tid == 0) s_err = 0u;
  __syncthreads();

  locate_tile(P, b, &s_S, &s_tile, &s_target, &s_err, pre);
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
    if (P.drawn_prob != nullptr) {
      // p_j of the drawn token in fp64 from its logit and the plan: 2^(x c - L_j)
      float pr = NAN;
      if (token >= 0) {
        const double x = static_cast<double>(load_elem<T>(chain_row<T>(P, b, pl.j), token));
        const double c64 = static_cast<double>(pl.c_hi) + static_cast<double>(pl.c_lo);
        pr = static_cast<float>(exp2(x * c64 - (static_cast<double>(pl.lt_hi) + static_cast<double>(pl.lt_lo))));
      }
      P.drawn_prob[b] = pr;
    }
    raise_error(P.err_flags, s_err);
  }
}

// Tiles [t_begin, t_end) of sequence b's sampling row pair (plan pl): the
// weights of each tile, TPB tiles with their loads in flight together, and
// each tile's total published to its slot.
// kKeep: the caller's tiles fit one group (t_end - t_begin <= TPB), and the
// weights of tile t_begin + i and their running sum stay in keep[i],
// keepx[i] (for the draw of the small call).
template <class T, int TPB, bool kDraft, bool kKeep = false>
__device__ __forceinline__ void tile_totals(const ChainParams& P, int b, const SeqPlan& pl, int t_begin, int t_end,
                            float (*keep)[kSampleEPT] = nullptr, float* keepx = nullptr) {
  constexpr int NV = kEptVecs<T>;
  __shared__ double s_red[TPB][kWaves];
  const SampleRows S = sample_rows<T>(P, b, pl, false);
#pragma unroll 1
  for (int t0 = t_begin; t0 < t_end; t0 += TPB) {
    uint4 rt[TPB][NV], rd[kDraft ? TPB : 1][NV] = {};
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
      if (t0 + i < t_end) {
        const int64_t e0 =
            static_cast<int64_t>(t0 + i) * kSampleTile + static_cast<int64_t>(threadIdx.x) * kSampleEPT;
        load_raw<T>(S.t, e0, P.V, rt[i]);
        if (kDraft && S.d != nullptr) load_raw<T>(S.d, e0, P.V, rd[kDraft ? i : 0]);
      }
    }
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
      float w[kSampleEPT];
      float x = 0.0f;
      if (t0 + i < t_end) x = tile_compute<T>(S, rt[i], rd[kDraft ? i : 0], w);
      const double part = (t0 + i < t_end) ? wave_sum_f64_dpp(static_cast<double>(x)) : 0.0;
      if (lane_id() == 0) s_red[i][wave_id()] = part;
      if constexpr (kKeep) {
#pragma unroll
        for (int e = 0; e < kSampleEPT; ++e) keep[i][e] = w[e];
        keepx[i] = x;
      }
    }
    __syncthreads();
    if (threadIdx.x < TPB && t0 + static_cast<int>(threadIdx.x) < t_end) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += s_red[threadIdx.x][w];
      publish(&P.tile_sum[static_cast<int64_t>(b) * P.ntiles + t0 + threadIdx.x], tag_nonneg_double(tot));
    }
    __syncthreads();  // s_red is reused by the next group
  }
}

// The end of a sequence's sampling, by each of its `total` sampling
// workgroups once its tile totals are published: the last to arrive at
// *cnt draws the token and returns the sequence's workspace (statistics
// pieces, gathered logits, tile totals, and with `small` its plan words)
// to zero, and the counters `cnt` and `also` (if any) to zero.
template <class T, bool kEnt, bool kSmall = false>
__device__ void sample_finish(const ChainParams& P, int b, const SeqPlan& pl, uint32_t* cnt, uint32_t total,
                              uint32_t* also, bool draw = true, uint32_t also_total = 0u) {
  __shared__ int s_flag;
  // Wave 0 reads the sequence's tile totals beside the arrival count, so
  // that the last to arrive starts its draw without another round trip
  // (a slot read as zero here is read again by locate_tile).
  uint64_t pre = 0ull;
  if (draw && pl.j >= 0 && P.ntiles <= kWave && wave_id() == 0)
    pre = peek(&P.tile_sum[static_cast<int64_t>(b) * P.ntiles + (lane_id() < P.ntiles ? lane_id() : 0)]);
  if (!arrive_and_check_last(cnt, total, &s_flag)) return;
  // Every workgroup of the sequence has read the statistics pieces and
  // published its totals: leave the sequence's workspace all zero, the
  // pieces and gathered logits at once (the draw reads neither), the tile
  // totals once the draw has read them.
  const int64_t per_seq = slots_per_seq(P.L);
  for (int64_t sl = static_cast<int64_t>(b) * per_seq + threadIdx.x; sl < (static_cast<int64_t>(b) + 1) * per_seq;
       sl += kThreads) {
    P.part_m[sl] = 0ull;
    P.part_s[sl] = 0ull;
    if constexpr (kEnt) P.part_a[sl] = 0ull;
  }
  const int R = 2 * P.K + 1;
  for (int r = threadIdx.x; r < R; r += kThreads) P.gat[static_cast<int64_t>(b) * R + r] = 0ull;
  if (draw && pl.j >= 0) chain_draw<T>(P, b, pl, pre);
  __syncthreads();
  if (kSmall || pl.j >= 0)  // (a small call's last workgroup may not have read the plan)
    for (int t = threadIdx.x; t < P.ntiles; t += kThreads) clear_slot(&P.tile_sum[static_cast<int64_t>(b) * P.ntiles + t]);
  if constexpr (kSmall)
    for (int w = threadIdx.x; w < kPlanWords; w += kThreads) clear_slot(&P.plan[static_cast<int64_t>(b) * kPlanStride + w]);
  reset_counter(cnt);
  if (also != nullptr) {
    // every count into `also` is issued by a running workgroup whose slots
    // were all read: wait for the last ones to land before the reset
    // (bounded; on expiry the reset is skipped and SV_ERRF_INTERNAL raised)
    if (threadIdx.x == 0 && also_total > 0u) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(also, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < also_total) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
          raise_error(P.err_flags, kErrInternal);
          publish(P.abort, 1ull);
          return;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    reset_counter(also);
  }
}

// Sampling workgroup g of sequence b: its wave 0 makes the sequence's
// decision (group 0 writes it out), then the workgroup forms the weights of
// tiles [g * tiles_per_block, (g + 1) * tiles_per_block) of the sampling row
// pair, TPB at a time, and publishes their totals; the last workgroup of the
// sequence to finish draws the token and returns the sequence's workspace
// (statistics pieces, gathered logits, tile totals, arrival counter) to zero.
// kLive: the one-launch call (statistics of the same launch, see
// decide_live); a decision that never completes reports the sequence as an
// invalid row with SV_ERRF_INTERNAL.
template <class T, int TPB, bool kDraft, bool kEnt, bool kLive = false>
__device__ void sample_seq(const ChainParams& P, int b, int blk) {
  __shared__ SeqPlan s_plan;
  if (wave_id() == 0) {
    if constexpr (kLive) {
      if (!decide_live<T, kEnt>(P, b, &s_plan, blk == 0) && lane_id() == 0) {
        if (blk == 0) {
          P.accept_len[b] = -1;
          for (int i = 0; i <= P.K; ++i) P.out_tokens[static_cast<int64_t>(b) * (P.K + 1) + i] = -1;
          if (P.residual_mass != nullptr) P.residual_mass[b] = -1.0f;
          if (kEnt)
            for (int r = 0; r <= 2 * P.K; ++r) P.entropy[static_cast<int64_t>(b) * (2 * P.K + 1) + r] = NAN;
        }
        raise_error(P.err_flags, kErrInternal);
        s_plan.j = -1;
      }
    } else {
      decide_wave<T, kEnt>(P, b, &s_plan, blk == 0);
    }
  }
  __syncthreads();
  if (kLive && SV_TAIL_PRIO > 0 && (SV_TAIL_PRIO_ALL || b >= P.B - SV_LATE_PRIO_SEQS))
    __builtin_amdgcn_s_setprio(SV_TAIL_PRIO);
  const SeqPlan pl = s_plan;
  if (pl.j >= 0) {  // an invalid row has nothing to draw: its outputs are -1
    const int t_begin = blk * P.tiles_per_block;
    tile_totals<T, TPB, kDraft>(P, b, pl, t_begin, min(t_begin + P.tiles_per_block, P.ntiles));
  }
  uint32_t* cnt = P.cnt + static_cast<int64_t>(b) * (kLive ? kCtrStride : 1);
  sample_finish<T, kEnt>(P, b, pl, cnt, static_cast<uint32_t>(P.nblk_b),
                         kLive ? P.done + static_cast<int64_t>(b) * kCtrStride : nullptr, true,
                         kLive ? static_cast<uint32_t>(P.L.cps) : 0u);
}

// ---------------------------------------------------------------- small calls

// The plan of sequence b as tagged words (never zero once written).
__device__ __forceinline__ void publish_plan(const ChainParams& P, int b, const SeqPlan& pl) {
  uint64_t* w = P.plan + static_cast<int64_t>(b) * kPlanStride;
  publish(&w[1], tag_float(pl.c_hi));
  publish(&w[2], tag_float(pl.c_lo));
  publish(&w[3], tag_float(pl.lt_hi));
  publish(&w[4], tag_float(pl.lt_lo));
  publish(&w[5], tag_float(pl.d_hi));
  publish(&w[6], tag_float(pl.d_lo));
  publish(&w[0], (1ull << 63) | static_cast<uint64_t>(static_cast<uint32_t>(pl.j + 1)));
}

// Read sequence b's plan (wave 0, one round of loads); false while a word
// is not visible yet.
__device__ __forceinline__ bool read_plan(const ChainParams& P, int b, SeqPlan* s_plan) {
  const uint64_t* w = P.plan + static_cast<int64_t>(b) * kPlanStride;
  const int lane = lane_id();
  const uint64_t v = peek(&w[lane < 7 ? lane : 0]);
  if (__ballot(v == 0ull) != 0ull) return false;
  const uint64_t w0 = __shfl(v, 0, kWave);
  if (lane == 0) {
    s_plan->j = static_cast<int32_t>(static_cast<uint32_t>(w0)) - 1;
    s_plan->pad = 0u;
  }
  const float f = untag_float(v);
  switch (lane) {
    case 1: s_plan->c_hi = f; break;
    case 2: s_plan->c_lo = f; break;
    case 3: s_plan->lt_hi = f; break;
    case 4: s_plan->lt_lo = f; break;
    case 5: s_plan->d_hi = f; break;
    case 6: s_plan->d_lo = f; break;
    default: break;
  }
  return true;
}

// Wave 0 of the decider: the decision from the published statistics (read
// again while a slot is not visible yet), written out, and the plan
// published for the sequence's other workgroups. Every slot it reads was
// stored by a workgroup that counted its chunk after its stores completed,
// so the loop ends; bounded like await_slot all the same. On expiry the
// sequence is reported as an invalid row (plan j = -1, SV_ERRF_INTERNAL).
template <class T, bool kPublish = true>
__device__ void small_decide(const ChainParams& P, int b, SeqPlan* s_plan) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const DecideIn in = decide_inputs(P, b);
  bool ok = true;
  while (!decide_live_wave<T>(P, b, s_plan, true, in)) {
    if (peek(P.abort) != 0ull || __builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      if (peek(P.abort) == 0ull) publish(P.abort, 1ull);
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ok && lane_id() == 0) {
    P.accept_len[b] = -1;
    for (int i = 0; i <= P.K; ++i) P.out_tokens[static_cast<int64_t>(b) * (P.K + 1) + i] = -1;
    if (P.residual_mass != nullptr) P.residual_mass[b] = -1.0f;
    raise_error(P.err_flags, kErrInternal);
    s_plan->j = -1;
  }
  if (kPublish && lane_id() == 0) publish_plan(P, b, *s_plan);
}

// Wave 0 of any other workgroup: wait for the decider's plan. The decider
// counted its chunk after every other chunk of the sequence, so it is
// running and waits for nothing but visible stores: the wait ends (bounded
// all the same; on expiry the sequence draws nothing here, SV_ERRF_INTERNAL).
__device__ void small_await_plan(const ChainParams& P, int b, SeqPlan* s_plan) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (!read_plan(P, b, s_plan)) {
    if (peek(P.abort) != 0ull || __builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      if (peek(P.abort) == 0ull) publish(P.abort, 1ull);
      if (lane_id() == 0) {
        raise_error(P.err_flags, kErrInternal);
        s_plan->j = -1;
      }
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The small call's draw, by every workgroup that holds tiles (their
// weights in keep, tiles [t_begin, t_end)) once it has published their
// totals: wave 0 reads every tile total of the sequence (they come from
// workgroups that have all started, since each counted its chunk before the
// plan existed, and that wait for nothing more) and finds the tile holding
// the target, as chain_draw does; the workgroup that holds that tile draws
// from its weights, with chain_draw's operations, so the same token. A
// residual that vanished in fp32, or no tile with weight, leaves the draw
// to the workgroup holding tile 0, which runs chain_draw itself.
template <class T, int TPB>
__device__ __forceinline__ void small_owner_draw(const ChainParams& P, int b, const SeqPlan& pl, int t_begin, int t_end,
                                 const float (&keep)[TPB][kSampleEPT], const float (&keepx)[TPB]) {
  __shared__ double s_scan[kWaves];
  __shared__ int s_redi[2 * kWaves];
  __shared__ double s_S, s_target;
  __shared__ int s_tile;
  __shared__ uint32_t s_err;
  if (threadIdx.x == 0) s_err = 0u;
  __syncthreads();
  locate_tile(P, b, &s_S, &s_tile, &s_target, &s_err);
  __syncthreads();
  const double S_res = s_S;
  const int tile = s_tile;
  if ((!(S_res > 0.0) && pl.j < P.K) || tile < 0) {
    if (t_begin == 0) chain_draw<T>(P, b, pl);
    return;
  }
  if (tile < t_begin || tile >= t_end) return;
  float w[kSampleEPT];
  float x = 0.0f;
#pragma unroll
  for (int i = 0; i < TPB; ++i) {
    if (t_begin + i == tile) {
#pragma unroll
      for (int e = 0; e < kSampleEPT; ++e) w[e] = keep[i][e];
      x = keepx[i];
    }
  }
  const int token = draw_in_weights(tile, w, x, s_target, s_scan, s_redi);
  if (threadIdx.x == 0) {
    P.out_tokens[static_cast<int64_t>(b) * (P.K + 1) + pl.j] = token;
    if (P.residual_mass != nullptr) P.residual_mass[b] = (pl.j < P.K) ? static_cast<float>(S_res) : -1.0f;
    raise_error(P.err_flags, s_err);
  }
}

}  // namespace

// Pass 1, chunked layout: one workgroup per chunk.
template <class T, bool kEnt>
__device__ __forceinline__ void stats_chunk_item(const ChainParams& P) {
  // blockIdx.x and the chunks per sequence fit 32 bits (checked on the host)
  const uint32_t cps = static_cast<uint32_t>(P.L.cps);
  const uint32_t b = blockIdx.x / cps;
  stats_chunk<T, kStatsTPB, kEnt>(P, static_cast<int>(b), static_cast<int>(blockIdx.x - b * cps));
}

template <class T>
__global__ __launch_bounds__(kStatsTPB) __attribute__((amdgpu_waves_per_eu(SV_STATS_WAVES, SV_STATS_WAVES))) void chain_stats_chunk_kernel(ChainParams P) {
  stats_chunk_item<T, false>(P);
}

// The same pass with the entropy of every row requested (one more
// accumulator per thread), compiled for its own occupancy.
template <class T>
__global__ __launch_bounds__(kStatsTPB) __attribute__((amdgpu_waves_per_eu(SV_STATS_WAVES_ENT, SV_STATS_WAVES_ENT))) void chain_stats_chunk_entropy_kernel(ChainParams P) {
  stats_chunk_item<T, true>(P);
}

// Pass 1, segments layout: one workgroup per row segment.
template <class T, bool kEnt>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void chain_stats_segment_kernel(ChainParams P) {
  const uint32_t per_seq = static_cast<uint32_t>(items_per_seq(P.L));
  const int b = static_cast<int>(blockIdx.x / per_seq);
  const int rem = static_cast<int>(blockIdx.x - static_cast<uint32_t>(b) * per_seq);
  stats_segment<T, kEnt>(P, b, rem / P.L.nseg, rem % P.L.nseg);
}

// Pass 2: nblk_b workgroups per sequence, assigned round-robin over the
// sequences: workgroups are dispatched in index order over a few
// microseconds, so every sequence's first workgroup (its decider, usually)
// starts among the first B.
// kEnt: the statistics pass also published A per piece (entropy requested).
template <class T, bool kEnt>
__global__ __launch_bounds__(kThreads) void chain_sample_kernel(ChainParams P) {
  const uint32_t B = static_cast<uint32_t>(P.B);
  sample_seq<T, SampleTiles<T>::kPerBlock, true, kEnt>(P, static_cast<int>(blockIdx.x % B),
                                                       static_cast<int>(blockIdx.x / B));
}

// K = 0 (draft-side sampling): one row per draw, more tiles per workgroup.
template <class T, bool kEnt>
__global__ __launch_bounds__(kThreads) void chain_sample_one_row_kernel(ChainParams P) {
  const uint32_t B = static_cast<uint32_t>(P.B);
  sample_seq<T, SampleTiles<T>::kPerBlock * kSampleTilesK0Factor, false, kEnt>(P, static_cast<int>(blockIdx.x % B),
                                                                                static_cast<int>(blockIdx.x / B));
}

// The sequence whose ticket queue block `blk` of the one-launch grid serves.
// Grid order: the statistics blocks of sequences 0 .. lag-1 (cps each); then
// for s = lag .. B-1 the statistics blocks of s followed by the sampling
// blocks of s - lag (nblk each); then the sampling blocks of the last lag
// sequences. Every sequence owns cps + nblk blocks.
__device__ __forceinline__ uint32_t one_launch_sequence(uint32_t blk, uint32_t B, uint32_t cps, uint32_t nblk) {
  const uint32_t lag = min(static_cast<uint32_t>(kSampleLag), B);
  if (blk < lag * cps) return blk / cps;
  const uint32_t i = blk - lag * cps;
  const uint32_t seg = cps + nblk;
  const uint32_t nmid = B - lag;
  if (i < nmid * seg) {
    const uint32_t s = lag + i / seg;
    return (i % seg < cps) ? s : s - lag;
  }
  return nmid + (i - nmid * seg) / nblk;
}

// One-launch call (rows on 16-byte boundaries, K >= 1): the
// statistics chunks and the sampling workgroups of every sequence in one
// grid, so that the sampling of the sequences streamed first overlaps the
// streaming of the later ones instead of waiting for the whole pass.
//
// Roles come from one ticket queue per sequence. Sequence b owns cps
// statistics blocks (blocks b cps .. b cps + cps - 1) and nblk_b sampling
// blocks (after every sequence's statistics blocks); a workgroup of b's
// blocks takes the next ticket of b's queue when it starts. Tickets
// 0 .. cps-1 stream b's chunks, tickets cps .. cps+nblk_b-1 sample b. A
// sampling role therefore waits only for chunks whose tickets were taken
// earlier, by workgroups that are running and wait for nothing: every wait
// ends, whatever order the hardware dispatches workgroups in and whatever
// else runs beside the launch. With the usual in-order dispatch the block
// order (statistics first, sequence by sequence) starts the sampling of the
// first sequences while the last ones stream. The workgroup that takes the
// last ticket of a queue returns its counter to zero; a statistics role
// counts its chunk in P.done[b] once its slot stores have completed.
template <class T, bool kEnt>
__device__ __forceinline__ void one_launch_item(const ChainParams& P) {
  __shared__ uint32_t s_ticket;
  const uint32_t cps = static_cast<uint32_t>(P.L.cps);
  const uint32_t nblk = static_cast<uint32_t>(P.nblk_b);
  const uint32_t b = one_launch_sequence(blockIdx.x, static_cast<uint32_t>(P.B), cps, nblk);
  if (threadIdx.x == 0) {
    uint32_t* tk = P.tk + static_cast<int64_t>(b) * kCtrStride;
    const uint32_t t = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t + 1u == cps + nblk) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ticket = t;
  }
  __syncthreads();
  const uint32_t t = s_ticket;
  if (t >= cps + nblk) {  // a ticket counter not left at zero: the workspace was not re-zeroed
    if (threadIdx.x == 0) {
      raise_error(P.err_flags, kErrInternal);
      publish(P.abort, 1ull);
    }
    return;
  }
  if (t < cps) {
    stats_chunk<T, kStatsTPB, kEnt>(P, static_cast<int>(b), static_cast<int>(t));
    if (threadIdx.x == 0) {
      // count the chunk; its slot stores may still be on their way (the
      // readers check every slot's tag and read again while one is zero)
      if (SV_COUNT_WAIT) __builtin_amdgcn_s_waitcnt(0);
      __hip_atomic_fetch_add(P.done + static_cast<int64_t>(b) * kCtrStride, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    if (SV_SAMPLE_PRIO > 0) __builtin_amdgcn_s_setprio(SV_SAMPLE_PRIO);  // (not used: 0)
    sample_seq<T, live_tiles<T>(), true, kEnt, true>(P, static_cast<int>(b), static_cast<int>(t - cps));
  }
}

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SV_ONE_LAUNCH_WAVES, SV_ONE_LAUNCH_WAVES))) void chain_one_launch_kernel(ChainParams P) {
  one_launch_item<T, false>(P);
}

// The same call with the entropy of every row requested: the statistics
// roles also publish A per piece, the deciding workgroup writes the entropy.
template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SV_ONE_LAUNCH_WAVES, SV_ONE_LAUNCH_WAVES))) void chain_one_launch_entropy_kernel(ChainParams P) {
  one_launch_item<T, true>(P);
}

// Small call (at most a few hundred rows in all, the grid resident at once):
// one launch of B cps workgroups, one per statistics chunk, which also
// decide and sample. Workgroup (b, ch) streams chunk ch of sequence b and
// counts it in done[b] once its slot stores have completed. The last of
// b's chunks to be counted makes b's decision (wave 0, writing the outputs
// it fixes) and publishes the plan; the other workgroups of b wait for the
// plan. Every workgroup then forms the weights of its share of the
// sampling row pair's tiles and publishes their totals, and the last of b's
// workgroups to arrive draws the token and clears b's workspace.
//
// Why the waits end in any dispatch order, whatever else runs: a workgroup
// waits only for the plan of its own sequence, which comes from the
// workgroup that counted the last chunk; that workgroup has started, and its
// decision reads only slots stored by workgroups that counted their chunks
// after their stores completed. No workgroup waits for one that has not
// started. The waits are bounded all the same (await_slot's limit).
template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((flatten)) void chain_small_kernel(ChainParams P) {
  static_assert(kStatsTPB == kThreads, "the statistics chunk runs on the whole workgroup");
  __shared__ SeqPlan s_plan;
  __shared__ int s_last;
  const uint32_t cps = static_cast<uint32_t>(P.L.cps);
  const uint32_t bu = blockIdx.x / cps;
  const int b = static_cast<int>(bu);
  const int ch = static_cast<int>(blockIdx.x - bu * cps);
  if (!stats_chunk_prefetched<T, kStatsTPB, kSmallMaxBatches>(P, b, ch)) stats_chunk<T, kStatsTPB, false>(P, b, ch);
  uint32_t* done = P.done + static_cast<int64_t>(b) * kCtrStride;
  __shared__ int s_seen;
  if (wave_id() == 0) {
    if (SV_SMALL_PRIO > 0) __builtin_amdgcn_s_setprio(SV_SMALL_PRIO);
    uint32_t prev = 0u;
    if (threadIdx.x == 0) {
      // count the chunk (with SV_SMALL_COUNT_WAIT once this thread's slot
      // stores have completed; the decider checks every slot's tag and
      // reads again while one is zero)
      if (SV_SMALL_COUNT_WAIT) __builtin_amdgcn_s_waitcnt(0);
      prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Beside the count, every workgroup reads the sequence's slots once and
    // decides if all are visible (the same decision, and the same outputs,
    // as the one the last to count makes): the last one then usually has
    // its plan one round trip sooner, and others need not wait for it.
    const DecideIn in = decide_inputs(P, b);
    const bool seen = SV_SMALL_SPEC ? decide_live_wave<T>(P, b, &s_plan, true, in) : false;
    if (lane_id() == 0) {
      s_last = (prev + 1u == cps) ? 1 : 0;
      s_seen = seen ? 1 : 0;
      if (prev >= cps) {  // a counter not left at zero: the workspace was not re-zeroed
        raise_error(P.err_flags, kErrInternal);
        publish(P.abort, 1ull);
      }
    }
  }
  __syncthreads();
  // the draw by the workgroup holding the target's tile when every
  // workgroup's tiles fit one group, else by the last to arrive (which
  // then needs the plan); a workgroup without tiles otherwise does not
  const bool owners = P.tiles_per_block <= kSmallTiles;
  const int t_begin = ch * P.tiles_per_block;
  const int t_end = min(t_begin + P.tiles_per_block, P.ntiles);
  if (wave_id() == 0) {
    if (SV_SMALL_POLL_SLOTS) {
      // Every workgroup that needs the plan reads the slots again until all
      // are visible and decides itself: no hand-off of the plan. Every slot
      // comes from a workgroup of this grid, which the device holds at once
      // (checked on the host), so each is written: the wait ends (bounded
      // as small_decide's).
      if (s_seen) {
        // decided from the first read
      } else if (s_last || !owners || t_begin < t_end) {
        small_decide<T, false>(P, b, &s_plan);
      } else if (lane_id() == 0) {
        s_plan.j = -1;
      }
    } else if (s_last) {
      if (s_seen) {
        if (lane_id() == 0) publish_plan(P, b, s_plan);
      } else {
        small_decide<T>(P, b, &s_plan);
      }
    } else if (s_seen) {
      // the plan is already here
    } else if (!owners || t_begin < t_end) {
      small_await_plan(P, b, &s_plan);
    } else if (lane_id() == 0) {
      s_plan.j = -1;
    }
  }
  __syncthreads();
  const SeqPlan pl = s_plan;
  if (pl.j >= 0) {
    if (owners) {
      float keep[kSmallTiles][kSampleEPT];
      float keepx[kSmallTiles];
      tile_totals<T, kSmallTiles, true, true>(P, b, pl, t_begin, t_end, keep, keepx);
      if (t_begin < t_end) small_owner_draw<T, kSmallTiles>(P, b, pl, t_begin, t_end, keep, keepx);
    } else {
      tile_totals<T, live_tiles<T>(), true>(P, b, pl, t_begin, t_end);
    }
  }
  sample_finish<T, false, true>(P, b, pl, P.cnt + static_cast<int64_t>(b) * kCtrStride, cps, done, !owners);
}

// ---------------------------------------------------------------- launcher

template <class T>
static hipError_t launch_chain_t(const ChainParams& p, const PassEvents& ev, hipStream_t stream) {
  const int64_t grid_a = static_cast<int64_t>(p.B) * items_per_seq(p.L);
  const int64_t grid_c = static_cast<int64_t>(p.B) * p.nblk_b;
  if (grid_a > INT32_MAX || grid_c > INT32_MAX) return hipErrorInvalidConfiguration;
  // Armed events take the statistics kernel's own start and end timestamps
  // (the whole call's, for the one-launch kernel).
  const bool ent = p.entropy != nullptr;
  if (p.one_launch == 2) {
    const int64_t grid = static_cast<int64_t>(p.B) * p.L.cps;
    if (grid > INT32_MAX || p.plan == nullptr) return hipErrorInvalidConfiguration;
    launch_stream_pass(chain_small_kernel<T>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), stream, ev, p);
    return hipGetLastError();
  }
  if (p.one_launch) {
    const int64_t grid = static_cast<int64_t>(p.B) * (p.L.cps + p.nblk_b);
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    launch_stream_pass(ent ? chain_one_launch_entropy_kernel<T> : chain_one_launch_kernel<T>,
                       dim3(static_cast<uint32_t>(grid)), dim3(kThreads), stream, ev, p);
    return hipGetLastError();
  }
  if (p.L.cps > 0)
    launch_stream_pass(ent ? chain_stats_chunk_entropy_kernel<T> : chain_stats_chunk_kernel<T>,
                       dim3(static_cast<uint32_t>(grid_a)), dim3(kStatsTPB), stream, ev, p);
  else
    launch_stream_pass(ent ? chain_stats_segment_kernel<T, true> : chain_stats_segment_kernel<T, false>,
                       dim3(static_cast<uint32_t>(grid_a)), dim3(kThreads), stream, ev, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void (*sample)(ChainParams);
  if (p.K == 0)
    sample = ent ? chain_sample_one_row_kernel<T, true> : chain_sample_one_row_kernel<T, false>;
  else
    sample = ent ? chain_sample_kernel<T, true> : chain_sample_kernel<T, false>;
  hipLaunchKernelGGL(sample, dim3(static_cast<uint32_t>(grid_c)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- LM-head chain call

// After the LM-head GEMM: blocks below B K stream one draft row each (the
// statistics pass over the whole-row layout: rows K+1 .. 2K of each
// sequence); the others combine the GEMM's pieces of the target rows, one
// wave per row. A row's pieces are folded in fp64 like the decision folds a
// row's pieces (a running fp32 reference, sums rescaled by 2^(lower -
// higher reference)), each lane over every 64th piece, then across the wave;
// the row's (reference, sum) goes to its slot and, for a drafted position,
// the stored logit at the drafted token to its gather slot. The pieces are
// left zero (the workspace contract).
template <class T>
__global__ __launch_bounds__(kThreads) void lm_head_stats_kernel(ChainParams P) {
  const uint32_t K = static_cast<uint32_t>(P.K);
  const uint32_t ndraft = static_cast<uint32_t>(P.B) * K;
  if (blockIdx.x < ndraft) {
    const uint32_t b = blockIdx.x / K;
    stats_chunk<T, kStatsTPB, false>(P, static_cast<int>(b), static_cast<int>(K + 1 + (blockIdx.x - b * K)));
    return;
  }
  const int64_t M = static_cast<int64_t>(P.B) * (K + 1);
  const int64_t m = static_cast<int64_t>(blockIdx.x - ndraft) * kWaves + wave_id();
  if (m >= M) return;
  const int lane = lane_id();
  float2* pc = P.lm_pieces + m * P.lm_ntn;
  float mf = -INFINITY;
  double zf = 0.0;
  for (int i = lane; i < P.lm_ntn; i += kWave) {
    const float2 v = pc[i];
    pc[i] = make_float2(0.0f, 0.0f);
    if (v.x == -INFINITY) continue;
    const double sv = static_cast<double>(v.y);
    if (v.x > mf) {
      zf = zf * ((mf == -INFINITY) ? 0.0 : ref_factor(mf, v.x)) + sv;
      mf = v.x;
    } else {
      zf += sv * ref_factor(v.x, mf);
    }
  }
  const float Mx = wave_max(mf);
  double z = (mf == -INFINITY) ? 0.0 : zf * ref_factor(mf, Mx);
  z = wave_sum(z);
  if (lane == 0) {
    const int b = static_cast<int>(m / (K + 1));
    const int r = static_cast<int>(m - static_cast<int64_t>(b) * (K + 1));  // target row r of sequence b
    const int64_t slot = (static_cast<int64_t>(b) * P.L.cps + r) * P.L.kmax;
    publish(&P.part_m[slot], tag_float(Mx));
    publish(&P.part_s[slot], tag_nonneg_double(z));
    const int x = row_token(P, b, r);
    if (x >= 0 && x < P.V) publish_gather<T>(P, b, r, chain_row<T>(P, b, r), x);
  }
}

hipError_t launch_chain_lm_head(const LMHeadParams& g, const ChainParams& p, const PassEvents& ev,
                                hipStream_t stream) {
  hipError_t e = launch_lm_head_gemm(g, true, ev, stream);
  if (e != hipSuccess) return e;
  const int64_t M = static_cast<int64_t>(p.B) * (p.K + 1);
  const int64_t grid_s = static_cast<int64_t>(p.B) * p.K + (M + kWaves - 1) / kWaves;
  const int64_t grid_c = static_cast<int64_t>(p.B) * p.nblk_b;
  if (grid_s > INT32_MAX || grid_c > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(lm_head_stats_kernel<BF16>, dim3(static_cast<uint32_t>(grid_s)), dim3(kThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  void (*sample)(ChainParams) = p.K == 0 ? chain_sample_one_row_kernel<BF16, false> : chain_sample_kernel<BF16, false>;
  hipLaunchKernelGGL(sample, dim3(static_cast<uint32_t>(grid_c)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chain(const ChainParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream) {
  return dtype == SV_DTYPE_BF16 ? launch_chain_t<BF16>(p, ev, stream) : launch_chain_t<F32>(p, ev, stream);
}

}  // namespace sv
