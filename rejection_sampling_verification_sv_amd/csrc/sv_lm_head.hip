// The target's LM head as a bf16 MFMA GEMM, with the verification statistics
// of every row taken in its epilogue.
//
// [Topologies] "Speculative Decoding & Draft Model Topologies", section 2
// timeline figure, step 2: the target scores every drafted position in one
// forward pass; [Draft-and-Verify] "Speculative Decoding for LLM Inference",
// "Why autoregressive decoding is slow": that pass is bound by streaming the
// model's weights. Its last layer maps each position's final hidden state to
// one logit per vocabulary entry,
//   logits[m, v] = sum_h hidden[m, h] * weight[v, h],
// and verification then needs, per row, the log-normaliser of the
// temperature softmax. lm_head_gemm_kernel computes the logits with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation), stores them rounded to bf16
// (kept for the residual or bonus draw, and returned to the caller), and,
// with kStats, reduces every 128-column piece of each row of its tile to
// the pair the verification's combine reads: the fp32 reference
// fl(max * c_hi) and the fp32 sum of 2^(x c - reference) over the stored
// (rounded) values x, c = log2(e) / T of the row's sequence. The logits are
// therefore never read back for the statistics.
//
// Tiling: one 256-thread workgroup per 128 x 128 output tile, four waves of
// 64 x 64 (2 x 2 blocks of 32 x 32 accumulators), k-steps of 64 through
// double-buffered LDS (rows padded by 16 bytes, so the 32 rows a
// ds_read_b128 touches start on different bank groups). Both operands are
// k-contiguous in memory (hidden [M, H], weight [V, H]), as the MFMA
// operands are per lane. Block order: the M tiles of one N tile are
// consecutive blocks of one XCD (blocks are dealt to the eight XCDs in
// turn), so the weight tile comes from HBM once and from that XCD's L2 for
// the other M tiles.
#include <hip/hip_runtime.h>
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

constexpr int kGM = 128;              // output rows per tile
constexpr int kGN = 128;              // output columns per tile
constexpr int kGK = 64;               // k per step
constexpr int kLdsRow = kGK + 8;      // bf16 per LDS operand row (16 bytes of padding)
constexpr int kStageRow = kGN + 8;    // bf16 per staging row of the output tile
constexpr int kXcds = 8;              // XCDs the blocks of a launch are dealt to in turn

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs: the
// accumulators of finite bf16 products).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <bool kStats>
__global__ __launch_bounds__(256, 2) void lm_head_gemm_kernel(LMHeadParams P) {
  // two operand buffers of A and B; the output tile is staged in the A buffers
  __shared__ __align__(16) uint16_t smem[2 * (kGM + kGN) * kLdsRow];
  static_assert(kGM * kStageRow <= 2 * kGM * kLdsRow, "staging fits the A buffers");
  // operand buffer `buf` of A at smem + buf * kGM * kLdsRow, of B after both A buffers
  auto sA = [&](int buf) { return smem + buf * (kGM * kLdsRow); };
  auto sB = [&](int buf) { return smem + 2 * kGM * kLdsRow + buf * (kGN * kLdsRow); };

  const uint32_t mt = static_cast<uint32_t>(P.mtiles);
  const uint32_t xcd = blockIdx.x % kXcds;
  const uint32_t j = blockIdx.x / kXcds;
  const uint32_t n_tile = (j / mt) * kXcds + xcd;
  if (n_tile >= static_cast<uint32_t>(P.ntiles_n)) return;  // padding block of the last round
  const int m0 = static_cast<int>(j % mt) * kGM;
  const int n0 = static_cast<int>(n_tile) * kGN;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t H = P.H;
  const uint16_t* A = static_cast<const uint16_t*>(P.hidden);
  const uint16_t* W = static_cast<const uint16_t*>(P.weight);

  // this thread's four 16-byte pieces of each operand tile per k-step:
  // row idx >> 3, k offset (idx & 7) * 8, idx = tid + 256 q. Rows past M
  // (past N) read the last row instead: the loads stay unconditional 16-byte
  // loads, and what those rows produce is neither stored nor counted.
  const uint16_t* ga[4];
  const uint16_t* gb[4];
  int lds_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + 256 * q;
    const int row = idx >> 3, ch = idx & 7;
    ga[q] = A + static_cast<int64_t>(min(m0 + row, P.M - 1)) * H + ch * 8;
    gb[q] = W + static_cast<int64_t>(min(n0 + row, P.N - 1)) * H + ch * 8;
    lds_off[q] = row * kLdsRow + ch * 8;
  }
  uint4 ra[4], rb[4];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = load16(ga[q] + k0);
      rb[q] = load16(gb[q] + k0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<uint4*>(sA(buf) + lds_off[q]) = ra[q];
      *reinterpret_cast<uint4*>(sB(buf) + lds_off[q]) = rb[q];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.0f;

  // lane's operand rows within the wave tile, and its k half of each k16 step
  const int a_row = wm * 64 + (lane & 31);
  const int b_row = wn * 64 + (lane & 31);
  const int k_half = (lane >> 5) * 8;

  const int nk = static_cast<int>(H / kGK);
  fetch(0);
  stash(0);
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch(static_cast<int64_t>(kt + 1) * kGK);
#pragma unroll
    for (int kk = 0; kk < kGK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) a[bi] = as_bf16x8(load16(sA(buf) + (a_row + bi * 32) * kLdsRow + kk * 16 + k_half));
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) b[bj] = as_bf16x8(load16(sB(buf) + (b_row + bj * 32) * kLdsRow + kk * 16 + k_half));
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
    }
    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: round to bf16 and stage the tile in LDS (row-major, padded
  // rows): lane holds column (lane & 31) of each 32 x 32 block and rows
  // (r / 4) * 8 + (lane / 32) * 4 + r % 4 of it.
  uint16_t* stage = smem;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + bi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * 64 + bj * 32 + (lane & 31);
        stage[row * kStageRow + col] = static_cast<uint16_t>(bf16_bits_rne(acc[bi][bj][r]));
      }
  __syncthreads();

  // Coalesced stores of the tile: 16 threads per row of 128 bf16 (N is a
  // multiple of 8, so a 16-byte piece is either whole or past the end).
  uint16_t* C = static_cast<uint16_t*>(P.logits);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int idx = tid + 256 * q;
    const int row = idx >> 4, ch = idx & 15;
    const int n = n0 + ch * 8;
    if (m0 + row < P.M && n < P.N)
      *reinterpret_cast<uint4*>(C + static_cast<int64_t>(m0 + row) * P.N + n) = load16(stage + row * kStageRow + ch * 8);
  }

  if constexpr (kStats) {
    // Two threads per row: the row's reference over the 128 stored values
    // (columns past N excluded), then the sum of 2^(x c - reference).
    const int row = tid >> 1, half = tid & 1;
    const int m = m0 + row;
    float x[64];
    const uint16_t* src = stage + row * kStageRow + half * 64;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint4 w = load16(src + v * 8);
      unpack<BF16>(w, &x[v * 8]);
    }
    const int nvalid = min(64, max(0, P.N - (n0 + half * 64)));
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (i >= nvalid) x[i] = -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
    const Scale c = exponent_scale(m < P.M ? temperature_of(P.temperature, m / P.K1) : 1.0f);
    const float neg_m = neg_reference(mx, c);
    float acc8[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = fast_exp2(scaled_arg(x[g * 8 + i], c, neg_m));
      acc8[g] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    }
    float s = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
    s += __shfl_xor(s, 1, kWave);
    if (half == 0 && m < P.M) {
      const float ref = (mx == -INFINITY) ? -INFINITY : mx * c.hi;
      P.pieces[static_cast<int64_t>(m) * P.ntiles_n + n_tile] = make_float2(ref, s);
    }
  }
}

}  // namespace

int64_t lm_head_grid(const LMHeadParams& p) {
  const int64_t rounds = (static_cast<int64_t>(p.ntiles_n) + kXcds - 1) / kXcds;
  return rounds * kXcds * p.mtiles;
}

hipError_t launch_lm_head_gemm(const LMHeadParams& p, bool stats, const PassEvents& ev, hipStream_t stream) {
  const int64_t grid = lm_head_grid(p);
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  // every buffer the kernel writes or reads must be there
  if (p.hidden == nullptr || p.weight == nullptr || p.logits == nullptr || (stats && p.pieces == nullptr))
    return hipErrorInvalidValue;
  if (stats)
    launch_stream_pass(lm_head_gemm_kernel<true>, dim3(static_cast<uint32_t>(grid)), dim3(256), stream, ev, p);
  else
    launch_stream_pass(lm_head_gemm_kernel<false>, dim3(static_cast<uint32_t>(grid)), dim3(256), stream, ev, p);
  return hipGetLastError();
}

}  // namespace sv
