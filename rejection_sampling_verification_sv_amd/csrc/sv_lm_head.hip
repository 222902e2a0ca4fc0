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
// with kStats, reduces every 128-column piece of each row to the pair the
// verification's combine reads: the fp32 reference fl(max * c_hi) and the
// fp32 sum of 2^(x c - reference) over the stored (rounded) values x,
// c = log2(e) / T of the row's sequence. The logits are therefore never
// read back for the statistics.
//
// Tiling (kTM x kTN output tile per workgroup of kWM x kWN waves, one
// workgroup per CU): both operands are k-contiguous in memory (hidden
// [M, H], weight [V, H]), as the MFMA operands are per lane, so each
// pipeline stage holds kKS = 32 values of k for every row of the tile: 64
// bytes, four 16-byte chunks. The chunks go from memory straight into LDS
// (global_load_lds_dwordx4: lane i of a wave fills bytes 16 i.. of a
// wave-uniform base), kStages stages deep, so that several stages of loads
// are in flight while one is multiplied; waits count this wave's own loads
// (vmcnt) and a bare s_barrier publishes them, so no wait drains the loads
// of later stages. The barrier sits in the middle of a stage: the operand
// fragments of the next stage's first k16 step are read from LDS while the
// MFMAs of this stage's second step run, so the matrix pipe does not wait
// out the LDS latency at every stage. Chunk c of tile row r sits at
// position c ^ ((r >> 2) & 3) of its row, which measured free of bank
// conflicts for the MFMA operand reads (ds_read_b128 of rows r = 0..31,
// two chunks) on gfx950, where (r >> 1) & 3, r & 7 on 128-byte rows and
// (r >> 1 ^ r >> 3) & 3 conflict two ways. Block order: the M tiles of one
// N tile are consecutive blocks of one XCD (blocks are dealt to the eight
// XCDs in turn), so the weight tile comes from HBM once and from that
// XCD's L2 for the others.
#include <hip/hip_runtime.h>
#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"

#ifndef SV_LM_TM
#define SV_LM_TM 192  // output rows per workgroup tile
#endif
#ifndef SV_LM_TN
#define SV_LM_TN 256  // output columns per workgroup tile
#endif
#ifndef SV_LM_WM
#define SV_LM_WM 2  // waves along M
#endif
#ifndef SV_LM_WN
#define SV_LM_WN 2  // waves along N
#endif
#ifndef SV_LM_STAGES
#define SV_LM_STAGES 5  // pipeline stages of kKS values of k
#endif
#ifndef SV_LM_KS
#define SV_LM_KS 32  // values of k per pipeline stage (32: 64-byte row pieces, 64: whole 128-byte lines)
#endif
#ifndef SV_LM_EARLY
#define SV_LM_EARLY 0  // 1: the stage barrier at the start of a stage instead of before its last k16 step
#endif
#ifndef SV_LM_LOADERS
#define SV_LM_LOADERS (SV_LM_WM * SV_LM_WN)  // waves that issue the operand loads (the first ones)
#endif

namespace sv {

namespace {

constexpr int kTM = SV_LM_TM;
constexpr int kTN = SV_LM_TN;
constexpr int kWM = SV_LM_WM;
constexpr int kWN = SV_LM_WN;
constexpr int kStages = SV_LM_STAGES;
constexpr int kLoaders = SV_LM_LOADERS;
constexpr int kKS = SV_LM_KS;                     // k per stage
constexpr int kRowBytes = kKS * 2;                // bytes per operand row and stage
constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per operand row and stage
constexpr int kSub = kKS / 16;                    // k16 MFMA steps per stage
constexpr bool kEarly = SV_LM_EARLY != 0;
constexpr int kThreadsG = kWM * kWN * kWave;      // threads per workgroup
constexpr int kStageBytes = (kTM + kTN) * kRowBytes;
constexpr int kLoadThreads = kLoaders * kWave;   // threads of the loading waves
constexpr int kLoads = (kTM + kTN) * kChunks / kLoadThreads;  // 16-byte chunks per loading thread and stage
constexpr int kBI = kTM / kWM / 32;               // 32 x 32 accumulator blocks per wave along M
constexpr int kBJ = kTN / kWN / 32;               // ... along N
constexpr int kOutRow = kTN + 8;                  // bf16 per staged output row (16 bytes of padding)
// the output tile is staged in one band of rows, or in two when the whole
// tile does not fit in the operand stages' LDS
constexpr int kEpiPasses = kTM * kOutRow * 2 <= kStages * kStageBytes ? 1 : 2;
constexpr int kEpiRows = kTM / kEpiPasses;        // output rows staged at a time
constexpr int kLdsBytes =
    kStages * kStageBytes > kEpiRows * kOutRow * 2 ? kStages * kStageBytes : kEpiRows * kOutRow * 2;
constexpr int kXcds = 8;                          // XCDs the blocks of a launch are dealt to in turn

static_assert(kTM % (32 * kWM) == 0 && kTN % (32 * kWN) == 0, "whole 32 x 32 blocks per wave");
static_assert(kLoaders >= 1 && kLoaders <= kWM * kWN, "loading waves are waves of the workgroup");
static_assert(kKS == 32 || kKS == 64, "four or eight chunks per row and stage");
static_assert((kTM + kTN) * kChunks % kLoadThreads == 0, "every loading thread loads the same number of chunks");
static_assert(kTM * kChunks % kLoadThreads == 0, "a thread's chunk q is either hidden or weight for all q");
static_assert(kTN % kLMPiece == 0, "whole statistics pieces per tile");
static_assert(kStages >= (kEarly ? 3 : 4) && kLoads * (kStages - 2) <= 63, "vmcnt holds the loads of the later stages");
static_assert(kLdsBytes <= 160 * 1024, "fits the LDS of a CU");
static_assert(kWM % kEpiPasses == 0, "each epilogue band is the rows of whole waves");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs: the
// accumulators of finite bf16 products).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// LDS position of 16-byte chunk c (0..3) of tile row r
__device__ __forceinline__ int chunk_pos(int r, int c) {
  return kChunks == 4 ? c ^ ((r >> 2) & 3) : c ^ ((r >> 1) & 7);
}

// s_waitcnt vmcnt(n), the other counters left alone (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A workgroup barrier that waits for nothing itself (the callers' waitcnt
// decides which loads must have landed); the empty asm statements keep the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool kStats>
__global__ __launch_bounds__(kThreadsG, 1) void lm_head_gemm_kernel(LMHeadParams P) {
  __shared__ __align__(16) uint8_t smem[kLdsBytes];

  const uint32_t mt = static_cast<uint32_t>(P.mt);
  const uint32_t xcd = blockIdx.x % kXcds;
  const uint32_t j = blockIdx.x / kXcds;
  const uint32_t n_tile = (j / mt) * kXcds + xcd;
  if (n_tile >= static_cast<uint32_t>(P.nt)) return;  // padding block of the last round
  const int m0 = static_cast<int>(j % mt) * kTM;
  const int n0 = static_cast<int>(n_tile) * kTN;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int64_t H = P.H;
  const uint16_t* A = static_cast<const uint16_t*>(P.hidden);
  const uint16_t* W = static_cast<const uint16_t*>(P.weight);

  // This thread's chunk q of a stage (threads of the loading waves): tile
  // row idx / kChunks, LDS position idx % kChunks, idx = q * kLoadThreads + tid (rows
  // below kTM are hidden rows, the rest weight rows). Rows past M (past N)
  // read the last row: the loads stay in bounds and unconditional, and what
  // those rows produce is neither stored nor counted.
  const bool loader = wave < kLoaders;
  const uint16_t* src[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int idx = q * kLoadThreads + (loader ? tid : 0);
    const int r = idx / kChunks;
    if (q * kLoadThreads < kTM * kChunks) {  // the chunks of q are those of hidden rows
      src[q] = A + static_cast<int64_t>(min(m0 + r, P.M - 1)) * H + chunk_pos(r, idx % kChunks) * 8;
    } else {
      const int rb = r - kTM;
      src[q] = W + static_cast<int64_t>(min(n0 + rb, P.N - 1)) * H + chunk_pos(rb, idx % kChunks) * 8;
    }
  }
  // k-step kt into stage s (loading waves only): each wave instruction
  // fills 1 KB of LDS
  auto issue = [&](int kt, int s) {
    if (!loader) return;
    uint8_t* dst = smem + s * kStageBytes + wave * (kWave * 16);
    const int64_t k0 = static_cast<int64_t>(kt) * kKS;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[q] + k0),
                                       (lds_void*)(dst + q * (kLoadThreads * 16)), 16, 0, 0);
  };

  f32x16 acc[kBI][kBJ];
#pragma unroll
  for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
    for (int bj = 0; bj < kBJ; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.0f;

  // operand rows of this lane (row lane & 31 of each 32-row block of the
  // wave) and the byte offsets of its k chunk in the two k16 steps of a
  // stage (the wave's row bases are multiples of 32, so the position only
  // depends on lane & 31)
  const int arow = wm * (kTM / kWM) + (lane & 31);
  const int brow = kTM + wn * (kTN / kWN) + (lane & 31);
  int coff[kSub];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) coff[sub] = chunk_pos(lane & 31, 2 * sub + (lane >> 5)) * 16;

  const int nk = static_cast<int>(H / kKS);
  bf16x8 fa[2][kBI], fb[2][kBJ];  // operand fragments of two k16 steps
  // fragments of k16 step `sub` of stage s into buffer sub & 1
  auto read_frags = [&](int s, int sub) {
    const uint8_t* st = smem + s * kStageBytes;
    const int co = coff[sub];
    const int kk = sub & 1;
#pragma unroll
    for (int bi = 0; bi < kBI; ++bi)
      fa[kk][bi] = *reinterpret_cast<const bf16x8*>(st + (arow + bi * 32) * kRowBytes + co);
#pragma unroll
    for (int bj = 0; bj < kBJ; ++bj)
      fb[kk][bj] = *reinterpret_cast<const bf16x8*>(st + (brow + bj * 32) * kRowBytes + co);
  };
  auto mfmas = [&](int kk) {
#pragma unroll
    for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
      for (int bj = 0; bj < kBJ; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][bi], fb[kk][bj], acc[bi][bj], 0, 0, 0);
  };
  // the scheduler is to issue the LDS reads of the next k16 step right
  // after the first MFMA of this one (whose operands were read a step
  // earlier, so that its wait drains nothing new), and the rest of this
  // step's MFMAs while they are in flight (sched_group_barrier masks:
  // 0x008 MFMA, 0x100 LDS reads)
  auto reads_then_mfmas = [] {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kBI + kBJ, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kBI * kBJ - 1, 0);
  };
  // k16 steps 0 .. kSub - 2 of stage s (the fragments of step 0 read)
  auto steps_but_last = [&](int s) {
#pragma unroll
    for (int sub = 0; sub + 1 < kSub; ++sub) {
      read_frags(s, sub + 1);
      mfmas(sub & 1);
      reads_then_mfmas();
    }
  };

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) issue(s, s);
  int s_cur = 0;                // stage of k-step kt
  int s_new = kStages - 1;      // stage of k-step kt + kStages - 1 (that of step kt - 1)
  if constexpr (kEarly) {
    // barrier at the start of each stage: the loads of step kt + kStages - 1
    // go out once every wave is done with step kt - 1
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + kStages - 2 < nk)
        wait_vmcnt<kLoads * (kStages - 2)>();
      else
        wait_vmcnt<0>();
      bare_barrier();
      if (kt + kStages - 1 < nk) issue(kt + kStages - 1, s_new);
      read_frags(s_cur, 0);
      steps_but_last(s_cur);
      mfmas((kSub - 1) & 1);
      s_cur = (s_cur + 1 == kStages) ? 0 : s_cur + 1;
      s_new = (s_new + 1 == kStages) ? 0 : s_new + 1;
    }
  } else {
    // barrier before the last k16 step of each stage: the fragments of the
    // next stage's first step are read while the last step's MFMAs run
    if (kStages - 2 < nk)
      wait_vmcnt<kLoads * (kStages - 2)>();
    else
      wait_vmcnt<0>();
    bare_barrier();
    read_frags(0, 0);
#pragma unroll 1
    for (int kt = 0; kt + 1 < nk; ++kt) {
      steps_but_last(s_cur);
      const int s_nxt = (s_cur + 1 == kStages) ? 0 : s_cur + 1;
      // step kt + 1 has landed (this wave's chunks) once no more than the
      // chunks of the steps issued after it are outstanding
      if (kt + kStages - 2 < nk)
        wait_vmcnt<kLoads * (kStages - 3)>();
      else
        wait_vmcnt<0>();
      // every wave's chunks of step kt + 1 are in LDS, and every wave has
      // consumed its fragments of step kt - 1, whose stage is refilled next
      bare_barrier();
      if (kt + kStages - 1 < nk) issue(kt + kStages - 1, s_new);
      read_frags(s_nxt, 0);
      mfmas((kSub - 1) & 1);
      reads_then_mfmas();
      s_cur = s_nxt;
      s_new = (s_new + 1 == kStages) ? 0 : s_new + 1;
    }
    // the last step (nothing left to load)
    steps_but_last(s_cur);
    mfmas((kSub - 1) & 1);
  }
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with the operand stages

  // Epilogue, kEpiPasses row bands of kEpiRows rows: round to bf16 and
  // stage the band in LDS (row-major, padded rows; lane holds column
  // (lane & 31) of each 32 x 32 block and rows (r / 4) * 8 + (lane / 32) * 4
  // + r % 4 of it), store it with coalesced 16-byte stores (N is a multiple
  // of 8, so a chunk is either whole or past the end), then, with kStats,
  // reduce its pieces.
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
  uint16_t* C = static_cast<uint16_t*>(P.logits);
  constexpr int kRowChunks = kTN / 8;
#pragma unroll 1
  for (int pass = 0; pass < kEpiPasses; ++pass) {
    const int r0 = pass * kEpiRows;  // first tile row of the band
    if (wm / (kWM / kEpiPasses) == pass) {
#pragma unroll
      for (int bi = 0; bi < kBI; ++bi)
#pragma unroll
        for (int bj = 0; bj < kBJ; ++bj)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm * (kTM / kWM) + bi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) - r0;
            const int col = wn * (kTN / kWN) + bj * 32 + (lane & 31);
            stage[row * kOutRow + col] = static_cast<uint16_t>(bf16_bits_rne(acc[bi][bj][r]));
          }
    }
    __syncthreads();

#pragma unroll 4
    for (int idx = tid; idx < kEpiRows * kRowChunks; idx += kThreadsG) {
      const int row = idx / kRowChunks, ch = idx % kRowChunks;
      const int m = m0 + r0 + row;
      const int n = n0 + ch * 8;
      if (m < P.M && n < P.N)
        *reinterpret_cast<uint4*>(C + static_cast<int64_t>(m) * P.N + n) = load16(stage + row * kOutRow + ch * 8);
    }

    if constexpr (kStats) {
      // Two threads per row and 128-column piece (64 values each): the
      // piece's reference over its stored values (columns past N
      // excluded), then the sum of 2^(x c - reference).
      constexpr int kPieces = kTN / kLMPiece;
      constexpr int kHalves = kEpiRows * kPieces * 2;
      static_assert(kHalves % kWave == 0, "whole waves per pass (the two halves of a piece meet by a lane shuffle)");
#pragma unroll 1
      for (int u = tid; u < kHalves; u += kThreadsG) {
        const int half = u & 1;
        const int pc = (u >> 1) % kPieces;
        const int row = (u >> 1) / kPieces;
        const int m = m0 + r0 + row;
        const int nstart = n0 + pc * kLMPiece;
        float x[64];
        const uint16_t* srcs = stage + row * kOutRow + pc * kLMPiece + half * 64;
#pragma unroll
        for (int v = 0; v < 8; ++v) unpack<BF16>(load16(srcs + v * 8), &x[v * 8]);
        const int nvalid = min(64, max(0, P.N - (nstart + half * 64)));
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
        float sum = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
        sum += __shfl_xor(sum, 1, kWave);
        if (half == 0 && m < P.M && nstart < P.N) {
          const float ref = (mx == -INFINITY) ? -INFINITY : mx * c.hi;
          P.pieces[static_cast<int64_t>(m) * P.npieces + nstart / kLMPiece] = make_float2(ref, sum);
        }
      }
    }
    if (pass + 1 < kEpiPasses) __syncthreads();  // the next band overwrites the staging rows
  }
}

LMHeadParams with_tiles(const LMHeadParams& p) {
  LMHeadParams q = p;
  q.mt = static_cast<int32_t>((static_cast<int64_t>(p.M) + kTM - 1) / kTM);
  q.nt = static_cast<int32_t>((static_cast<int64_t>(p.N) + kTN - 1) / kTN);
  return q;
}

}  // namespace

int64_t lm_head_grid(const LMHeadParams& p) {
  const LMHeadParams q = with_tiles(p);
  const int64_t rounds = (static_cast<int64_t>(q.nt) + kXcds - 1) / kXcds;
  return rounds * kXcds * q.mt;
}

hipError_t launch_lm_head_gemm(const LMHeadParams& p, bool stats, const PassEvents& ev, hipStream_t stream) {
  const int64_t grid = lm_head_grid(p);
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  // every buffer the kernel writes or reads must be there, and the shapes
  // it assumes must hold
  if (p.hidden == nullptr || p.weight == nullptr || p.logits == nullptr || (stats && p.pieces == nullptr))
    return hipErrorInvalidValue;
  if (p.M < 1 || p.N < 8 || p.N % 8 != 0 || p.H < kKS || p.H % kKS != 0 ||
      (stats && p.npieces != (p.N + kLMPiece - 1) / kLMPiece))
    return hipErrorInvalidValue;
  const LMHeadParams q = with_tiles(p);
  if (stats)
    launch_stream_pass(lm_head_gemm_kernel<true>, dim3(static_cast<uint32_t>(grid)), dim3(kThreadsG), stream, ev, q);
  else
    launch_stream_pass(lm_head_gemm_kernel<false>, dim3(static_cast<uint32_t>(grid)), dim3(kThreadsG), stream, ev, q);
  return hipGetLastError();
}

}  // namespace sv
