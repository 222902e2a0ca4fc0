// Internal host/device interface between the C-ABI entry points and the
// kernels. Not installed; the public contract is include/specverify.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specverify.h"
#include "sv_device.h"

namespace sv {

// The decision of one sequence as the sampling step needs it: which row pair
// to draw from and the rows' normalisers (made by every sampling workgroup
// of the sequence for itself).
struct SeqPlan {
  int32_t j;     // first rejected position; K = bonus draw; -1 = invalid row
  float c_hi;    // log2(e) / T as an unevaluated fp32 sum c_hi + c_lo
  float c_lo;
  float lt_hi;   // L_t = log2 of the target row's normaliser at exponent scale
  float lt_lo;   //   c, as lt_hi + lt_lo:  p_t(v) = 2^(x_t c - L_t)
  float d_hi;    // D = L_d - L_t as d_hi + d_lo:  p_d(v) / p_t(v) =
  float d_lo;    //   2^((x_d - x_t) c - D)    (unused for the bonus draw)
  uint32_t pad;
};

// How a streaming pass cuts the logit rows of a call into work items, and
// where each item publishes one 64-bit slot per row piece. Two layouts:
//  chunked (every row starts on a 16-byte boundary): the `rows` rows of a
//    sequence, laid end to end, are cut into cps chunks of `per` 16-byte
//    vectors; a chunk publishes one slot per row it touches (at most kmax),
//    slot (b * cps + chunk) * kmax + (row - first row of the chunk);
//  segments (any alignment): nseg segments of seg_vecs vectors per row, slot
//    (b * rows + row) * nseg + segment.
struct PieceLayout {
  int32_t rows;      // logit rows per sequence
  int32_t cps;       // > 0: chunked layout
  int32_t kmax;
  int64_t nvec;      // 16-byte vectors per row (chunked layout)
  int64_t per;
  int32_t nseg;      // segments layout
  int32_t seg_vecs;
};

// Work items per sequence, and slots per sequence.
__host__ __device__ __forceinline__ int64_t items_per_seq(const PieceLayout& L) {
  return L.cps > 0 ? L.cps : static_cast<int64_t>(L.rows) * L.nseg;
}
__host__ __device__ __forceinline__ int64_t slots_per_seq(const PieceLayout& L) {
  return L.cps > 0 ? static_cast<int64_t>(L.cps) * L.kmax : static_cast<int64_t>(L.rows) * L.nseg;
}

// a / b for non-negative 64-bit values, in 32-bit arithmetic when both fit
// (a hardware-friendly path for every realistic size).
__device__ __forceinline__ int64_t div_nonneg(int64_t a, int64_t b) {
  if (((a | b) >> 32) == 0) return static_cast<int64_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(b));
  return a / b;
}

// Slot of piece p of row r of sequence b, or -1 past the row's last piece.
__device__ __forceinline__ int64_t piece_slot(const PieceLayout& L, int b, int r, int p) {
  if (L.cps > 0) {
    const int64_t ch = div_nonneg(r * L.nvec, L.per) + p;
    if (ch > div_nonneg((r + 1) * L.nvec - 1, L.per)) return -1;
    return (static_cast<int64_t>(b) * L.cps + ch) * L.kmax + (r - div_nonneg(ch * L.per, L.nvec));
  }
  return p < L.nseg ? (static_cast<int64_t>(b) * L.rows + r) * L.nseg + p : -1;
}

// Largest number of pieces of any row.
__device__ __forceinline__ int max_pieces(const PieceLayout& L) {
  if (L.cps > 0) return static_cast<int>(div_nonneg(L.nvec + L.per - 2, L.per)) + 1;
  return L.nseg;
}

struct ChainParams {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* temperature;
  const float* uniforms;
  int32_t B, K, V;
  PieceLayout L;           // statistics pass; rows = 2K+1 (target 0..K, then draft)
  // Sampling: nblk_b workgroups per sequence, each over tiles_per_block
  // tiles of kSampleTile tokens (a multiple of the kernel's group of tiles).
  int32_t ntiles;
  int32_t tiles_per_block;
  int32_t nblk_b;
  int32_t* accept_len;  // null only for draft-side sampling (K = 0)
  int32_t* out_tokens;
  float* p_draft;
  float* q_draft;
  float* residual_mass;
  float* drawn_prob;  // [B] or null: p of the token drawn at j (draft-side sampling, K = 0)
  float* entropy;     // [B, 2K+1] or null: entropy (nats) of every row's distribution
  int32_t* err_flags;
  // workspace (all zero between calls)
  uint64_t* part_m;   // per row piece: tagged fp32 reference fl(max * c_hi)
  uint64_t* part_s;   // per row piece: tagged fp64 sum of 2^(x c - reference)
  uint64_t* part_a;   // per row piece, entropy only: tagged (complemented)
                      // fp64 sum of 2^a * a, a = x c - reference
  uint32_t* cnt;      // [B] sampling workgroups finished
  uint64_t* tile_sum; // [B, ntiles] tagged fp64 sampling weight per tile
  uint64_t* gat;      // [B, 2K+1] tagged fp32 logit of row r at its drafted
                      // token (rows 0..K-1 and K+1..2K; set by the pass that
                      // streams the piece holding it)
  uint64_t* abort;    // [1] set when a bounded wait expires (drains the launch)
  // One-launch call (statistics and sampling in one grid, see
  // chain_one_launch_kernel): per sequence, the ticket counter of its queue
  // and the number of statistics chunks counted.
  int32_t one_launch;
  uint32_t* tk;       // [B]
  uint32_t* done;     // [B]
  // Small call (chain_small_kernel, one_launch == 2): the statistics
  // workgroups also sample. The last of a sequence's chunks to be counted in
  // done[b] makes the decision and publishes its plan here, kPlanStride
  // words per sequence, the first 8 of them tagged (j + 1, c_hi, c_lo,
  // lt_hi, lt_lo, d_hi, d_lo; one unused).
  uint64_t* plan;
  // LM-head chain call: the GEMM's statistics pieces of the target rows,
  // [B (K+1), lm_ntn] (reference, sum), combined into the row slots (and
  // zeroed) by lm_head_stats_kernel
  float2* lm_pieces;
  int32_t lm_ntn;
};

// The target's LM head as a GEMM: logits [M, N] = hidden [M, H] x weight
// [N, H]^T, bf16 in and out, fp32 accumulation; with the statistics, one
// (reference, sum) piece per row and 128-column piece (see sv_lm_head.hip).
struct LMHeadParams {
  const void* hidden;        // [M, H] bf16, 16-byte aligned
  const void* weight;        // [N, H] bf16, 16-byte aligned
  void* logits;              // [M, N] bf16 out, 16-byte aligned
  int32_t M, N;              // N a multiple of 8
  int64_t H;                 // a multiple of 64
  int32_t K1;                // rows per sequence: row m belongs to sequence m / K1
  const float* temperature;  // [M / K1] or null (1.0)
  int32_t npieces;           // 128-column statistics pieces per row, ceil(N / 128)
  float2* pieces;            // [M, npieces] out (statistics only)
  int32_t mt, nt;            // GEMM tiles along M and N (set by launch_lm_head_gemm)
};
constexpr int kLMPiece = 128;


// Sampling verification of a candidate tree: the run records of the target
// rows [B, N+1, V] (records rows 0 .. B(N+1)-1) and of the draft rows
// (records rows B(N+1) ..), then one walk per sequence.
struct TreeSampleParams {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* parents;
  const float* temperature;
  const float* uniforms;   // [B, N+1]
  int32_t B, N, V;
  int64_t nvec;            // 16-byte vectors per row
  int32_t nrun;            // runs of kRunVecs vectors per row (the walk's passes)
  int32_t nrec;            // statistics records (row chunks) per row
  uint64_t* rec;           // workspace [2 B (N+1), nrec]: (reference, sum) of chunk c of row r
  int32_t* accept_len;
  int32_t* path_nodes;
  int32_t* next_token;
  int32_t* err_flags;
  // G > 1: G walk workgroups per sequence share every pass over a row pair
  int32_t G;
  uint64_t* slots;         // workspace [B, 2, nrun]: a pass's run totals, tagged with the pass number
  uint32_t* cnt;           // workspace [B + 2]: per sequence walk workgroups finished; ticket; grid finished
  uint64_t* abort;         // workspace [1]: set when a bounded wait expires
};

// Walk workgroups per sequence, at most.
constexpr int kMaxWalkGroups = 8;
// Statistics chunks per sampling-tree call, about (every row cut into the
// same whole number of chunks).
#ifndef SV_CHUNKS_TREE_SAMPLE
#define SV_CHUNKS_TREE_SAMPLE 8192
#endif
constexpr int kChunksTreeSample = SV_CHUNKS_TREE_SAMPLE;

// Runs per row the walk keeps totals of in LDS.
constexpr int kMaxWalkRuns = 1024;

struct TreeParams {
  const void* target;
  const int32_t* tokens;
  const int32_t* parents;
  int32_t B, N, V;
  PieceLayout L;      // argmax pass; rows = N+1
  int32_t* accept_len;
  int32_t* path_nodes;
  int32_t* next_token;
  int32_t* err_flags;
  uint64_t* part;     // per row piece: (max value bits << 32) | (lowest index + 1)
};

// Runs of kRunVecs 16-byte vectors (the last run of a row may be short):
// the unit of the sampling-tree walk's passes over a row pair.
#ifndef SV_RUN_VECS
#define SV_RUN_VECS 128
#endif
constexpr int kRunVecs = SV_RUN_VECS;
constexpr int kRunLaneVecs = kRunVecs / kWave;  // vectors per lane per run

// One-launch draft-side sampling (rows on 16-byte boundaries). Each row is
// cut into units of kUnitVecs 16-byte vectors (upr per row, the last may be
// short), and every unit into segments of kSegVecs vectors, one record per
// segment (nrec = upr * kSegsPerUnit per row, in token order; segments past
// the row's end are empty records). The call's R * upr units are split into
// ngroups contiguous ranges; group k's range is streamed by the waves of
// blocks k, k + ngroups, k + 2 ngroups, ... (wpg blocks: one of every
// round in which the hardware hands blocks out), which take its units in
// order from the group's counter, one unit per wave at a time. A second
// launch draws each row's token from its records and one segment.
#ifndef SV_SEG_VECS
#define SV_SEG_VECS 256
#endif
constexpr int kSegVecs = SV_SEG_VECS;
#ifndef SV_SEGS_PER_UNIT
#define SV_SEGS_PER_UNIT 4
#endif
constexpr int kSegsPerUnit = SV_SEGS_PER_UNIT;
constexpr int kUnitVecs = kSegVecs * kSegsPerUnit;
#ifndef SV_SAMPLE_WGS_PER_CU
#define SV_SAMPLE_WGS_PER_CU 8
#endif
constexpr int kSampleWGsPerCU = SV_SAMPLE_WGS_PER_CU;
#ifndef SV_SAMPLE_GROUPS
#define SV_SAMPLE_GROUPS 256
#endif
constexpr int kSampleGroups = SV_SAMPLE_GROUPS;
// Units per wave the grid is sized for, at least (small calls launch fewer
// blocks). Measured on MI355X, s2 = 320 rows of V = 128256 bf16 and
// s3 = 2048 rows of V = 152064 bf16, stream kernel by its launch events:
// 1024-vector units, one unit per wave 19.4 / 108.3 us; two units per wave
// 23.1 / 107.0 us; 512-vector units 19.7-20.5 / 109.1-109.2 us; 256-vector
// units 21.8 / 114.2 us. A static split (one piece per wave, no counter)
// measured 18.4 / 110.7 us.
#ifndef SV_SAMPLE_UNITS_PER_WAVE
#define SV_SAMPLE_UNITS_PER_WAVE 1
#endif
constexpr int kSampleUnitsPerWave = SV_SAMPLE_UNITS_PER_WAVE;
constexpr int kSegLaneVecs = kSegVecs / kWave;  // vectors per lane of the draw's rescan
static_assert(kSegVecs % (kWave * 2) == 0, "segments are whole batches of the stream");

struct SampleParams {
  const void* logits;      // [R, V] rows; row r uses temperature[r]
  const float* temperature;
  const float* uniforms;
  int32_t R, V;
  int64_t nvec;        // 16-byte vectors per row
  int32_t upr;         // units per row
  int32_t nrec;        // records per row (upr * kSegsPerUnit)
  int32_t ngroups;     // unit groups (and counters)
  int32_t wpg;         // blocks per group
  int32_t* out_tokens;
  float* out_prob;
  int32_t* err_flags;
  uint64_t* rec_m;     // workspace [R, nrec]: tagged fp32 reference of a segment
  uint64_t* rec_s;     // workspace [R, nrec]: tagged fp64 sum of 2^(x c - reference)
  uint32_t* take;      // workspace [ngroups * kCtrStride]: units of the group handed out (+ failed takes)
};

// A run record of the sampling-tree walk: the fp32 reference in the upper
// half, the fp32 sum with its sign bit set in the lower half (so a written
// record is never zero).
__device__ __forceinline__ uint64_t tag_run(float ref, float sum) {
  return (static_cast<uint64_t>(__float_as_uint(ref)) << 32) |
         static_cast<uint64_t>(__float_as_uint(sum) | 0x80000000u);
}
__device__ __forceinline__ float run_ref(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v >> 32)); }
__device__ __forceinline__ float run_sum(uint64_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) & 0x7fffffffu);
}

constexpr int kSampleEPT = 8;                      // sampling elements per thread per tile
constexpr int kSampleTile = 256 * kSampleEPT;      // elements per sampling tile
// Tiles per sampling workgroup (the same bytes of each sampled row for both
// dtypes).
#ifndef SV_SAMPLE_TILES_BF16
#define SV_SAMPLE_TILES_BF16 4
#endif
constexpr int kSampleTilesBF16 = SV_SAMPLE_TILES_BF16;
constexpr int kSampleTilesF32 = kSampleTilesBF16 / 2;
// With K = 0 (draft-side sampling) only one row is drawn from, and each
// workgroup takes this many times as many tiles.
#ifndef SV_SAMPLE_TILES_K0_FACTOR
#define SV_SAMPLE_TILES_K0_FACTOR 4
#endif
constexpr int kSampleTilesK0Factor = SV_SAMPLE_TILES_K0_FACTOR;
// Sampling workgroups per call the tile groups are spread over (a workgroup
// takes several groups in turn when B * ntiles is large).
#ifndef SV_SAMPLE_BLOCKS
#define SV_SAMPLE_BLOCKS 2048
#endif
constexpr int kSampleBlocks = SV_SAMPLE_BLOCKS;

// Segments layout: kThreads * kStatsUnroll * kStatsBatches vectors per segment.
constexpr int kStatsUnroll = 4;
constexpr int kStatsBatches = 2;
constexpr int kStatsSegVecs = 256 * kStatsUnroll * kStatsBatches;

// Chunked statistics stream: 16-byte vectors per thread per batch (the
// batch's maximum is taken before its exponentials are summed).
#ifndef SV_STREAM_U
#define SV_STREAM_U 2
#endif
constexpr int kStreamU = SV_STREAM_U;
// The same for the entropy variant of the stream (2: the same batches, so the
// same rounding of every other output, as the plain stream).
#ifndef SV_STREAM_U_ENT
#define SV_STREAM_U_ENT 2
#endif
constexpr int kStreamUEnt = SV_STREAM_U_ENT;
// Threads per workgroup of the chunked statistics stream.
#ifndef SV_STATS_TPB
#define SV_STATS_TPB 256
#endif
constexpr int kStatsTPB = SV_STATS_TPB;
// The one-launch chain call: on (1) for the calls it serves (see
// one_launch_ok on the host), or off (0: always two launches). Waves per
// SIMD its kernel (statistics and sampling roles) is compiled for, and the
// sampling tiles whose loads a workgroup keeps in flight together: 69 VGPRs
// with four tiles (7 waves/SIMD), 62 with one or two (8 waves; measured
// 52.1 us per B=64 K=5 V=128256 bf16 call with two, 50.8-51.4 us with four
// at 7 waves).
#ifndef SV_ONE_LAUNCH
#define SV_ONE_LAUNCH 1
#endif
#ifndef SV_ONE_LAUNCH_WAVES
#define SV_ONE_LAUNCH_WAVES 7
#endif
constexpr int kOneLaunchWGsPerCU = SV_ONE_LAUNCH_WAVES;  // 4-wave workgroups on 4 SIMDs
#ifndef SV_LIVE_TILES
#define SV_LIVE_TILES 4
#endif
constexpr int kLiveTiles = SV_LIVE_TILES;
// The same in tiles of a dtype: fp32 tiles are twice the bytes of bf16 ones,
// so half as many keep the same loads in flight (with four, the fp32 kernel
// spilled 30 VGPRs to scratch at 7 waves/SIMD).
template <class T>
constexpr int live_tiles() {
  return T::kBytes == 2 ? kLiveTiles : (kLiveTiles + 1) / 2;
}
// Per-sequence counters of the one-launch call (ticket, chunks counted,
// sampling arrivals) lie this many 32-bit words apart. Packed counters put
// the polls of the waiting sampling workgroups and the contended ticket
// atomics on one memory channel, and the streaming workgroups, which have
// loads queued on every channel, stall behind them: on B=64 K=5 V=128256
// bf16 the call took 109-116 us with packed counters, 50.8 us with counters
// 256 bytes apart, 51.4 us 4 KB apart and 53.3 us 64 bytes apart.
#ifndef SV_CTR_STRIDE
#define SV_CTR_STRIDE 64
#endif
constexpr int kCtrStride = SV_CTR_STRIDE;
// Pause between two polls of a waiting sampling workgroup (s_sleep units
// of 64 cycles), and the wave priority (0-3) of the sampling roles (3
// measured 52.3 us per B=64 K=5 call against 51.4 us at 0, polls 8 or 32
// the same).
#ifndef SV_POLL_SLEEP
#define SV_POLL_SLEEP 8
#endif
#ifndef SV_SAMPLE_PRIO
#define SV_SAMPLE_PRIO 0
#endif
// Wave priority (0-3) of wave 0 of a one-launch sampling role once its
// sequence's statistics are all counted (the decision, then the rest of the
// role; SV_TAIL_PRIO_ALL raises the role's other waves too), and whether a
// statistics role waits for its slot stores before counting its chunk (1)
// or counts at once (0; the readers retry while a slot is zero). On B=64
// K=5 V=128256 bf16, priority 1 or 3 took the call from 48.6-48.8 us to
// 47.4-47.6 us; raising all four waves, or 8 waves/SIMD, was slower
// (48.6-49.1 us), and so was the large call B=256 K=8 V=152064 with all four
// raised (240 us against 234 us).
#ifndef SV_TAIL_PRIO
#define SV_TAIL_PRIO 3
#endif
#ifndef SV_COUNT_WAIT
#define SV_COUNT_WAIT 0
#endif
#ifndef SV_TAIL_PRIO_ALL
#define SV_TAIL_PRIO_ALL 0
#endif
// The last SV_LATE_PRIO_SEQS sequences (the last streamed) raise all the
// waves of their sampling roles, and a sampling role reads the statistics
// slots directly once at most SV_EAGER_CHUNKS chunks of its sequence are
// uncounted. On B=64 K=5 V=128256 bf16: 47.8-48.0 us per call with neither,
// 47.2-47.6 us with 2 eager chunks (1, 3 and 4 within 0.3 us of it), kernel
// 43.9 us against 44.2-44.3 us with the last 8 sequences raised as well (16:
// 44.5-45.0 us).
#ifndef SV_LATE_PRIO_SEQS
#define SV_LATE_PRIO_SEQS 8
#endif
#ifndef SV_EAGER_CHUNKS
#define SV_EAGER_CHUNKS 2
#endif
// Small chain call: whether a statistics workgroup waits for its slot stores
// before counting its chunk, and the wave priority of the deciding wave
// (K=5 V=128256 bf16, B=16: 23.6-23.8 us per call at 3 against 24.2 us at
// 0; B=1, B=4 and B=4 K=4 V=32000 fp32 the same either way, counting
// without the wait too).
#ifndef SV_SMALL_COUNT_WAIT
#define SV_SMALL_COUNT_WAIT 1
#endif
#ifndef SV_SMALL_PRIO
#define SV_SMALL_PRIO 3
#endif
#ifndef SV_SMALL_SPEC
#define SV_SMALL_SPEC 1
#endif
#ifndef SV_SMALL_POLL_SLOTS
#define SV_SMALL_POLL_SLOTS 1
#endif
// Block order of the one-launch grid: the sampling blocks of sequence b
// follow the statistics blocks of sequence b + lag (the last lag sequences'
// sampling blocks close the grid), so that with in-order dispatch they start
// about when b's statistics are done. lag >= B puts every sampling block
// after every statistics block (a lag of 16 or 32 sequences measured 56.7
// and 52.8 us per B=64 K=5 call against 51.4 us).
#ifndef SV_SAMPLE_LAG
#define SV_SAMPLE_LAG 1000000
#endif
constexpr int kSampleLag = SV_SAMPLE_LAG;
// Waves per SIMD the chunked statistics stream is compiled for (8: at most 64
// VGPRs; 4: at most 128).
#ifndef SV_STATS_WAVES
#define SV_STATS_WAVES 8
#endif
// The same for the entropy variant of the stream (66 VGPRs with bf16: its
// extra accumulator and the two forms of a batch's sum of A).
#ifndef SV_STATS_WAVES_ENT
#define SV_STATS_WAVES_ENT 7
#endif

// Chunked layouts: each row is cut into k equal chunks (one workgroup each),
// k the nearest integer to this target over the rows of the call, each chunk
// of at least kChunkMinVecs 16-byte vectors. Measured best: 2816 for the
// chain stream (quarter rows on B=64 K=5 V=128256), 4096 for the tree stream
// (half rows on B=32 N=64 V=128256: 82-84 us against 85 us for 4096 chunks
// cut across rows).
#ifndef SV_CHUNKS_CHAIN
#define SV_CHUNKS_CHAIN 2816
#endif
constexpr int kChunksChain = SV_CHUNKS_CHAIN;
#ifndef SV_CHUNKS_TREE
#define SV_CHUNKS_TREE 4096
#endif
constexpr int kChunksTree = SV_CHUNKS_TREE;
#ifndef SV_CHUNK_MIN_VECS
#define SV_CHUNK_MIN_VECS 2048
#endif
// Small calls (at most kSmallMaxRows logit rows in all, B (2K+1)): one
// launch whose statistics workgroups also decide and sample. Chunk size
// aimed at (16-byte vectors), the most chunks per call, and the workgroups
// per compute unit the whole grid must fit in to take the path.
#ifndef SV_SMALL
#define SV_SMALL 1
#endif
#ifndef SV_SMALL_MAX_ROWS
#define SV_SMALL_MAX_ROWS 256
#endif
#ifndef SV_SMALL_TARGET_VECS
#define SV_SMALL_TARGET_VECS 1400
#endif
#ifndef SV_SMALL_CHUNKS
#define SV_SMALL_CHUNKS 768
#endif
#ifndef SV_SMALL_WGS_PER_CU
#define SV_SMALL_WGS_PER_CU 6
#endif
constexpr int kSmallMaxRows = SV_SMALL_MAX_ROWS;
constexpr int kSmallTargetVecs = SV_SMALL_TARGET_VECS;
constexpr int kSmallChunks = SV_SMALL_CHUNKS;
constexpr int kSmallWGsPerCU = SV_SMALL_WGS_PER_CU;
constexpr int kPlanWords = 8;     // plan words per sequence
constexpr int kPlanStride = 32;   // words between two sequences' plans (256 bytes: the plans of
                                  // different sequences, polled by their workgroups, on different channels)
// Batches of kStreamU vectors per thread the small call's statistics chunk
// keeps in registers (all its loads in flight together).
constexpr int kSmallMaxBatches = 6;
// Tiles per workgroup of the small call's sampling (at least, and the most
// for which its workgroups keep their tile weights and the one holding the
// target's tile draws): few workgroups hold tiles, so few wait for the plan
// and read the tile totals.
#ifndef SV_SMALL_TILES
#define SV_SMALL_TILES 1
#endif
constexpr int kSmallTiles = SV_SMALL_TILES;
constexpr int kChunkMinVecs = SV_CHUNK_MIN_VECS;

static_assert(kErrInternal == SV_ERRF_INTERNAL, "error bit mismatch");

// Events armed by sv_time_next_stream_pass for the calling thread's next
// call; take_pass_events() returns them and disarms the hook.
struct PassEvents {
  hipEvent_t before;
  hipEvent_t after;
};
PassEvents take_pass_events();

// Launch a streaming kernel: with armed events through hipExtLaunchKernel
// (the events then carry that kernel's own start and end), otherwise as a
// plain launch, the form a stream capture records.
template <class Params>
inline void launch_stream_pass(void (*kernel)(Params), dim3 grid, dim3 block, hipStream_t stream,
                               const PassEvents& ev, const Params& p) {
  if (ev.before != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.before, ev.after, 0u, p);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
}

// The launches of a chain call (statistics; decision and sampling) and of a tree
// call (argmax, decision); `ev` (possibly null events) become the start and
// stop events of the streaming pass.
hipError_t launch_chain(const ChainParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream);
hipError_t launch_sample(const SampleParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream);
hipError_t launch_tree_sample(const TreeSampleParams& p, sv_dtype dtype,
                              const PassEvents& ev, hipStream_t stream);
hipError_t launch_tree(const TreeParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream);
hipError_t launch_tree_mask(const int32_t* parents, int32_t N, uint8_t* mask, int32_t* err_flags,
                            hipStream_t stream);
int64_t lm_head_grid(const LMHeadParams& p);
hipError_t launch_lm_head_gemm(const LMHeadParams& p, bool stats, const PassEvents& ev, hipStream_t stream);
// The LM-head chain call: the GEMM with statistics, the statistics of the
// draft rows and the combine of the target rows' pieces (one launch), then
// the sampling pass (the chain call's, whole-row layout).
hipError_t launch_chain_lm_head(const LMHeadParams& g, const ChainParams& p, const PassEvents& ev,
                                hipStream_t stream);

}  // namespace sv
