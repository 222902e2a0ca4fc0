// Internal host/device interface between the C-ABI entry points and the
// kernels. Not installed; the public contract is include/specverify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specverify.h"
#include "sv_device.h"

namespace sv {

// The decision of one sequence as the sampling step needs it: which row pair
// to draw from and the rows' normalisers (written by the decision kernel,
// read by every sampling workgroup of the sequence).
struct SeqPlan {
  int32_t j;     // first rejected position; K = bonus draw; -1 = invalid row
  float c_hi;    // log2(e) / T as an unevaluated fp32 sum c_hi + c_lo
  float c_lo;
  float lt_hi;   // L_t = log2 of the target row's normaliser at exponent scale
  float lt_lo;   //   c, as lt_hi + lt_lo:  p_t(v) = 2^(x_t c - L_t)
  float d_hi;    // D = L_d - L_t as d_hi + d_lo:  p_d(v) / p_t(v) =
  float d_lo;    //   2^((x_d - x_t) c - D)    (unused for the bonus draw)
  uint32_t valid;  // 1 once written (the workspace is zero otherwise)
};

struct ChainParams {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* temperature;
  const float* uniforms;
  int32_t B, K, V;
  // Statistics layout, one of:
  //  chunked (every row on a 16-byte boundary): each sequence's 2K+1 rows,
  //    concatenated, are cut into cps chunks of `per` 16-byte vectors; a chunk
  //    publishes one piece per row it touches (at most kmax);
  //  rows (any alignment): nseg segments of seg_vecs vectors per row.
  int32_t cps;             // > 0: chunked layout
  int32_t kmax;
  int64_t nvec;            // 16-byte vectors per row (chunked layout)
  int64_t per;
  int32_t nseg;
  int32_t seg_vecs;
  // Sampling: nblk_b workgroups per sequence, each over tiles_per_block
  // tiles of kSampleTile tokens.
  int32_t ntiles;
  int32_t tiles_per_block;
  int32_t nblk_b;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_draft;
  float* q_draft;
  float* residual_mass;
  int32_t* err_flags;
  // workspace (all zero between calls)
  uint64_t* part_m;   // per row piece: tagged fp32 reference fl(max * c_hi),
                      // [B, cps, kmax] (chunked) or [B, 2K+1, nseg] (rows)
  uint64_t* part_s;   // per row piece: tagged fp64 sum of 2^(x c - reference)
  SeqPlan* plan;      // [B] decision -> sampling hand-off
  uint32_t* cnt;      // [B] sampling arrivals
  uint64_t* tile_sum; // [B, ntiles] tagged fp64 sampling weight per tile
  uint64_t* gat;      // [B, 2K+1] tagged fp32 logit of row r at its drafted
                      // token (rows 0..K-1 and K+1..2K; set by the pass that
                      // streams the piece holding it)
  uint64_t* abort;    // [1] set when a bounded wait expires (drains the launch)
};

struct TreeParams {
  const void* target;
  const int32_t* tokens;
  const int32_t* parents;
  int32_t B, N, V;
  int32_t nseg;
  int32_t seg_vecs;
  int32_t* accept_len;
  int32_t* path_nodes;
  int32_t* next_token;
  int32_t* err_flags;
  uint64_t* part;    // [B, N+1, nseg] per-segment (max value, lowest index + 1)
  uint32_t* cnt;     // [B]
  uint64_t* abort;   // [1] set when a bounded wait expires
};

constexpr int kSampleEPT = 8;                      // sampling elements per thread per tile
constexpr int kSampleTile = 256 * kSampleEPT;      // elements per sampling tile
// Tiles per resolving workgroup: 16 KB of each sampled row either way.
constexpr int kSampleTilesBF16 = 4;
constexpr int kSampleTilesF32 = 2;

// Statistics segment (rows layout): kThreads * kStatsUnroll * kStatsBatches vectors.
constexpr int kStatsUnroll = 4;
constexpr int kStatsBatches = 2;
constexpr int kStatsSegVecs = 256 * kStatsUnroll * kStatsBatches;

// Chunked statistics layout: about this many chunks per call, each with at
// least kChunkMinVecs 16-byte vectors.
#ifndef SV_CHUNKS
#define SV_CHUNKS 4096
#endif
constexpr int kChunksTarget = SV_CHUNKS;
constexpr int kChunkMinVecs = 256 * kStatsUnroll * 2;

static_assert(kErrInternal == SV_ERRF_INTERNAL, "error bit mismatch");

// Events armed by sv_time_next_stream_pass for the calling thread's next
// call; take_pass_events() returns them and disarms the hook.
struct PassEvents {
  hipEvent_t before;
  hipEvent_t after;
};
PassEvents take_pass_events();

// Statistics work items of the call, and the three launches of a chain call.
int64_t chain_stats_items(const ChainParams& p);
// `ev` (possibly null events) brackets the streaming pass of the call.
hipError_t launch_chain(const ChainParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream);
hipError_t launch_tree(const TreeParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream);
hipError_t launch_tree_mask(const int32_t* parents, int32_t N, uint8_t* mask, int32_t* err_flags,
                            hipStream_t stream);

}  // namespace sv
