// Internal host/device interface between the C-ABI entry points and the
// kernels. Not installed; the public contract is include/specverify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specverify.h"
#include "sv_device.h"

namespace sv {

// Hand-off from the decision kernel to the sampling kernel, one per
// sequence: which row pair to sample from and its normalisers.
struct SeqPlan {
  int32_t j;     // first rejected position; K = bonus draw; -1 = invalid row
  float c_hi;    // log2(e) / T as an unevaluated fp32 sum c_hi + c_lo
  float c_lo;
  float lt_hi;   // L_t = log2 of the target row's normaliser at exponent scale
  float lt_lo;   //   c, as lt_hi + lt_lo:  p_t(v) = 2^(x_t c - L_t)
  float d_hi;    // D = L_d - L_t as d_hi + d_lo:  p_d(v) / p_t(v) =
  float d_lo;    //   2^((x_d - x_t) c - D)    (unused for the bonus draw)
  float pad;
};

constexpr int kPlanWords = 8;  // 32-bit fields of a SeqPlan

struct ChainParams {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* temperature;
  const float* uniforms;
  int32_t B, K, V;
  int32_t nseg;            // statistics segments per logit row (row layout)
  int32_t seg_vecs;        // 16-byte vectors per statistics segment
  int32_t fl_blocks;       // > 0: flattened layout with this many statistics blocks
  int32_t fl_kmax;         //   row pieces per block (upper bound)
  int64_t fl_nvec;         //   16-byte vectors per row
  int64_t fl_per;          //   vectors per block
  int32_t ntiles;          // sampling tiles per row (kSampleTile elements each)
  int32_t tiles_per_block; // sampling tiles handled by one workgroup
  int32_t nblk_b;          // sampling workgroups per sequence
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_draft;
  float* q_draft;
  float* residual_mass;
  int32_t* err_flags;
  // workspace (all zero between calls)
  uint64_t* part_m;   // per row piece: tagged fp32 reference fl(max * c_hi),
                      // [B, 2K+1, nseg] (row layout) or [fl_blocks, fl_kmax]
  uint64_t* part_s;   // per row piece: tagged fp64 sum of 2^(x c - reference)
  uint64_t* plan_w;   // [B, kPlanWords] tagged decision -> sampling hand-off
  uint32_t* cnt;      // [B] sampling arrivals
  uint64_t* tile_sum; // [B, ntiles] tagged fp64 sampling weight per tile
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

// Statistics segment: kThreads * kStatsUnroll * kStatsBatches vectors.
constexpr int kStatsUnroll = 4;
constexpr int kStatsBatches = 2;
constexpr int kStatsSegVecs = 256 * kStatsUnroll * kStatsBatches;
constexpr int kSampleTilesPerBlock = 4;

// Flattened statistics layout: about this many chunks, each with at least
// kFlatMinVecsPerBlock 16-byte vectors.
#ifndef SV_FLAT_CHUNKS
#define SV_FLAT_CHUNKS 4096
#endif
constexpr int kFlatChunksTarget = SV_FLAT_CHUNKS;
constexpr int kFlatMinVecsPerBlock = 256 * kStatsUnroll * 2;

static_assert(kErrInternal == SV_ERRF_INTERNAL, "error bit mismatch");

hipError_t launch_chain(const ChainParams& p, sv_dtype dtype, hipStream_t stream);
hipError_t launch_tree(const TreeParams& p, sv_dtype dtype, hipStream_t stream);
hipError_t launch_tree_mask(const int32_t* parents, int32_t N, uint8_t* mask, int32_t* err_flags,
                            hipStream_t stream);

}  // namespace sv
