// C-ABI entry points of libspecverify: argument validation, workspace
// carve-up and kernel launches on the caller's stream. The contract of every
// function is documented in include/specverify.h.
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "sv_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(sv_dtype d) { return d == SV_DTYPE_F32 || d == SV_DTYPE_BF16; }
int dtype_bytes(sv_dtype d) { return d == SV_DTYPE_BF16 ? 2 : 4; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Statistics segments per row for a row of V elements.
int32_t stats_segments(int32_t V, sv_dtype d) {
  const int64_t vec = 16 / dtype_bytes(d);
  const int64_t nvec = ceil_div(V, vec);
  const int64_t n = ceil_div(nvec, sv::kStatsSegVecs);
  return static_cast<int32_t>(n < 1 ? 1 : n);
}

int64_t row_vecs(int32_t V, sv_dtype d) { return static_cast<int64_t>(V) * dtype_bytes(d) / 16; }

// A streaming pass over B sequences of `rows` rows of V elements, cut into
// work items; `chunked` (rows of whole 16-byte vectors on 16-byte
// boundaries) selects the chunked layout: chunks of at most `chunk_vecs`
// vectors, balanced within each sequence.
sv::PieceLayout piece_layout(int32_t rows, int32_t V, sv_dtype d, bool chunked, int64_t chunk_vecs) {
  sv::PieceLayout L{};
  L.rows = rows;
  L.nseg = stats_segments(V, d);
  L.seg_vecs = sv::kStatsSegVecs;
  if (chunked) {
    const int64_t nvec = row_vecs(V, d);
    const int64_t seq_vecs = rows * nvec;
    L.cps = static_cast<int32_t>(ceil_div(seq_vecs, chunk_vecs));
    L.per = ceil_div(seq_vecs, L.cps);
    L.nvec = nvec;
    L.kmax = static_cast<int32_t>((L.per + nvec - 2) / nvec + 1);
  }
  return L;
}

bool whole_vector_rows(int32_t V, sv_dtype d) { return (static_cast<int64_t>(V) * dtype_bytes(d)) % 16 == 0; }

// Chunk size of a streaming pass cut into about `chunks` chunks per call,
// each of at least kChunkMinVecs vectors.
int64_t chunk_vecs(int64_t B, int32_t rows, int32_t V, sv_dtype d, int chunks) {
  const int64_t p = ceil_div(B * rows * row_vecs(V, d), chunks);
  return p < sv::kChunkMinVecs ? sv::kChunkMinVecs : p;
}

// Chunk size of a chain or tree streaming pass: every row cut into k equal
// pieces, k the nearest integer to `chunks` / (B * rows) (at least 1, and
// pieces of at least kChunkMinVecs vectors). When k divides the row, no chunk
// crosses a row boundary, and no workgroup pauses for a block combine halfway
// through its chunk: on B=64 K=5 V=128256 bf16, quarter rows (2816 chunks)
// streamed in 32.0 us against 34.4-34.6 us for 2560 and 3072 chunks that cut
// across rows; 1 to 1.5 rows per chunk measured best on B=256 K=8 and B=1024
// K=6.
int64_t row_chunk_vecs(int64_t B, int32_t rows, int32_t V, sv_dtype d, int chunks) {
  const int64_t nvec = row_vecs(V, d);
  const int64_t seq_rows = B * rows;
  int64_t k = seq_rows > 0 ? (chunks + seq_rows / 2) / seq_rows : 1;
  const int64_t kmax = nvec / sv::kChunkMinVecs;
  if (k > kmax) k = kmax;
  if (k < 1) k = 1;
  const int64_t p = ceil_div(nvec, k);
  return p < sv::kChunkMinVecs ? sv::kChunkMinVecs : p;
}

// Slots the pass needs under either layout (the workspace does not depend on
// the alignment of the logits the call is made with).
int64_t piece_slots(int64_t B, int32_t rows, int32_t V, sv_dtype d, int64_t chunk_vecs) {
  const int64_t seg = B * sv::slots_per_seq(piece_layout(rows, V, d, false, chunk_vecs));
  if (!whole_vector_rows(V, d) || B == 0) return seg;
  const int64_t ch = B * sv::slots_per_seq(piece_layout(rows, V, d, true, chunk_vecs));
  return ch > seg ? ch : seg;
}

// Compute units of the current device (0 if the runtime cannot say).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 0;
  return cus;
}

// The one-launch chain call (statistics and sampling in one grid) serves
// the calls whose grid is larger than the device holds at once, where the
// sampling of the first sequences can overlap the streaming of the last
// ones: on MI355X B=64 K=5 V=128256 bf16 took 50.8 us against 52.8 us in two
// launches, B=256 K=8 V=152064 239 us against 250 us, B=1024 K=6 V=256000
// 1173 us against 1190 us. A smaller grid starts all at once, so all the
// workgroups of a sequence take their tickets together and queue on one
// counter: B=4 K=4 V=32000 fp32 took 26.1 us against 20.1 us. It also needs
// rows on 16-byte boundaries (the chunked layout), at least one drafted
// token, no drawn probability requested (the entropy takes a kernel variant
// of its own), and statistics that the decision reads in one round: every piece of each of the 2K+1 rows among
// G lanes of one wave with at most 4 pieces per lane (G as the decision
// takes it), chunk indices within 32 bits. Other calls keep the statistics
// pass and the sampling pass as two launches.
bool one_launch_ok(const sv::PieceLayout& L, int32_t B, int32_t K, int32_t nblk_b, bool drawn_prob) {
  if (!SV_ONE_LAUNCH || L.cps <= 0 || K <= 0 || drawn_prob) return false;
  const int64_t grid = static_cast<int64_t>(B) * (L.cps + nblk_b);
  const int cus = device_cus();
  if (cus < 1 || grid <= static_cast<int64_t>(cus) * sv::kOneLaunchWGsPerCU) return false;
  const int64_t R = 2LL * K + 1;
  if (R * L.nvec > static_cast<int64_t>(UINT32_MAX)) return false;
  const int64_t pmax = (L.nvec + L.per - 2) / L.per + 1;  // pieces of a row, at most
  int64_t G = 1;
  while (G < pmax && R * 2 * G <= 64) G <<= 1;
  return R * G <= 64 && pmax <= 4 * G;
}

// The most pieces of a row the decision reads in one round: G lanes per
// row (G the largest power of two with 2K+1 rows of 2G lanes in one wave)
// with up to 4 pieces each.
int64_t one_round_pieces(int32_t K) {
  const int64_t R = 2LL * K + 1;
  int64_t G = 1;
  while (R * 2 * G <= 64) G <<= 1;
  return 4 * G;
}

// Chunk size of the small call: every row cut into k pieces, k a divisor
// of the row's vector count (so no chunk crosses a row end: one piece, one
// combine and one slot per chunk) closest to a piece of kSmallTargetVecs
// vectors (about 22 KB: smaller chunks cost more arrivals and a wider
// decision, larger ones more than one round trip of loads), with no more
// than kSmallChunks chunks per call nor more pieces than one decision round
// reads. Measured on MI355X, per call:
//   B=4 K=4 V=32000 fp32:    9 KB chunks across row ends 16.9 us, 21 KB
//                            across 15.6 us, 16-31 KB on row ends 14.8-15.0 us;
//   B=4 K=5 V=128256 bf16:   21 KB on row ends 18.2 us, 23 KB across 19.1 us.
int64_t small_chunk_vecs(int64_t B, int32_t K, int32_t V, sv_dtype d) {
  const int32_t R = 2 * K + 1;
  const int64_t nvec = row_vecs(V, d);
  const int64_t seq_rows = B * R;
  const int64_t k0 = ceil_div(nvec, sv::kSmallTargetVecs);
  int64_t kmax = 2 * k0;
  const int64_t kcall = seq_rows > 0 ? sv::kSmallChunks / seq_rows : 1;
  if (kmax > kcall) kmax = kcall;
  const int64_t kcap = one_round_pieces(K) - 1;
  if (kmax > kcap) kmax = kcap;
  int64_t k = 1;  // 1 divides every row
  for (int64_t c = 2; c <= kmax; ++c) {
    if (nvec % c != 0) continue;
    const int64_t dc = c > k0 ? c - k0 : k0 - c, dk = k > k0 ? k - k0 : k0 - k;
    if (dc <= dk) k = c;
  }
  return ceil_div(nvec, k);
}

// Whether a chain call may take the small form at all: every form of such a
// call then cuts its rows into the small call's chunks, so that the forms
// keep giving bit-identical outputs.
bool small_shape(int32_t B, int32_t K, int32_t V, sv_dtype d) {
  return SV_SMALL && K >= 1 && whole_vector_rows(V, d) &&
         static_cast<int64_t>(B) * (2 * K + 1) <= sv::kSmallMaxRows;
}

// Chunk size of a chain call's statistics pass (chunked layout).
int64_t chain_chunk_vecs(int32_t B, int32_t K, int32_t V, sv_dtype d) {
  return small_shape(B, K, V, d) ? small_chunk_vecs(B, K, V, d)
                                 : row_chunk_vecs(B, 2 * K + 1, V, d, sv::kChunksChain);
}

// The small chain call (chain_small_kernel: the statistics workgroups also
// decide and sample) serves calls of at most kSmallMaxRows rows in all whose
// grid the device holds at once (kSmallWGsPerCU workgroups per compute
// unit), with rows on 16-byte boundaries, at least one drafted token, no
// entropy or drawn probability requested, and statistics that the decision
// reads in one round (as one_launch_ok).
bool small_ok(const sv::PieceLayout& L, int32_t B, int32_t K, int32_t V, sv_dtype d, bool extra_outputs) {
  if (!small_shape(B, K, V, d) || L.cps <= 0 || extra_outputs) return false;
  const int cus = device_cus();
  if (cus < 1 || static_cast<int64_t>(B) * L.cps > static_cast<int64_t>(cus) * sv::kSmallWGsPerCU) return false;
  const int64_t R = 2LL * K + 1;
  if (R * L.nvec > static_cast<int64_t>(UINT32_MAX)) return false;
  const int64_t pmax = (L.nvec + L.per - 2) / L.per + 1;  // pieces of a row, at most
  int64_t G = 1;
  while (G < pmax && R * 2 * G <= 64) G <<= 1;
  return R * G <= 64 && pmax <= 4 * G;
}

struct ChainLayout {
  int32_t ntiles, tiles_per_block, nblk_b;
  size_t off_part_m, off_part_s, off_part_a, off_cnt, off_tiles, off_gat, off_abort, off_tk, off_done, off_plan,
      total;
};

// min_parts: slots the call's statistics need at least (a layout other than
// the ones sized here, e.g. the LM-head call's one piece per row).
ChainLayout chain_layout(int32_t B, int32_t K, int32_t V, sv_dtype d, int64_t min_parts = 0) {
  ChainLayout L{};
  const int32_t R = 2 * K + 1;
  L.ntiles = static_cast<int32_t>(ceil_div(V, sv::kSampleTile));
  // groups of tiles whose loads a sampling workgroup keeps in flight together;
  // each workgroup takes enough groups to keep about kSampleBlocks workgroups
  // per call (its decision is redone by every workgroup)
  const int64_t group = (d == SV_DTYPE_BF16 ? sv::kSampleTilesBF16 : sv::kSampleTilesF32) *
                        (K == 0 ? sv::kSampleTilesK0Factor : 1);
  const int64_t groups = ceil_div(static_cast<int64_t>(B) * ceil_div(L.ntiles, group), sv::kSampleBlocks);
  L.tiles_per_block = static_cast<int32_t>(group * (groups < 1 ? 1 : groups));
  L.nblk_b = static_cast<int32_t>(ceil_div(L.ntiles, L.tiles_per_block));
  int64_t parts = piece_slots(B, R, V, d, chain_chunk_vecs(B, K, V, d));
  if (parts < min_parts) parts = min_parts;
  size_t off = 0;
  L.off_part_m = off;
  off = align_up(off + sizeof(uint64_t) * parts);
  L.off_part_s = off;
  off = align_up(off + sizeof(uint64_t) * parts);
  L.off_part_a = off;
  off = align_up(off + sizeof(uint64_t) * parts);
  L.off_cnt = off;
  off = align_up(off + sizeof(uint32_t) * B * sv::kCtrStride);
  L.off_tiles = off;
  off = align_up(off + sizeof(uint64_t) * static_cast<int64_t>(B) * L.ntiles);
  L.off_gat = off;
  off = align_up(off + sizeof(uint64_t) * static_cast<int64_t>(B) * R);
  L.off_abort = off;
  off = align_up(off + sizeof(uint64_t));
  L.off_tk = off;
  off = align_up(off + sizeof(uint32_t) * B * sv::kCtrStride);
  L.off_done = off;
  off = align_up(off + sizeof(uint32_t) * B * sv::kCtrStride);
  L.off_plan = off;
  off = align_up(off + sizeof(uint64_t) * static_cast<int64_t>(B) * sv::kPlanStride);
  L.total = off;
  return L;
}

// Draft-side sampling (rows on 16-byte boundaries): units of kUnitVecs vectors (upr per row),
// records of kSegVecs vectors (nrec per row); a grid of about one round of
// resident blocks on MI355X (256 compute units x kSampleWGsPerCU), fewer
// for small calls (about kSampleUnitsPerWave units per wave), in ngroups
// groups of wpg blocks. The layout depends on the call's shape only (not on
// the device), so the workspace size does too.
struct SampleLayout {
  int32_t upr, nrec, ngroups, wpg;
  size_t off_m, off_s, off_take, total;
};

SampleLayout sample_layout(int32_t R, int32_t V, sv_dtype d) {
  SampleLayout L{};
  const int64_t nvec = row_vecs(V, d);
  const int64_t upr = nvec > 0 ? ceil_div(nvec, sv::kUnitVecs) : 1;
  const int64_t units = static_cast<int64_t>(R) * upr;
  int64_t blocks = ceil_div(units, static_cast<int64_t>(sv::kWaves) * sv::kSampleUnitsPerWave);
  const int64_t most = 256LL * sv::kSampleWGsPerCU;
  blocks = blocks < 1 ? 1 : (blocks > most ? most : blocks);
  const int64_t groups = blocks < sv::kSampleGroups ? blocks : sv::kSampleGroups;
  L.upr = static_cast<int32_t>(upr);
  L.nrec = static_cast<int32_t>(upr * sv::kSegsPerUnit);
  L.ngroups = static_cast<int32_t>(groups);
  L.wpg = static_cast<int32_t>(ceil_div(blocks, groups));
  const int64_t nrec = static_cast<int64_t>(R) * L.nrec;
  size_t off = 0;
  L.off_m = off;
  off = align_up(off + sizeof(uint64_t) * nrec);
  L.off_s = off;
  off = align_up(off + sizeof(uint64_t) * nrec);
  L.off_take = off;
  off = align_up(off + sizeof(uint32_t) * static_cast<int64_t>(sv::kSampleGroups) * sv::kCtrStride);
  L.total = off;
  return L;
}

struct TreeLayout {
  size_t off_part, total;
};

TreeLayout tree_layout(int32_t B, int32_t N, int32_t V, sv_dtype d) {
  TreeLayout L{};
  size_t off = 0;
  L.off_part = off;
  off = align_up(off + sizeof(uint64_t) * piece_slots(B, N + 1, V, d, row_chunk_vecs(B, N + 1, V, d, sv::kChunksTree)));
  L.total = off;
  return L;
}

bool chain_sizes_ok(int32_t B, int32_t K, int32_t V) { return B >= 0 && K >= 0 && K <= SV_MAX_K && V >= 1; }
bool tree_sizes_ok(int32_t B, int32_t N, int32_t V) {
  return B >= 0 && N >= 1 && N <= SV_MAX_TREE_NODES && V >= 1;
}

bool aligned_to(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

sv_status from_hip(hipError_t e) { return e == hipSuccess ? SV_OK : SV_ERR_HIP; }

// Sampling verification of a tree: the run records of the B (N+1) target rows
// then of the B (N+1) draft rows.
bool tree_sampling_rows(int32_t B, int32_t N, int64_t* rows) {
  *rows = 2LL * B * (N + 1);
  return *rows <= INT32_MAX;
}

// Workspace of a sampling-tree call: the statistics records (nrec chunks of
// every target and draft row), then the walk's exchange slots (two per run of
// each sequence), counters and abort flag.
struct TreeSamplingLayout {
  int32_t nrun, nrec;
  size_t off_slots, off_cnt, off_abort, total;
};

TreeSamplingLayout tree_sampling_layout(int32_t B, int32_t N, int32_t V, sv_dtype d) {
  TreeSamplingLayout L{};
  const int64_t rows = 2LL * B * (N + 1);
  const int64_t nvec = row_vecs(V, d);
  L.nrun = static_cast<int32_t>(ceil_div(nvec, sv::kRunVecs));
  L.nrec = static_cast<int32_t>(ceil_div(nvec, row_chunk_vecs(1, static_cast<int32_t>(rows), V, d,
                                                              sv::kChunksTreeSample)));
  size_t off = align_up(sizeof(uint64_t) * rows * L.nrec);
  L.off_slots = off;
  off = align_up(off + sizeof(uint64_t) * 2 * static_cast<int64_t>(B) * L.nrun);
  L.off_cnt = off;
  off = align_up(off + sizeof(uint32_t) * (static_cast<int64_t>(B) + 2));
  L.off_abort = off;
  off = align_up(off + sizeof(uint64_t));
  L.total = off;
  return L;
}

// Walk workgroups per sequence: enough to spread the call's passes over the
// compute units (B G about the number of compute units), each with at least
// one run per wave, at most kMaxWalkGroups.
int32_t walk_groups(int32_t B, int32_t nrun) {
  const int cus = device_cus();
  if (cus < 1) return 1;
  const int64_t by_cus = cus / (B > 0 ? B : 1);
  const int64_t by_runs = ceil_div(nrun, 16);
  int64_t g = by_cus < by_runs ? by_cus : by_runs;
  if (g > sv::kMaxWalkGroups) g = sv::kMaxWalkGroups;
  return g < 1 ? 1 : static_cast<int32_t>(g);
}

thread_local sv::PassEvents g_pass_events{nullptr, nullptr};

}  // namespace

sv::PassEvents sv::take_pass_events() {
  const PassEvents e = g_pass_events;
  g_pass_events = PassEvents{nullptr, nullptr};
  return e;
}

extern "C" {

const char* sv_status_string(sv_status status) {
  switch (status) {
    case SV_OK:
      return "SV_OK";
    case SV_ERR_INVALID_ARGUMENT:
      return "SV_ERR_INVALID_ARGUMENT";
    case SV_ERR_UNSUPPORTED:
      return "SV_ERR_UNSUPPORTED";
    case SV_ERR_WORKSPACE:
      return "SV_ERR_WORKSPACE";
    case SV_ERR_HIP:
      return "SV_ERR_HIP";
  }
  return "SV_ERR_UNKNOWN";
}

size_t sv_chain_workspace_bytes(int32_t B, int32_t K, int32_t V, sv_dtype dtype) {
  if (!chain_sizes_ok(B, K, V) || !dtype_ok(dtype)) return 0;
  return chain_layout(B, K, V, dtype).total;
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- the chain call that allocates nothing
//
// sv_verify_chain_noalloc uses this array as its workspace: one copy per
// GPU, held until the process ends, shared by every such call on that GPU.
// Host code never uses the array's name as an address (on the host it is a
// stand-in, not device memory): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the array (SV_ERR_HIP if the runtime cannot
// give its address).
sv_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SV_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SV_OK;
}

// Zero n16 16-byte words at p (a kernel, not a memset node, so a caller may
// capture it in a graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, uint64_t n16) {
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256u + threadIdx.x; i < n16;
       i += static_cast<uint64_t>(gridDim.x) * 256u)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Zero the first `bytes` bytes (a multiple of 256, as every workspace
// layout's total is) of a 256-byte-aligned buffer on `stream`.
hipError_t zero_fill(void* buf, size_t bytes, hipStream_t stream) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const uint64_t blocks = (n16 + 255) / 256;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<uint32_t>(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                     stream, static_cast<uint4*>(buf), n16);
  return hipGetLastError();
}

// A chain verification call; draft-side sampling is the K = 0 case with the
// drawn token's probability requested.
sv_status chain_call(const void* target_logits, const void* draft_logits, sv_dtype dtype, const int32_t* draft_tokens,
                     const float* temperature, const float* uniforms, int32_t B, int32_t K, int32_t V,
                     int32_t* accept_len, int32_t* out_tokens, float* p_draft, float* q_draft, float* residual_mass,
                     float* entropy, float* drawn_prob, int32_t* err_flags, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, const sv::PassEvents& ev, bool zero_first = false) {
  if (!dtype_ok(dtype) || !chain_sizes_ok(B, K, V)) return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (target_logits == nullptr || uniforms == nullptr || out_tokens == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (K > 0 && (draft_logits == nullptr || draft_tokens == nullptr)) return SV_ERR_INVALID_ARGUMENT;
  const int eb = dtype_bytes(dtype);
  if (!aligned_to(target_logits, eb) || (draft_logits != nullptr && !aligned_to(draft_logits, eb)))
    return SV_ERR_INVALID_ARGUMENT;
  const ChainLayout L = chain_layout(B, K, V, dtype);
  if (workspace == nullptr || workspace_bytes < L.total || !aligned_to(workspace, 8)) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  sv::ChainParams p{};
  p.target = target_logits;
  p.draft = draft_logits;
  p.tokens = draft_tokens;
  p.temperature = temperature;
  p.uniforms = uniforms;
  p.B = B;
  p.K = K;
  p.V = V;
  // The chunked layout needs every row on a 16-byte boundary.
  const bool chunked = whole_vector_rows(V, dtype) && aligned_to(target_logits, 16) &&
                       (K == 0 || aligned_to(draft_logits, 16));
  p.L = piece_layout(2 * K + 1, V, dtype, chunked, chain_chunk_vecs(B, K, V, dtype));
  p.ntiles = L.ntiles;
  p.tiles_per_block = L.tiles_per_block;
  p.nblk_b = L.nblk_b;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  p.p_draft = p_draft;
  p.q_draft = q_draft;
  p.residual_mass = residual_mass;
  p.drawn_prob = drawn_prob;
  p.entropy = entropy;
  p.err_flags = err_flags;
  p.part_m = reinterpret_cast<uint64_t*>(ws + L.off_part_m);
  p.part_s = reinterpret_cast<uint64_t*>(ws + L.off_part_s);
  p.part_a = reinterpret_cast<uint64_t*>(ws + L.off_part_a);
  p.cnt = reinterpret_cast<uint32_t*>(ws + L.off_cnt);
  p.tile_sum = reinterpret_cast<uint64_t*>(ws + L.off_tiles);
  p.gat = reinterpret_cast<uint64_t*>(ws + L.off_gat);
  p.abort = reinterpret_cast<uint64_t*>(ws + L.off_abort);
  p.tk = reinterpret_cast<uint32_t*>(ws + L.off_tk);
  p.done = reinterpret_cast<uint32_t*>(ws + L.off_done);
  p.plan = reinterpret_cast<uint64_t*>(ws + L.off_plan);
  const bool extra = entropy != nullptr || drawn_prob != nullptr;
  p.one_launch = one_launch_ok(p.L, B, K, p.nblk_b, drawn_prob != nullptr) ? 1 : 0;
  if (chunked && small_ok(p.L, B, K, V, dtype, extra)) {
    p.one_launch = 2;
    const int64_t tpb = ceil_div(L.ntiles, p.L.cps);
    p.tiles_per_block = static_cast<int32_t>(tpb < sv::kSmallTiles ? sv::kSmallTiles : tpb);
  }

  if (static_cast<int64_t>(B) * (sv::items_per_seq(p.L) + p.nblk_b) > INT32_MAX)
    return SV_ERR_UNSUPPORTED;
  if (zero_first) {  // the part of the workspace this call uses, cleared on its stream first
    const hipError_t e = zero_fill(workspace, L.total, stream);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  return from_hip(sv::launch_chain(p, dtype, ev, stream));
}

// The form a chain call of this shape takes on the current device: 1 small
// (chain_small_kernel), 2 one launch with ticket queues
// (chain_one_launch_kernel), 3 two launches; 0 for invalid sizes or dtype
// or B = 0.
int32_t chain_form(int32_t B, int32_t K, int32_t V, sv_dtype dtype, int32_t rows_aligned, int32_t with_entropy) {
  if (!dtype_ok(dtype) || !chain_sizes_ok(B, K, V)) return 0;
  if (B == 0) return 0;
  const bool chunked = rows_aligned != 0 && whole_vector_rows(V, dtype);
  const sv::PieceLayout L = piece_layout(2 * K + 1, V, dtype, chunked, chain_chunk_vecs(B, K, V, dtype));
  if (chunked && small_ok(L, B, K, V, dtype, with_entropy != 0)) return 1;
  return one_launch_ok(L, B, K, chain_layout(B, K, V, dtype).nblk_b, false) ? 2 : 3;
}

}  // namespace

extern "C" {

int32_t sv_chain_launches(int32_t B, int32_t K, int32_t V, sv_dtype dtype, int32_t rows_aligned,
                          int32_t with_entropy) {
  if (!dtype_ok(dtype) || !chain_sizes_ok(B, K, V)) return 0;
  if (B == 0) return 0;
  const int32_t form = chain_form(B, K, V, dtype, rows_aligned, with_entropy);
  return form == 0 ? 0 : (form == 3 ? 2 : 1);
}

int32_t sv_chain_form(int32_t B, int32_t K, int32_t V, sv_dtype dtype, int32_t rows_aligned, int32_t with_entropy) {
  return chain_form(B, K, V, dtype, rows_aligned, with_entropy);
}

sv_status sv_verify_chain(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                          const int32_t* draft_tokens, const float* temperature, const float* uniforms,
                          int32_t B, int32_t K, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                          float* p_draft, float* q_draft, float* residual_mass, float* entropy,
                          int32_t* err_flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const sv::PassEvents ev = sv::take_pass_events();
  if (!dtype_ok(dtype) || !chain_sizes_ok(B, K, V)) return SV_ERR_INVALID_ARGUMENT;
  if (B > 0 && accept_len == nullptr) return SV_ERR_INVALID_ARGUMENT;
  return chain_call(target_logits, draft_logits, dtype, draft_tokens, temperature, uniforms, B, K, V, accept_len,
                    out_tokens, p_draft, q_draft, residual_mass, entropy, nullptr, err_flags, workspace,
                    workspace_bytes, stream, ev);
}

sv_status sv_verify_chain_noalloc(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                                  const int32_t* draft_tokens, const float* temperature, const float* uniforms,
                                  int32_t B, int32_t K, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                                  float* p_draft, float* q_draft, float* residual_mass, float* entropy,
                                  int32_t* err_flags, hipStream_t stream) {
  const sv::PassEvents ev = sv::take_pass_events();
  if (!dtype_ok(dtype) || !chain_sizes_ok(B, K, V)) return SV_ERR_INVALID_ARGUMENT;
  if (B > 0 && accept_len == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  const size_t need = chain_layout(B, K, V, dtype).total;
  if (need > static_cast<size_t>(SV_NOALLOC_SCRATCH_BYTES)) return SV_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const sv_status st = scratch_of_current_device(&ws);
  if (st != SV_OK) return st;
  return chain_call(target_logits, draft_logits, dtype, draft_tokens, temperature, uniforms, B, K, V, accept_len,
                    out_tokens, p_draft, q_draft, residual_mass, entropy, nullptr, err_flags, ws, need, stream, ev,
                    /*zero_first=*/true);
}

}  // extern "C"

namespace {

// The LM-head chain call: shapes it serves (bf16 only; H a multiple of 64,
// V of 8) and its workspace: the chain call's regions (slots for the
// whole-row layout), then the GEMM's statistics pieces.
bool lm_head_sizes_ok(int32_t B, int32_t K, int32_t V, int32_t H) {
  return chain_sizes_ok(B, K, V) && V >= 8 && V % 8 == 0 && H >= 64 && H % 64 == 0 &&
         static_cast<int64_t>(B) * (K + 1) <= INT32_MAX;
}

struct LMHeadLayout {
  ChainLayout chain;
  int32_t ntn;
  size_t off_pieces, total;
};

// One piece per row: every row a chunk of its own.
sv::PieceLayout lm_head_piece_layout(int32_t K, int32_t V) {
  return piece_layout(2 * K + 1, V, SV_DTYPE_BF16, true, row_vecs(V, SV_DTYPE_BF16));
}

LMHeadLayout lm_head_layout(int32_t B, int32_t K, int32_t V) {
  LMHeadLayout L{};
  L.chain = chain_layout(B, K, V, SV_DTYPE_BF16, B * sv::slots_per_seq(lm_head_piece_layout(K, V)));
  L.ntn = static_cast<int32_t>(ceil_div(V, sv::kLMPiece));
  L.off_pieces = L.chain.total;
  L.total = align_up(L.off_pieces + sizeof(float2) * static_cast<int64_t>(B) * (K + 1) * L.ntn);
  return L;
}

sv::LMHeadParams lm_head_params(const void* hidden, const void* weight, void* logits, int32_t M, int32_t N,
                                int32_t H, int32_t K1, const float* temperature) {
  sv::LMHeadParams g{};
  g.hidden = hidden;
  g.weight = weight;
  g.logits = logits;
  g.M = M;
  g.N = N;
  g.H = H;
  g.K1 = K1;
  g.temperature = temperature;
  g.npieces = static_cast<int32_t>(ceil_div(N, sv::kLMPiece));
  return g;
}

}  // namespace

extern "C" {

size_t sv_lm_head_chain_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t H) {
  if (!lm_head_sizes_ok(B, K, V, H)) return 0;
  return lm_head_layout(B, K, V).total;
}

sv_status sv_lm_head_logits(const void* hidden, const void* head_weight, int32_t M, int32_t H, int32_t V,
                            void* logits, hipStream_t stream) {
  const sv::PassEvents ev = sv::take_pass_events();
  if (M < 0 || !lm_head_sizes_ok(1, 0, V, H)) return SV_ERR_INVALID_ARGUMENT;
  if (M == 0) return SV_OK;
  if (hidden == nullptr || head_weight == nullptr || logits == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (!aligned_to(hidden, 16) || !aligned_to(head_weight, 16) || !aligned_to(logits, 16))
    return SV_ERR_INVALID_ARGUMENT;
  const sv::LMHeadParams g = lm_head_params(hidden, head_weight, logits, M, V, H, 1, nullptr);
  if (sv::lm_head_grid(g) > INT32_MAX) return SV_ERR_UNSUPPORTED;
  return from_hip(sv::launch_lm_head_gemm(g, false, ev, stream));
}

sv_status sv_verify_chain_lm_head(const void* hidden, const void* head_weight, int32_t H, void* target_logits,
                                  const void* draft_logits, const int32_t* draft_tokens, const float* temperature,
                                  const float* uniforms, int32_t B, int32_t K, int32_t V, int32_t* accept_len,
                                  int32_t* out_tokens, float* p_draft, float* q_draft, float* residual_mass,
                                  int32_t* err_flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const sv::PassEvents ev = sv::take_pass_events();
  if (!lm_head_sizes_ok(B, K, V, H)) return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (hidden == nullptr || head_weight == nullptr || target_logits == nullptr || uniforms == nullptr ||
      accept_len == nullptr || out_tokens == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  if (K > 0 && (draft_logits == nullptr || draft_tokens == nullptr)) return SV_ERR_INVALID_ARGUMENT;
  if (!aligned_to(hidden, 16) || !aligned_to(head_weight, 16) || !aligned_to(target_logits, 16) ||
      (K > 0 && !aligned_to(draft_logits, 16)))
    return SV_ERR_INVALID_ARGUMENT;
  const LMHeadLayout LL = lm_head_layout(B, K, V);
  if (workspace == nullptr || workspace_bytes < LL.total || !aligned_to(workspace, 8)) return SV_ERR_WORKSPACE;
  const int32_t M = B * (K + 1);
  char* ws = static_cast<char*>(workspace);
  sv::LMHeadParams g = lm_head_params(hidden, head_weight, target_logits, M, V, H, K + 1, temperature);
  g.pieces = reinterpret_cast<float2*>(ws + LL.off_pieces);  // the epilogue's statistics, [M, ntn]
  if (sv::lm_head_grid(g) > INT32_MAX) return SV_ERR_UNSUPPORTED;

  const ChainLayout& L = LL.chain;
  sv::ChainParams p{};
  p.target = target_logits;  // the GEMM's stored logits feed the gathers and the draw
  p.draft = draft_logits;
  p.tokens = draft_tokens;
  p.temperature = temperature;
  p.uniforms = uniforms;
  p.B = B;
  p.K = K;
  p.V = V;
  // one piece per row: the target rows' from the GEMM's pieces, the draft
  // rows' from one stream over each row
  p.L = lm_head_piece_layout(K, V);
  p.ntiles = L.ntiles;
  p.tiles_per_block = L.tiles_per_block;
  p.nblk_b = L.nblk_b;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  p.p_draft = p_draft;
  p.q_draft = q_draft;
  p.residual_mass = residual_mass;
  p.err_flags = err_flags;
  p.part_m = reinterpret_cast<uint64_t*>(ws + L.off_part_m);
  p.part_s = reinterpret_cast<uint64_t*>(ws + L.off_part_s);
  p.part_a = reinterpret_cast<uint64_t*>(ws + L.off_part_a);
  p.cnt = reinterpret_cast<uint32_t*>(ws + L.off_cnt);
  p.tile_sum = reinterpret_cast<uint64_t*>(ws + L.off_tiles);
  p.gat = reinterpret_cast<uint64_t*>(ws + L.off_gat);
  p.abort = reinterpret_cast<uint64_t*>(ws + L.off_abort);
  p.tk = reinterpret_cast<uint32_t*>(ws + L.off_tk);
  p.done = reinterpret_cast<uint32_t*>(ws + L.off_done);
  p.lm_pieces = reinterpret_cast<float2*>(ws + LL.off_pieces);
  p.lm_ntn = LL.ntn;
  if (static_cast<int64_t>(B) * K + (static_cast<int64_t>(M) + 3) / 4 > INT32_MAX ||
      static_cast<int64_t>(B) * p.nblk_b > INT32_MAX)
    return SV_ERR_UNSUPPORTED;
  return from_hip(sv::launch_chain_lm_head(g, p, ev, stream));
}

size_t sv_sample_workspace_bytes(int32_t R, int32_t V, sv_dtype dtype) {
  if (!chain_sizes_ok(R, 0, V) || !dtype_ok(dtype)) return 0;
  // rows on 16-byte boundaries use the segment records, others the chain
  // workspace of R sequences with K = 0; both start at offset 0
  const size_t chain = chain_layout(R, 0, V, dtype).total;
  const size_t segs = whole_vector_rows(V, dtype) ? sample_layout(R, V, dtype).total : 0;
  return chain > segs ? chain : segs;
}

sv_status sv_sample_rows(const void* logits, sv_dtype dtype, const float* temperature, const float* uniforms,
                         int32_t R, int32_t V, int32_t* out_tokens, float* out_prob, int32_t* err_flags,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const sv::PassEvents ev = sv::take_pass_events();
  if (!dtype_ok(dtype) || !chain_sizes_ok(R, 0, V)) return SV_ERR_INVALID_ARGUMENT;
  if (R == 0) return SV_OK;
  if (logits == nullptr || uniforms == nullptr || out_tokens == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (workspace == nullptr || workspace_bytes < sv_sample_workspace_bytes(R, V, dtype) || !aligned_to(workspace, 8))
    return SV_ERR_WORKSPACE;
  if (!aligned_to(logits, dtype_bytes(dtype))) return SV_ERR_INVALID_ARGUMENT;
  if (!whole_vector_rows(V, dtype) || !aligned_to(logits, 16))  // rows off 16-byte boundaries: two passes
    return chain_call(logits, nullptr, dtype, nullptr, temperature, uniforms, R, 0, V, nullptr, out_tokens, nullptr,
                      nullptr, nullptr, nullptr, out_prob, err_flags, workspace, workspace_bytes, stream, ev);
  const SampleLayout L = sample_layout(R, V, dtype);
  if (static_cast<int64_t>(R) * L.upr > INT32_MAX || static_cast<int64_t>(R) * L.nrec > INT32_MAX)
    return SV_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  sv::SampleParams p{};
  p.logits = logits;
  p.temperature = temperature;
  p.uniforms = uniforms;
  p.R = R;
  p.V = V;
  p.nvec = row_vecs(V, dtype);
  p.upr = L.upr;
  p.nrec = L.nrec;
  p.ngroups = L.ngroups;
  p.wpg = L.wpg;
  p.out_tokens = out_tokens;
  p.out_prob = out_prob;
  p.err_flags = err_flags;
  p.rec_m = reinterpret_cast<uint64_t*>(ws + L.off_m);
  p.rec_s = reinterpret_cast<uint64_t*>(ws + L.off_s);
  p.take = reinterpret_cast<uint32_t*>(ws + L.off_take);
  return from_hip(sv::launch_sample(p, dtype, ev, stream));
}

size_t sv_tree_workspace_bytes(int32_t B, int32_t N, int32_t V, sv_dtype dtype) {
  if (!tree_sizes_ok(B, N, V) || !dtype_ok(dtype)) return 0;
  return tree_layout(B, N, V, dtype).total;
}

sv_status sv_verify_tree_greedy(const void* target_logits, sv_dtype dtype, const int32_t* node_tokens,
                                const int32_t* parents, int32_t B, int32_t N, int32_t V, int32_t* accept_len,
                                int32_t* path_nodes, int32_t* next_token, int32_t* err_flags, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  const sv::PassEvents ev = sv::take_pass_events();
  if (!dtype_ok(dtype) || !tree_sizes_ok(B, N, V)) return SV_ERR_INVALID_ARGUMENT;
  if (B == 0) return SV_OK;
  if (target_logits == nullptr || node_tokens == nullptr || parents == nullptr || accept_len == nullptr ||
      path_nodes == nullptr || next_token == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  if (!aligned_to(target_logits, dtype_bytes(dtype))) return SV_ERR_INVALID_ARGUMENT;
  const TreeLayout L = tree_layout(B, N, V, dtype);
  if (workspace == nullptr || workspace_bytes < L.total || !aligned_to(workspace, 8)) return SV_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  sv::TreeParams p{};
  p.target = target_logits;
  p.tokens = node_tokens;
  p.parents = parents;
  p.B = B;
  p.N = N;
  p.V = V;
  p.L = piece_layout(N + 1, V, dtype, whole_vector_rows(V, dtype) && aligned_to(target_logits, 16),
                     row_chunk_vecs(B, N + 1, V, dtype, sv::kChunksTree));
  if (static_cast<int64_t>(B) * sv::items_per_seq(p.L) > INT32_MAX) return SV_ERR_UNSUPPORTED;
  p.accept_len = accept_len;
  p.path_nodes = path_nodes;
  p.next_token = next_token;
  p.err_flags = err_flags;
  p.part = reinterpret_cast<uint64_t*>(ws + L.off_part);
  return from_hip(sv::launch_tree(p, dtype, ev, stream));
}

size_t sv_tree_sampling_workspace_bytes(int32_t B, int32_t N, int32_t V, sv_dtype dtype) {
  int64_t rows = 0;
  if (!tree_sizes_ok(B, N, V) || !dtype_ok(dtype) || !tree_sampling_rows(B, N, &rows)) return 0;
  return tree_sampling_layout(B, N, V, dtype).total;
}

sv_status sv_verify_tree_sampling(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                                  const int32_t* node_tokens, const int32_t* parents, const float* temperature,
                                  const float* uniforms, int32_t B, int32_t N, int32_t V, int32_t* accept_len,
                                  int32_t* path_nodes, int32_t* next_token, int32_t* err_flags, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  const sv::PassEvents ev = sv::take_pass_events();
  int64_t rows = 0;
  if (!dtype_ok(dtype) || !tree_sizes_ok(B, N, V)) return SV_ERR_INVALID_ARGUMENT;
  if (!tree_sampling_rows(B, N, &rows)) return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (target_logits == nullptr || draft_logits == nullptr || node_tokens == nullptr || parents == nullptr ||
      uniforms == nullptr || accept_len == nullptr || path_nodes == nullptr || next_token == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  if (!aligned_to(target_logits, dtype_bytes(dtype)) || !aligned_to(draft_logits, dtype_bytes(dtype)))
    return SV_ERR_INVALID_ARGUMENT;
  const TreeSamplingLayout TL = tree_sampling_layout(B, N, V, dtype);
  if (workspace == nullptr || workspace_bytes < TL.total || !aligned_to(workspace, 8)) return SV_ERR_WORKSPACE;
  // the walk reads rows as 16-byte vectors and keeps one total per run in LDS
  if (!whole_vector_rows(V, dtype) || !aligned_to(target_logits, 16) || !aligned_to(draft_logits, 16) ||
      TL.nrun > sv::kMaxWalkRuns || rows * TL.nrec > INT32_MAX)
    return SV_ERR_UNSUPPORTED;

  sv::TreeSampleParams p{};
  p.target = target_logits;
  p.draft = draft_logits;
  p.tokens = node_tokens;
  p.parents = parents;
  p.temperature = temperature;
  p.uniforms = uniforms;
  p.B = B;
  p.N = N;
  p.V = V;
  p.nvec = row_vecs(V, dtype);
  p.nrun = TL.nrun;
  p.nrec = TL.nrec;
  p.rec = static_cast<uint64_t*>(workspace);
  p.accept_len = accept_len;
  p.path_nodes = path_nodes;
  p.next_token = next_token;
  p.err_flags = err_flags;
  char* ws = static_cast<char*>(workspace);
  p.G = walk_groups(B, TL.nrun);
  if (static_cast<int64_t>(B) * p.G > INT32_MAX) p.G = 1;
  p.slots = reinterpret_cast<uint64_t*>(ws + TL.off_slots);
  p.cnt = reinterpret_cast<uint32_t*>(ws + TL.off_cnt);
  p.abort = reinterpret_cast<uint64_t*>(ws + TL.off_abort);
  return from_hip(sv::launch_tree_sample(p, dtype, ev, stream));
}

sv_status sv_time_next_stream_pass(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr)) return SV_ERR_INVALID_ARGUMENT;
  g_pass_events = sv::PassEvents{before, after};
  return SV_OK;
}

sv_status sv_build_tree_mask(const int32_t* parents, int32_t N, uint8_t* mask, int32_t* err_flags,
                             hipStream_t stream) {
  if (N < 1 || N > SV_MAX_TREE_NODES || parents == nullptr || mask == nullptr) return SV_ERR_INVALID_ARGUMENT;
  return from_hip(sv::launch_tree_mask(parents, N, mask, err_flags, stream));
}

}  // extern "C"
