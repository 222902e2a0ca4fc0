// Greedy tree verification and the tree ancestor mask.
//
// tree_argmax_kernel, one workgroup per streaming item (a chunk of a
// sequence's N+1 rows laid end to end, or a segment of one row): streams the
// logits with 16-byte loads and keeps, per thread, the largest value and its
// lowest index (a batch is scanned for its first maximum only when it beats
// the running one). The block combines (value desc, index asc) and publishes
// one slot per row piece.
//
// tree_decide_kernel, one workgroup per sequence: combines the pieces into
// g[n] = argmax of every position and resolves the tree: node i is accepted
// iff its token equals g at its parent's position and its parent is
// accepted; acceptance and depth are propagated up the parent links by
// pointer jumping (log2(depth) rounds); the deepest accepted node (lowest
// index on ties) ends the path, and g at its position is the next token.
// [Topologies] "Speculative Decoding & Draft Model Topologies", section 4
// figure (all tree nodes checked in one pass, the longest accepted path kept);
// [In Production] "Speculative Decoding in Production", section 4;
// [At Scale] "Speculative Decoding at Scale", sequence diagram (matching
// proposals are kept, the target adds its own next token).
//
// tree_mask_kernel, one workgroup per node i: marks i and its ancestors in an
// LDS bitmap by walking the parent links, then writes row i of the mask.
// [Topologies] section 4 figure (2D tree-masked attention); [In Production]
// section 4 (custom 2D causal mask).
#include <limits.h>
#include <math.h>

#include <hip/hip_ext.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

// (value, index) with "better" = larger value, then smaller index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(i, o, kWave);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ void block_argmax(float& v, int& i, float* sv, int* si) {
  wave_argmax(v, i);
  if (lane_id() == 0) {
    sv[wave_id()] = v;
    si[wave_id()] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    if (better(sv[w], si[w], v, i)) {
      v = sv[w];
      i = si[w];
    }
  }
  __syncthreads();
}

__device__ void tree_decide(const TreeParams& P, int b) {
  __shared__ int s_g[SV_MAX_TREE_NODES + 1];
  __shared__ int s_par[SV_MAX_TREE_NODES];
  __shared__ int s_anc[2][SV_MAX_TREE_NODES];
  __shared__ int s_dep[2][SV_MAX_TREE_NODES];
  __shared__ unsigned char s_ok[2][SV_MAX_TREE_NODES];
  __shared__ uint32_t s_err;
  __shared__ int s_red[kWaves];
  const int N = P.N;
  const int N1 = N + 1;
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0u;
  __syncthreads();

  // g[n]: combine the pieces of every position (written by the argmax launch).
  const int pmax = max_pieces(P.L);
  for (int n = tid; n < N1; n += kThreads) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    uint32_t err = 0u;
    for (int p = 0; p < pmax; ++p) {
      const int64_t s = piece_slot(P.L, b, n, p);
      if (s < 0) break;
      const uint64_t slot = load_ready(&P.part[s], &err);
      const float v = __uint_as_float(static_cast<uint32_t>(slot >> 32));
      const int i = static_cast<int>(static_cast<uint32_t>(slot) - 1u);
      if (better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
    s_g[n] = (bi == INT_MAX) ? 0 : bi;  // a row of -inf only: its first index
    if (err != 0u) atomicOr(&s_err, err);
  }
  __syncthreads();

  // Node i: validity, match with its parent's argmax, first jump.
  for (int i = tid; i < N; i += kThreads) {
    const int par = P.parents[i];
    const int tok = P.tokens[static_cast<int64_t>(b) * N + i];
    uint32_t err = 0u;
    const bool par_ok = (par == -1) || (par >= 0 && par < i);
    if (!par_ok) err |= SV_ERRF_PARENT;
    if (tok < 0 || tok >= P.V) err |= SV_ERRF_TOKEN;
    if (err != 0u) atomicOr(&s_err, err);
    const int pos = (par_ok && par >= 0) ? par + 1 : 0;
    s_par[i] = par_ok ? par : -1;
    s_anc[0][i] = par_ok ? par : -1;
    s_ok[0][i] = (par_ok && tok == s_g[pos]) ? 1 : 0;
    s_dep[0][i] = 1;
  }
  __syncthreads();

  // Pointer jumping. Invariant: the segment from i up to (not including)
  // anc[i] has dep[i] nodes, and ok[i] is the AND of their matches. With 11
  // rounds the jump length 2^11 exceeds any depth <= SV_MAX_TREE_NODES.
  int cur = 0;
  for (int round = 0; round < 11; ++round) {
    const int nxt = cur ^ 1;
    for (int i = tid; i < N; i += kThreads) {
      const int a = s_anc[cur][i];
      if (a >= 0) {
        s_ok[nxt][i] = s_ok[cur][i] & s_ok[cur][a];
        s_dep[nxt][i] = s_dep[cur][i] + s_dep[cur][a];
        s_anc[nxt][i] = s_anc[cur][a];
      } else {
        s_ok[nxt][i] = s_ok[cur][i];
        s_dep[nxt][i] = s_dep[cur][i];
        s_anc[nxt][i] = -1;
      }
    }
    __syncthreads();
    cur = nxt;
  }

  // Deepest accepted node, lowest index on ties: max of (depth, 2047 - i).
  int key = -1;
  for (int i = tid; i < N; i += kThreads)
    if (s_ok[cur][i]) key = max(key, (s_dep[cur][i] << 11) | (2047 - i));
  key = block_max_int(key, s_red);
  const int best = key < 0 ? -1 : 2047 - (key & 2047);
  const int depth = key < 0 ? 0 : (key >> 11);
  const bool bad = s_err != 0u;

  // Path from the root side, built in LDS (reusing the jump buffer).
  int* s_path = s_anc[cur ^ 1];
  if (tid == 0 && !bad) {
    int k = best;
    for (int d = depth - 1; d >= 0 && k >= 0; --d) {
      s_path[d] = k;
      k = s_par[k];
    }
  }
  __syncthreads();
  for (int i = tid; i < N; i += kThreads)
    P.path_nodes[static_cast<int64_t>(b) * N + i] = (!bad && i < depth) ? s_path[i] : -1;
  if (tid == 0) {
    P.accept_len[b] = bad ? -1 : depth;
    P.next_token[b] = bad ? -1 : s_g[best + 1];
    raise_error(P.err_flags, s_err);
  }
  // Consumed: the sequence's pieces go back to zero for the next call.
  const int64_t per_seq = slots_per_seq(P.L);
  for (int64_t s = static_cast<int64_t>(b) * per_seq + tid; s < (static_cast<int64_t>(b) + 1) * per_seq; s += kThreads)
    P.part[s] = 0ull;
}

// Trees of at most kWave nodes: the same decision made by one wave, one node
// per lane, with cross-lane shuffles instead of LDS and block barriers.
// Lane n also holds g at position n (lane 0 holds position 64 as well when
// N = 64); pointer jumping takes 6 rounds (2^6 = 64 >= any depth); the path
// is read off by walking up from the deepest accepted node.
__device__ void tree_decide_wave(const TreeParams& P, int b) {
  const int N = P.N;
  const int N1 = N + 1;
  const int lane = lane_id();
  uint32_t err = 0u;

  // g at positions lane and (lane 0 only) 64
  const int pmax = max_pieces(P.L);
  int g = 0, g64 = 0;
  for (int rep = 0; rep < 2; ++rep) {
    const int n = rep == 0 ? lane : kWave;
    if (n >= N1 || (rep == 1 && lane != 0)) continue;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int p = 0; p < pmax; ++p) {
      const int64_t sl = piece_slot(P.L, b, n, p);
      if (sl < 0) break;
      const uint64_t slot = load_ready(&P.part[sl], &err);
      const float v = __uint_as_float(static_cast<uint32_t>(slot >> 32));
      const int i = static_cast<int>(static_cast<uint32_t>(slot) - 1u);
      if (better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
    const int gi = (bi == INT_MAX) ? 0 : bi;  // a row of -inf only: its first index
    if (rep == 0) g = gi; else g64 = gi;
  }

  // node `lane`: validity, match with its parent's argmax (every shuffle
  // below is taken by the whole wave)
  const bool node = lane < N;
  int par = -1, tok = -1;
  bool par_ok = true;
  if (node) {
    par = P.parents[lane];
    tok = P.tokens[static_cast<int64_t>(b) * N + lane];
    par_ok = (par == -1) || (par >= 0 && par < lane);
    if (!par_ok) err |= SV_ERRF_PARENT;
    if (tok < 0 || tok >= P.V) err |= SV_ERRF_TOKEN;
    if (!par_ok) par = -1;
  }
  const int pos = par >= 0 ? par + 1 : 0;  // <= lane < 64: held by lane `pos`
  const int want = __shfl(g, pos, kWave);
  bool ok = node && par_ok && tok == want;
  // Pointer jumping: anc = first ancestor not yet folded in, dep = nodes
  // from this one up to (not including) anc, ok = AND of their matches.
  int anc = par, dep = 1;
#pragma unroll
  for (int round = 0; round < 6; ++round) {
    const int a = anc >= 0 ? anc : lane;
    const int ok_a = __shfl(static_cast<int>(ok), a, kWave);
    const int dep_a = __shfl(dep, a, kWave);
    const int anc_a = __shfl(anc, a, kWave);
    if (anc >= 0) {
      ok = ok && ok_a != 0;
      dep += dep_a;
      anc = anc_a;
    }
  }
  // deepest accepted node, lowest index on ties: max of (depth, 2047 - i)
  int key = (node && ok) ? ((dep << 11) | (2047 - lane)) : -1;
  key = wave_max_int(key);
  const int best = key < 0 ? -1 : 2047 - (key & 2047);
  const int depth = key < 0 ? 0 : (key >> 11);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) err |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(err), o, kWave));
  const bool bad = err != 0u;

  // the path, root side first: walk up from `best`, lane d keeps the node at depth d + 1
  int mine = -1;
  int k = best;
  for (int d = depth - 1; d >= 0; --d) {
    if (lane == d) mine = k;
    k = __shfl(par, k, kWave);  // k is the same in every lane
  }
  for (int i = lane; i < N; i += kWave)
    P.path_nodes[static_cast<int64_t>(b) * N + i] = (!bad && i < depth) ? mine : -1;
  const int npos = best + 1;  // the position after the accepted path
  const int g_next = npos < kWave ? __shfl(g, npos, kWave) : __shfl(g64, 0, kWave);
  if (lane == 0) {
    P.accept_len[b] = bad ? -1 : depth;
    P.next_token[b] = bad ? -1 : g_next;
    raise_error(P.err_flags, err);
  }
  // Consumed: the sequence's pieces go back to zero for the next call.
  const int64_t per_seq = slots_per_seq(P.L);
  for (int64_t sl = static_cast<int64_t>(b) * per_seq + lane; sl < (static_cast<int64_t>(b) + 1) * per_seq; sl += kWave)
    P.part[sl] = 0ull;
}

// One thread's share of the vectors [p0, p1) of a row (16-byte aligned body):
// full batches of kStatsUnroll vectors per thread without masking, then one
// ragged batch padded with -inf. Each thread sees its elements in ascending
// index order, so a strict '>' keeps the first occurrence of its maximum.
template <class T>
__device__ __forceinline__ void piece_argmax(const uint4* body, int64_t p0, int64_t p1, float& bv, int& bi) {
  constexpr int U = kStatsUnroll;
  constexpr int VEC = T::kVec;
  constexpr int64_t STEP = static_cast<int64_t>(kThreads) * U;
  const int64_t nfull = (p1 - p0) / STEP;
  const int64_t rest = (p1 - p0) - nfull * STEP;
  int64_t v = p0 + threadIdx.x;  // this thread's first vector of the batch
#pragma unroll 1
  for (int64_t i = 0; i <= nfull; ++i, v += STEP) {
    uint4 raw[U];
    if (i < nfull) {
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = stream_load(body + v + u * kThreads);
    } else {
      if (rest == 0) break;
#pragma unroll
      for (int u = 0; u < U; ++u)
        raw[u] = (u * kThreads + static_cast<int64_t>(threadIdx.x) < rest)
                     ? stream_load(body + v + u * kThreads)
                     : neg_inf_vec<T>();
    }
    float x[U * VEC];
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unpack<T>(raw[u], &x[u * VEC]);
#pragma unroll
      for (int k = 0; k < VEC; ++k) bm = fmaxf(bm, x[u * VEC + k]);
    }
    if (bm > bv) {
      int first = 0;
#pragma unroll
      for (int q = U * VEC - 1; q >= 0; --q)
        if (x[q] == bm) first = q;
      bv = bm;
      bi = static_cast<int>((v + (first / VEC) * kThreads) * VEC + (first % VEC));
    }
  }
}

__device__ __forceinline__ uint64_t pack_argmax(float v, int i) {
  return (static_cast<uint64_t>(__float_as_uint(v)) << 32) | static_cast<uint32_t>(i + 1);
}

// Chunked layout: chunk ch of sequence b, one slot per row piece.
template <class T>
__device__ void tree_chunk(const TreeParams& P, int b, int ch) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  const int64_t nvec = P.L.nvec;
  const int64_t lo = static_cast<int64_t>(ch) * P.L.per;
  const int64_t hi = min(static_cast<int64_t>(P.L.rows) * nvec, lo + P.L.per);
  const int r_lo = static_cast<int>(lo / nvec);
  const int r_hi = static_cast<int>((hi - 1) / nvec);
  for (int r = r_lo; r <= r_hi; ++r) {
    const int64_t p0 = max(lo, r * nvec) - r * nvec;
    const int64_t p1 = min(hi, (r + 1) * nvec) - r * nvec;
    const uint4* body = reinterpret_cast<const uint4*>(static_cast<const char*>(P.target) +
                                                       (static_cast<int64_t>(b) * P.L.rows + r) * nvec * 16);
    float bv = -INFINITY;
    int bi = INT_MAX;
    piece_argmax<T>(body, p0, p1, bv, bi);
    block_argmax(bv, bi, s_v, s_i);
    if (threadIdx.x == 0)
      P.part[(static_cast<int64_t>(b) * P.L.cps + ch) * P.L.kmax + (r - r_lo)] = pack_argmax(bv, bi);
  }
}

// Segments layout: segment seg of row r of sequence b (any alignment).
template <class T>
__device__ void tree_segment(const TreeParams& P, int b, int r, int seg) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  constexpr int VEC = T::kVec;
  const int tid = threadIdx.x;
  const void* row = static_cast<const char*>(P.target) + (static_cast<int64_t>(b) * P.L.rows + r) *
                                                             static_cast<int64_t>(P.V) * T::kBytes;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  const int head = min(static_cast<int>(((16u - (addr & 15u)) & 15u) / T::kBytes), P.V);
  const int64_t nvec = (P.V - head) / VEC;
  const int tail = static_cast<int>((P.V - head) - nvec * VEC);
  const int64_t v0 = static_cast<int64_t>(seg) * P.L.seg_vecs;
  const int64_t v1 = min(nvec, v0 + P.L.seg_vecs);
  const uint4* body = reinterpret_cast<const uint4*>(static_cast<const char*>(row) + head * T::kBytes);
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (seg == 0 && tid < head) {
    const float x = load_elem<T>(row, tid);
    if (x > bv) {
      bv = x;
      bi = tid;
    }
  }
  if (v1 > v0) {
    float pv = -INFINITY;
    int pi = INT_MAX;
    piece_argmax<T>(body, v0, v1, pv, pi);
    if (pv > bv) {  // body elements come after the head
      bv = pv;
      bi = head + pi;
    }
  }
  if (seg == P.L.nseg - 1 && tid < tail) {
    const int idx = static_cast<int>(head + nvec * VEC + tid);
    const float x = load_elem<T>(row, idx);
    if (x > bv) {
      bv = x;
      bi = idx;
    }
  }
  block_argmax(bv, bi, s_v, s_i);
  if (tid == 0) P.part[(static_cast<int64_t>(b) * P.L.rows + r) * P.L.nseg + seg] = pack_argmax(bv, bi);
}

}  // namespace

template <class T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void tree_argmax_kernel(TreeParams P) {
  const int64_t per_seq = items_per_seq(P.L);
  const int64_t k = blockIdx.x;
  const int b = static_cast<int>(k / per_seq);
  const int rem = static_cast<int>(k % per_seq);
  if (P.L.cps > 0)
    tree_chunk<T>(P, b, rem);
  else
    tree_segment<T>(P, b, rem / P.L.nseg, rem % P.L.nseg);
}

__global__ __launch_bounds__(kThreads) void tree_decide_kernel(TreeParams P) { tree_decide(P, blockIdx.x); }

// Trees of at most 64 nodes: one wave per sequence.
__global__ __launch_bounds__(kWave) void tree_decide_wave_kernel(TreeParams P) { tree_decide_wave(P, blockIdx.x); }

__global__ __launch_bounds__(kThreads) void tree_mask_kernel(const int32_t* parents, int N, uint8_t* mask,
                                                             int32_t* err_flags) {
  __shared__ uint32_t s_bits[SV_MAX_TREE_NODES / 32];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  for (int w = tid; w < SV_MAX_TREE_NODES / 32; w += kThreads) s_bits[w] = 0u;
  __syncthreads();
  if (tid == 0) {
    // parent indices strictly decrease along a valid chain, so the walk ends
    int k = i;
    uint32_t err = 0u;
    while (k >= 0) {
      s_bits[k >> 5] |= 1u << (k & 31);
      const int p = parents[k];
      if (p != -1 && (p < 0 || p >= k)) {
        err = SV_ERRF_PARENT;
        break;
      }
      k = p;
    }
    raise_error(err_flags, err);
  }
  __syncthreads();
  uint8_t* out = mask + static_cast<int64_t>(i) * N;
  for (int j = tid; j < N; j += kThreads) out[j] = static_cast<uint8_t>((s_bits[j >> 5] >> (j & 31)) & 1u);
}

template <class T>
static hipError_t launch_tree_t(const TreeParams& p, const PassEvents& ev, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(p.B) * items_per_seq(p.L);
  if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
  // Armed events take the argmax kernel's own start and end timestamps.
  launch_stream_pass(tree_argmax_kernel<T>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), stream, ev, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.N <= kWave)
    hipLaunchKernelGGL(tree_decide_wave_kernel, dim3(static_cast<uint32_t>(p.B)), dim3(kWave), 0, stream, p);
  else
    hipLaunchKernelGGL(tree_decide_kernel, dim3(static_cast<uint32_t>(p.B)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_tree(const TreeParams& p, sv_dtype dtype, const PassEvents& ev, hipStream_t stream) {
  return dtype == SV_DTYPE_BF16 ? launch_tree_t<BF16>(p, ev, stream) : launch_tree_t<F32>(p, ev, stream);
}

hipError_t launch_tree_mask(const int32_t* parents, int32_t N, uint8_t* mask, int32_t* err_flags,
                            hipStream_t stream) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(static_cast<uint32_t>(N)), dim3(kThreads), 0, stream, parents, N,
                     mask, err_flags);
  return hipGetLastError();
}

}  // namespace sv
