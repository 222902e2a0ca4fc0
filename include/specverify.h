/*
 * specverify — the verification step of speculative sampling on AMD Instinct
 * MI355X (gfx950), as a C ABI.
 *
 * A speculative-decoding iteration has a small draft model propose K tokens,
 * the target model score all of them in one pass, and a verification step
 * decide which proposals to keep. This library is that verification step:
 *
 *   sv_verify_chain        modified rejection sampling over a chain of K
 *                          proposals, with the residual resample at the first
 *                          rejection or a bonus token when all K are kept;
 *   sv_verify_tree_greedy  greedy (argmax-matching) verification of a
 *                          candidate tree given as a parent array;
 *   sv_build_tree_mask     the tree's ancestor ("2D tree attention") mask.
 *
 * Sources, cited by page title and section:
 *   [Topologies]       "Speculative Decoding & Draft Model Topologies: Slashing
 *                      Enterprise LLM Latency by 3.5x in 2026" — section 2
 *                      (acceptance probability, residual distribution, timeline
 *                      figure) and section 4 (EAGLE-2 tree figure).
 *   [Draft-and-Verify] "Speculative Decoding for LLM Inference: How
 *                      Draft-and-Verify Accelerates Token Generation" — "The
 *                      draft-and-verify loop", "The correctness guarantee".
 *   [At Scale]         "Speculative Decoding at Scale: Latency Reduction in
 *                      Distributed LLM Serving" — sequence diagram, section 1.
 *   [In Production]    "Speculative Decoding in Production: How Small Draft
 *                      Models & Medusa Heads Deliver 2x–3x LLM Speedups Without
 *                      Accuracy Loss" — section 2 (acceptance rules) and
 *                      section 4 (tree verification, custom 2D masks).
 *
 * Conventions shared by every call:
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or keeps them.
 *   - Calls are stream-ordered and asynchronous: they enqueue kernels on
 *     `stream` and return; outputs are valid once the caller has synchronised
 *     that stream. No call synchronises the host.
 *   - Argument errors (sizes, NULL pointers, dtype, workspace too small,
 *     misaligned logits) are returned synchronously and nothing is launched.
 *     A failed launch returns SV_ERR_HIP.
 *   - Data errors can only be seen on the device. They are OR-ed into
 *     `*err_flags` (when it is not NULL; the caller clears it) as SV_ERRF_*
 *     bits, and the affected sequence reports accept_len = -1 with every
 *     output token -1.
 *   - Logit tensors are dense row-major with rows of V elements; bf16 is the
 *     upper half of an IEEE binary32 (the PyTorch bfloat16 layout). NaN logits
 *     are outside the contract.
 *   - A workspace belongs to one call at a time: two calls that overlap in
 *     time (different streams, or different host threads) need two workspaces.
 */
#ifndef SPECVERIFY_H_
#define SPECVERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream and event handles (identical to its own declarations). */
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

/* In C++ both enums have int as their fixed underlying type, so every int a
 * C caller passes (an unknown status code, a bad dtype) is a valid value of
 * the type; the size and calling convention are those of int either way. */
#ifdef __cplusplus
#define SV_ENUM_INT : int
#else
#define SV_ENUM_INT
#endif

typedef enum sv_status SV_ENUM_INT {
  SV_OK = 0,
  SV_ERR_INVALID_ARGUMENT = 1, /* a size, pointer or alignment is invalid      */
  SV_ERR_UNSUPPORTED = 2,      /* valid but beyond this build's limits         */
  SV_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than required      */
  SV_ERR_HIP = 4               /* the HIP runtime refused the launch           */
} sv_status;

typedef enum sv_dtype SV_ENUM_INT {
  SV_DTYPE_F32 = 0, /* IEEE binary32 logits                                 */
  SV_DTYPE_BF16 = 1 /* bfloat16 logits (16 high bits of a binary32)          */
} sv_dtype;

/* Data-error bits written to *err_flags. */
#define SV_ERRF_TOKEN 0x1u       /* a draft / node token outside [0, V)          */
#define SV_ERRF_TEMPERATURE 0x2u /* a temperature <= 0, NaN or infinite          */
#define SV_ERRF_PARENT 0x4u      /* parents[i] is neither -1 nor in [0, i)       */
#define SV_ERRF_NONFINITE 0x8u   /* a row's maximum is +inf, or its normaliser    \
                                    is 0 / not finite                            */
#define SV_ERRF_INTERNAL 0x10u   /* a partial result never became visible to the  \
                                    block combining them within the bounded wait \
                                    (should not happen); the workspace then has  \
                                    to be zero-filled again                      */

#define SV_MAX_K 63           /* drafted tokens per sequence (K+1 fits a wave64) */
#define SV_MAX_TREE_NODES 1024 /* candidate-tree nodes per call                  */

/* Human-readable name of a status code (static storage, never NULL). */
const char* sv_status_string(sv_status status);

/* ------------------------------------------------------------------------
 * Chain verification.
 *
 * Bytes of device workspace sv_verify_chain needs for (B, K, V, dtype); 0 for
 * invalid sizes. The workspace must be zero-filled once before its first use
 * (e.g. hipMemset or torch.zeros). Every call that returns SV_OK leaves the
 * whole workspace zero again once its kernels have run, so one workspace can
 * serve any sequence of calls (of any shape, chain or tree) on one stream.
 * After a call that returned an error, or whose kernels raised
 * SV_ERRF_INTERNAL, zero-fill it again.
 */
size_t sv_chain_workspace_bytes(int32_t B, int32_t K, int32_t V, sv_dtype dtype);

/*
 * One verification step of chain speculative sampling for B independent
 * sequences. For sequence b, with T = temperature[b]:
 *
 *   p_k = softmax(target_logits[b,k,:] / T),  k = 0..K      ([Draft-and-Verify]
 *   q_k = softmax(draft_logits[b,k,:] / T),   k = 0..K-1     "draft-and-verify loop")
 *   x_k = draft_tokens[b,k];  alpha_k = min(1, p_k(x_k) / q_k(x_k))
 *       (alpha_k = 0 if p_k(x_k) = 0; = 1 if q_k(x_k) = 0 < p_k(x_k))
 *   proposal k is kept iff uniforms[b,k] < alpha_k, checked in order; the
 *   first rejected k is j (j = K when all are kept)  ([Topologies] section 2;
 *                                                      [In Production] section 2)
 *   if j < K: one token drawn from max(0, p_j - q_j) / sum(max(0, p_j - q_j))
 *             ([Topologies] residual equation; [At Scale] section 1);
 *             if that sum is 0 in the device's arithmetic, from p_j;
 *   if j = K: one bonus token drawn from p_K ([Draft-and-Verify] loop);
 *   the draw uses uniforms[b,K] and the inverse CDF in ascending token id:
 *   the first t whose cumulative weight exceeds uniforms[b,K] * total.
 *
 * Arguments (device pointers unless noted):
 *   target_logits  [B, K+1, V] dtype, row-major, element-aligned (read only)
 *   draft_logits   [B, K, V] dtype, same V (draft and target share one
 *                  vocabulary); may be NULL when K = 0 (read only)
 *   dtype          SV_DTYPE_F32 or SV_DTYPE_BF16, for both logit tensors
 *   draft_tokens   [B, K] int32, each in [0, V); may be NULL when K = 0
 *   temperature    [B] float32, each > 0 and finite; NULL means 1.0 for all
 *   uniforms       [B, K+1] float32 in [0, 1): columns 0..K-1 for the accept
 *                  tests, column K for the replacement / bonus draw
 *   B, K, V        host ints: 0 <= B, 0 <= K <= SV_MAX_K, 1 <= V
 *   accept_len     [B] int32 out: j (0..K), or -1 on a data error
 *   out_tokens     [B, K+1] int32 out: x_0..x_{j-1}, then the drawn token,
 *                  then -1 up to column K (1..K+1 tokens per sequence)
 *   p_draft        [B, K] float32 out or NULL: p_k(x_k) for every k < K
 *   q_draft        [B, K] float32 out or NULL: q_k(x_k) for every k < K
 *   residual_mass  [B] float32 out or NULL: sum max(0, p_j - q_j) when j < K,
 *                  -1 when all K were kept
 *   entropy        [B, 2K+1] float32 out or NULL: the entropy in nats,
 *                  -sum_v p(v) ln p(v), of every distribution of the step:
 *                  p_0 .. p_K, then q_0 .. q_{K-1} ([At Scale] section 3:
 *                  the speculation length is tuned from the predictions'
 *                  entropy). Computed by the same single pass over the
 *                  logits (one more accumulator per element); NaN for a row
 *                  whose statistics are not finite or whose temperature is
 *                  invalid. NULL skips it (the pass is then the plain one).
 *   err_flags      [1] int32 in/out or NULL: SV_ERRF_* bits are OR-ed in
 *   workspace      device buffer of at least sv_chain_workspace_bytes() bytes
 *   stream         HIP stream the kernels are enqueued on (NULL = default)
 */
sv_status sv_verify_chain(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                          const int32_t* draft_tokens, const float* temperature,
                          const float* uniforms, int32_t B, int32_t K, int32_t V,
                          int32_t* accept_len, int32_t* out_tokens, float* p_draft,
                          float* q_draft, float* residual_mass, float* entropy,
                          int32_t* err_flags, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * sv_verify_chain for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments without the workspace: the call uses a static array of
 * SV_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs
 * on until the process ends (8 MiB covers, for instance, B=1024 K=6
 * V=256000 bf16, which needs 6.7 MiB). It allocates nothing: no hipMalloc,
 * no hipFree. Each call first clears the part of the array it uses (one
 * small fill kernel on `stream`, then the kernels of sv_verify_chain), so
 * it does not depend on what an earlier call left there. Every call on one
 * GPU shares that GPU's array: two calls that overlap in time on one GPU
 * (different streams or host threads) race and give undefined results.
 * Outputs and error bits are those of sv_verify_chain on the same inputs.
 * Returns SV_ERR_UNSUPPORTED when sv_chain_workspace_bytes(B, K, V, dtype)
 * exceeds SV_NOALLOC_SCRATCH_BYTES, and otherwise what sv_verify_chain
 * returns (SV_ERR_HIP also if the array's address cannot be obtained); on an
 * error return nothing is enqueued. The launch counts of sv_chain_launches
 * hold, plus the fill kernel.
 */
#define SV_NOALLOC_SCRATCH_BYTES (8u << 20)
sv_status sv_verify_chain_noalloc(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                                  const int32_t* draft_tokens, const float* temperature, const float* uniforms,
                                  int32_t B, int32_t K, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                                  float* p_draft, float* q_draft, float* residual_mass, float* entropy,
                                  int32_t* err_flags, hipStream_t stream);

/*
 * How many kernel launches sv_verify_chain makes for a call of this shape on
 * the current device: 1 when the statistics pass and the sampling pass run
 * as one launch, 2 when they run as two; 0 for invalid sizes or dtype. The
 * one-launch form is taken when the call's grid (statistics chunks and
 * sampling workgroups) is larger than the device holds at once, the rows
 * start on 16-byte boundaries (rows_aligned != 0: V * element size a
 * multiple of 16 and both logit tensors 16-byte aligned), K >= 1 and the
 * statistics of a sequence fit the decision's single round of loads, with or
 * without the entropy (with_entropy != 0 when it is requested). Small calls
 * (B (2K+1) <= 256 rows in all, rows on 16-byte boundaries, K >= 1, no
 * entropy) whose grid the
 * device holds at once also run as one launch, in which the statistics
 * workgroups decide and sample (sv_chain_form tells the two apart). The
 * outputs are bit-identical whichever form a call takes; only the timing
 * differs (see the launch-events hook below, which times the first
 * launch). Host-only query; nothing is enqueued.
 */
int32_t sv_chain_launches(int32_t B, int32_t K, int32_t V, sv_dtype dtype, int32_t rows_aligned,
                          int32_t with_entropy);

/*
 * Which form sv_verify_chain takes for a call of this shape on the current
 * device (arguments as sv_chain_launches): 1 the small call (one launch,
 * chain_small_kernel: the statistics workgroups of each sequence also make
 * its decision and draw), 2 one launch with ticket queues
 * (chain_one_launch_kernel, or chain_one_launch_entropy_kernel with the
 * entropy requested), 3 two launches (statistics pass, then sampling
 * pass); 0 for invalid sizes or dtype, or B = 0. Host-only query.
 */
int32_t sv_chain_form(int32_t B, int32_t K, int32_t V, sv_dtype dtype, int32_t rows_aligned, int32_t with_entropy);

/* ------------------------------------------------------------------------
 * Chain verification with the target's LM head in the call.
 *
 * The target model scores every verified position in one forward pass, and
 * its last layer maps each position's final hidden state to one logit per
 * vocabulary entry ([Topologies] section 2 timeline figure, step 2;
 * [Draft-and-Verify] "Why autoregressive decoding is slow": the pass is
 * bound by streaming the weights):
 *
 *   logits[m, v] = sum_h hidden[m, h] * head_weight[v, h]
 *
 * sv_lm_head_logits computes that layer alone (a bf16 MFMA GEMM, fp32
 * accumulation, logits rounded to bf16, round to nearest even).
 * sv_verify_chain_lm_head computes it for the B (K+1) target rows of a
 * chain verification and takes each row's softmax statistics in the GEMM's
 * epilogue, from the rounded values it stores, so the target logits are not
 * read back for them; the draft rows are streamed once as in sv_verify_chain,
 * and the decision and the residual or bonus draw are sv_verify_chain's (the
 * draw re-reads the stored target row at the first rejection). The outputs
 * follow sv_verify_chain exactly, on target logits equal to the returned
 * `target_logits`.
 *
 * Both take bf16 only, H a multiple of 64 (>= 64), V a multiple of 8, and
 * 16-byte-aligned hidden, head_weight, logits and draft_logits; otherwise
 * SV_ERR_INVALID_ARGUMENT, and nothing is enqueued.
 */
size_t sv_lm_head_chain_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t H);

/*
 *   hidden         [M, H] bf16 (device, read only)
 *   head_weight    [V, H] bf16, one row per vocabulary entry (read only)
 *   M, H, V        host ints: M >= 0
 *   logits         [M, V] bf16 out
 *   stream         HIP stream (NULL = default)
 */
sv_status sv_lm_head_logits(const void* hidden, const void* head_weight, int32_t M, int32_t H, int32_t V,
                            void* logits, hipStream_t stream);

/*
 *   hidden         [B, K+1, H] bf16: the target's final hidden state at each
 *                  verified position (read only)
 *   head_weight    [V, H] bf16 (read only)
 *   H              host int: hidden size
 *   target_logits  [B, K+1, V] bf16 out: the target's logits (the GEMM's
 *                  stored output, which the call also reads for its draw)
 *   draft_logits .. err_flags: as sv_verify_chain (bf16 draft logits;
 *                  no entropy output)
 *   workspace      device buffer of at least
 *                  sv_lm_head_chain_workspace_bytes() bytes, zero-filled
 *                  before first use; each successful call leaves it zero
 *   stream         HIP stream (NULL = default)
 */
sv_status sv_verify_chain_lm_head(const void* hidden, const void* head_weight, int32_t H, void* target_logits,
                                  const void* draft_logits, const int32_t* draft_tokens, const float* temperature,
                                  const float* uniforms, int32_t B, int32_t K, int32_t V, int32_t* accept_len,
                                  int32_t* out_tokens, float* p_draft, float* q_draft, float* residual_mass,
                                  int32_t* err_flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Draft-side sampling.
 *
 * Bytes of device workspace sv_sample_rows needs; 0 for invalid sizes. Same
 * zero-fill contract as the chain workspace (a call leaves it all zero).
 */
size_t sv_sample_workspace_bytes(int32_t R, int32_t V, sv_dtype dtype);

/*
 * One token drawn per row from the row's temperature softmax: the drafter's
 * step x ~ q(x) before verification ([In Production] section 2: each step the
 * draft model samples a candidate; [Draft-and-Verify] "The draft-and-verify
 * loop": the draft proposes its tokens one position at a time). For row r,
 * with T = temperature[r]:
 *
 *   q = softmax(logits[r,:] / T)
 *   out_tokens[r] = the first t (ascending token id) whose cumulative q
 *                   exceeds uniforms[r] * sum(q); if rounding leaves none,
 *                   the last t with q(t) > 0
 *
 * When every row starts on a 16-byte boundary (V * element size a multiple
 * of 16 and a 16-byte-aligned base, the usual case), the logits are read
 * once: the streaming pass reduces each run of 1024 bf16 (512 fp32) tokens to
 * one (reference, sum) record, and the draw re-reads only the run holding the
 * drawn token. Other rows take the bonus-draw kernels of sv_verify_chain with
 * K = 0 (a second pass over the row).
 *
 * Arguments (device pointers unless noted):
 *   logits       [R, V] dtype, row-major, element-aligned (read only)
 *   dtype        SV_DTYPE_F32 or SV_DTYPE_BF16
 *   temperature  [R] float32, each > 0 and finite; NULL means 1.0 for all
 *   uniforms     [R] float32 in [0, 1)
 *   R, V         host ints: 0 <= R, 1 <= V
 *   out_tokens   [R] int32 out: the drawn token, or -1 on a data error
 *   out_prob     [R] float32 out or NULL: q(out_tokens[r]) (NaN on a data
 *                error)
 *   err_flags    [1] int32 in/out or NULL: SV_ERRF_* bits are OR-ed in
 *                (SV_ERRF_TEMPERATURE, SV_ERRF_NONFINITE, SV_ERRF_INTERNAL)
 *   workspace    device buffer of at least sv_sample_workspace_bytes() bytes
 *   stream       HIP stream the kernels are enqueued on (NULL = default)
 * Returns SV_ERR_INVALID_ARGUMENT for bad sizes, a bad dtype or a NULL
 * required pointer, SV_ERR_WORKSPACE for a missing or short workspace, and
 * SV_ERR_HIP when a launch fails; nothing is enqueued then.
 */
sv_status sv_sample_rows(const void* logits, sv_dtype dtype, const float* temperature, const float* uniforms,
                         int32_t R, int32_t V, int32_t* out_tokens, float* out_prob, int32_t* err_flags,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Greedy tree verification.
 *
 * Bytes of device workspace sv_verify_tree_greedy needs; 0 for invalid sizes.
 * Same zero-fill contract as the chain workspace (a call leaves it all zero).
 */
size_t sv_tree_workspace_bytes(int32_t B, int32_t N, int32_t V, sv_dtype dtype);

/*
 * Greedy verification of one candidate tree per sequence ([Topologies]
 * section 4 figure: all nodes checked in one target pass, the longest
 * accepted path kept; [In Production] section 4; [At Scale] sequence diagram:
 * matching proposals are kept and the target adds its own next token).
 *
 *   g[b,n] = argmax_v target_logits[b,n,v] (raw logits, lowest v on ties)
 *   node i is accepted iff node_tokens[b,i] == g[b, pos(parents[i])] and its
 *   parent is accepted (or is the root); pos(-1) = 0, pos(i) = i + 1.
 *   The deepest accepted node (lowest index on ties) ends the accepted path;
 *   the next token is g at that node's position (g[b,0] if none is accepted).
 *
 * Arguments (device pointers unless noted):
 *   target_logits  [B, N+1, V] dtype: position 0 = after the root (the last
 *                  accepted token), position i+1 = after node i (read only)
 *   node_tokens    [B, N] int32 in [0, V)
 *   parents        [N] int32, shared by all sequences: -1 for a child of the
 *                  root, else an earlier node's index (< i)
 *   B, N, V        host ints: 0 <= B, 1 <= N <= SV_MAX_TREE_NODES, 1 <= V
 *   accept_len     [B] int32 out: depth of the deepest accepted node (0 if
 *                  none), -1 on a data error
 *   path_nodes     [B, N] int32 out: accepted node ids from the root side,
 *                  -1 padded
 *   next_token     [B] int32 out: the target's token after the accepted path
 *   err_flags      [1] int32 in/out or NULL
 *   workspace      device buffer of at least sv_tree_workspace_bytes() bytes
 *   stream         HIP stream (NULL = default)
 */
sv_status sv_verify_tree_greedy(const void* target_logits, sv_dtype dtype,
                                const int32_t* node_tokens, const int32_t* parents, int32_t B,
                                int32_t N, int32_t V, int32_t* accept_len, int32_t* path_nodes,
                                int32_t* next_token, int32_t* err_flags, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sampling verification of a candidate tree.
 *
 * Bytes of device workspace sv_verify_tree_sampling needs (one 8-byte record
 * per statistics chunk of each target and draft row, whole rows cut into
 * about 8192 chunks per call; two 8-byte exchange slots per run of 128
 * 16-byte vectors of each sequence; B + 2 counters and an abort flag);
 * 0 for invalid sizes. Same zero-fill contract as the chain workspace (a
 * call leaves it all zero; after SV_ERRF_INTERNAL it must be zero-filled
 * again).
 */
size_t sv_tree_sampling_workspace_bytes(int32_t B, int32_t N, int32_t V, sv_dtype dtype);

/*
 * Lossless sampling verification of one candidate tree per sequence: the
 * tree is checked in one target pass and the longest accepted path kept
 * ([Topologies] section 4 figure; [In Production] section 4, a tree of
 * competing branches after SpecInfer), each node by the acceptance rule
 * min(1, p/q) with the residual max(0, p - q) normalised on a rejection
 * ([Topologies] section 2; [In Production] section 2). The children of a
 * node are taken to be drawn independently from the draft's distribution at
 * that node; for several children at one position the rule is multi-step
 * speculative sampling (the SpecInfer paper's): for sequence b, T =
 * temperature[b], p_n = softmax(target_logits[b,n,:] / T), q_n =
 * softmax(draft_logits[b,n,:] / T), starting at the root (node -1,
 * position 0) with P = p_0:
 *
 *   the children v of the current node (ascending index), token x =
 *   node_tokens[b,v], are tried in turn: v is accepted iff
 *   uniforms[b,v] < min(1, P(x) / q(x)) (0 if P(x) = 0, 1 if q(x) = 0 < P(x));
 *   a rejection sets P <- max(0, P - q) / sum(max(0, P - q)) (P unchanged if
 *   that sum, formed from fp32 weights, is below 2^-126, the smallest normal
 *   fp32 number), q being q_pos of the current position (pos = 0 at the
 *   root, v + 1 at node v); an accepted child v becomes the current node,
 *   with P = p_{v+1};
 *   when every child of the current node is rejected, or it has none, one
 *   token is drawn from P with uniforms[b,N] by the inverse CDF in ascending
 *   token id (the first t whose cumulative weight exceeds uniforms[b,N] *
 *   total). With one child per node this is sv_verify_chain's rule.
 *
 * Arguments (device pointers unless noted):
 *   target_logits  [B, N+1, V] dtype: position 0 = after the root, position
 *                  i+1 = after node i (read only)
 *   draft_logits   [B, N+1, V] dtype, the same positions: the draft's
 *                  distribution the children of each node were drawn from
 *                  (rows of nodes without children are read but do not
 *                  matter) (read only)
 *   dtype          SV_DTYPE_F32 or SV_DTYPE_BF16, for both logit tensors
 *   node_tokens    [B, N] int32 in [0, V)
 *   parents        [N] int32, shared by all sequences: -1 or an earlier
 *                  node's index
 *   temperature    [B] float32 > 0, or NULL for T = 1 (one T for p and q)
 *   uniforms       [B, N+1] float32 in [0, 1): column v tests node v,
 *                  column N drives the final draw
 *   B, N, V        host ints: 0 <= B, 1 <= N <= SV_MAX_TREE_NODES, 1 <= V,
 *                  2 B (N+1) <= INT32_MAX
 *   accept_len     [B] int32 out: accepted nodes on the path, -1 on a data
 *                  error (TOKEN, TEMPERATURE, PARENT, NONFINITE)
 *   path_nodes     [B, N] int32 out: the accepted node ids from the root
 *                  side, -1 padded
 *   next_token     [B] int32 out: the drawn token after the path (-1 on a
 *                  data error)
 *   err_flags      [1] int32 in/out or NULL
 *   workspace      device buffer of at least
 *                  sv_tree_sampling_workspace_bytes() bytes, 8-byte aligned
 *   stream         HIP stream (NULL = default)
 *
 * Returns SV_ERR_INVALID_ARGUMENT for bad sizes, a bad dtype, a NULL required
 * pointer or logits not aligned to their element; SV_ERR_WORKSPACE for a
 * missing or short workspace; SV_ERR_UNSUPPORTED when a row of either
 * tensor does not start on a 16-byte boundary (V * element size not a
 * multiple of 16, or a base pointer off 16 bytes) or V exceeds 1024 * 128
 * vectors (1 048 576 bf16, 524 288 fp32 tokens); SV_ERR_HIP when a launch
 * fails. Nothing is enqueued on an error return.
 *
 * When B is small against the device's compute units, several workgroups
 * (up to 8) follow each sequence's walk and share its passes over the row
 * pairs, exchanging run totals through the workspace with bounded waits:
 * the outputs are the same as with one workgroup per sequence. A wait that
 * expires (100 ms) sets SV_ERRF_INTERNAL.
 */
sv_status sv_verify_tree_sampling(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                                  const int32_t* node_tokens, const int32_t* parents,
                                  const float* temperature, const float* uniforms, int32_t B, int32_t N,
                                  int32_t V, int32_t* accept_len, int32_t* path_nodes, int32_t* next_token,
                                  int32_t* err_flags, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Ancestor mask of a candidate tree ([Topologies] section 4 figure: all nodes
 * verified through one 2D tree-masked attention; [In Production] section 4:
 * a custom 2D causal mask): mask[i*N + j] = 1 iff j == i or j is an ancestor
 * of i, else 0. Nodes only (the root is not a row or column).
 *
 *   parents    [N] int32 (device): -1 or an earlier node's index
 *   N          host int, 1 <= N <= SV_MAX_TREE_NODES
 *   mask       [N, N] uint8 out (device)
 *   err_flags  [1] int32 in/out or NULL: SV_ERRF_PARENT on a bad parent, in
 *              which case the mask contents are unspecified
 *   stream     HIP stream (NULL = default)
 */
sv_status sv_build_tree_mask(const int32_t* parents, int32_t N, uint8_t* mask, int32_t* err_flags,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * Profiling hook (not part of the verification contract).
 *
 * Arms the calling host thread's NEXT sv_verify_chain, sv_verify_tree_greedy,
 * sv_sample_rows, sv_verify_tree_sampling, sv_verify_chain_lm_head or
 * sv_lm_head_logits call to launch its first kernel (the kernel that reads
 * every logit once: chain statistics, the one-launch chain kernel, tree
 * argmax, run records; the LM-head GEMM) with `before` and `after` as the launch's start and stop events
 * (hipExtLaunchKernel), so that they carry that kernel's own start and end
 * timestamps; the call then disarms the hook. A call that
 * fails its argument checks records nothing and also disarms it.
 * hipEventElapsedTime(before, after) is then that one kernel's duration.
 *
 *   before, after  hipEvent_t handles created by the caller (both non-NULL),
 *                  or both NULL to disarm
 *
 * Returns SV_ERR_INVALID_ARGUMENT if exactly one is NULL. The armed pair is
 * the only mutable state the library keeps, and it is per host thread.
 */
sv_status sv_time_next_stream_pass(hipEvent_t before, hipEvent_t after);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H_ */
