/*
 * ssd.h -- C ABI of the MI355X (gfx950) batched lossless verify-and-resample
 * library for Speculative Speculative Decoding (SSD) and its Saguaro pieces.
 *
 * Sources, cited by page title and section (the pages carry no code and all
 * of their formulas were lost in extraction; the readings are stated at each
 * call):
 *   [SSD-A] "全球最強推理引擎還快2倍，斯坦福、普林斯頓破解大模型串行魔咒" (repost of a
 *           機器之心 article), section "SSD 如何實現草擬與驗證并行？".
 *   [SSD-B] "超越传统SD：SSD框架全异步解码实现4.7倍平均加速", sections
 *           "投机解码的瓶颈与 SSD 的核心机制" and "Saguaro 算法：解决异步推测的三大挑战"
 *           (parts "1. 验证结果预测与缓存拓扑优化", "2. 操纵残差分布",
 *           "3. 大 Batch 下的退避策略").
 *   Acceptance rule and residual: the textbook speculative-sampling rule
 *   (Leviathan, Kalman, Matias, ICML 2023), which [SSD-A] describes in words.
 *   Random numbers: Philox4x32-10 (Salmon et al., "Parallel Random Numbers:
 *   As Easy as 1, 2, 3", SC'11).
 *
 * Common conventions
 * ------------------
 * - Logits are row-major, vocabulary contiguous: row r starts at element
 *   r * ld.  Sample/verify tensors are [B, K+1, V] rows (row = b*(K+1) + j).
 *   Entries must be finite or -inf (weight zero); each row needs one finite
 *   entry.  NaN and +inf are not supported.
 * - Pointers named "device" are HIP device memory owned by the caller; the
 *   library allocates no device memory and keeps no state between calls
 *   (the optional kernel timer below and the static scratch of
 *   ssd_round_noalloc aside).
 * - `stream` is a hipStream_t (NULL = default stream).  Every call is
 *   asynchronous: it validates its scalar arguments, enqueues its kernels
 *   and returns; nothing synchronises inside the library.
 * - Errors: argument checks run on the host before any launch and return
 *   SSD_ERR_INVALID_ARG / SSD_ERR_UNSUPPORTED / SSD_ERR_WORKSPACE without
 *   enqueuing anything; a failed launch returns SSD_ERR_HIP.  No call aborts
 *   or throws.  Values that live in device memory (temperatures, token ids,
 *   accepted lengths, depth offsets) cannot be checked on the host; the
 *   kernels guard every index they derive from them (see each call).
 * - Temperatures: one per row (softmax_t) or per sequence (sample, verify).
 *   A temperature that is not > 0 selects the greedy path (argmax, no
 *   randomness).
 * - Ties (argmax, top-F order, Gumbel scores) go to the lowest index.
 * - Workspace: a device buffer of at least ssd_workspace_bytes(...) bytes,
 *   256-byte aligned, contents irrelevant: every call writes each region
 *   before reading it.  It holds per-block partials between the kernels of
 *   one call, so calls that share a workspace must not overlap in time (use
 *   one stream or one workspace per stream).
 * - Randomness: key = (seed & 0xffffffff, seed >> 32); counter =
 *   (idx >> 2, b, j, stream id); the draw is output word idx & 3, with idx the
 *   token id (token streams), the 2048-token block id (block streams) or 0
 *   (acceptance).  Stream ids: 0 draft token, 1 draft block, 2 acceptance,
 *   3 bonus token, 4 bonus block, 5 miss fallback.  Uniform u = ((w >> 9) +
 *   0.5) * 2^-23; Gumbel g = -ln(-ln u).
 * - Sampling from weights w uses the exact two-level Gumbel-max rule over
 *   2048-token blocks: block beta* = argmax ln W_beta + g(beta) over blocks of
 *   nonzero mass, then token = argmax ln w_x + g(x) inside beta*.  The
 *   kernels evaluate each argmax in the equivalent form argmin (-ln u) / w
 *   (g = -ln(-ln u) is decreasing in -ln u), in binary32.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_BLOCK 2048         /* vocabulary block of the two-level sampler */
#define SSD_MAX_V (1 << 20)    /* largest vocabulary */
#define SSD_MAX_K 32           /* largest number of drafted tokens */
#define SSD_MAX_F 64           /* largest top-F */
#define SSD_MAX_TREE_NODES 64  /* largest drafted token tree, root included */

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1, /* null pointer, size out of range, bad C, ... */
  SSD_ERR_UNSUPPORTED = 2, /* valid request this build does not handle   */
  SSD_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned */
  SSD_ERR_HIP = 4,         /* a HIP launch failed                        */
  SSD_ERR_SCRATCH_LIMIT = 5 /* ssd_round_noalloc: the request needs more than
                               the library's static scratch               */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_F16 = 2 } ssd_dtype;

typedef enum {
  SSD_OP_SOFTMAX_T = 0,
  SSD_OP_TOPF = 1,
  SSD_OP_SAMPLE = 2,
  SSD_OP_VERIFY = 3,
  SSD_OP_VERIFY_TREE = 4  /* ssd_verify_tree: n = B, K = N (nodes besides the root) */
} ssd_op;

/* Per-row statistics (16 bytes).  max = largest logit; argmax = its lowest
 * index; lse = ln sum_x w_x relative to max, i.e. the row's normaliser in
 * nats with w_x = exp((z_x - max)/T) (times C on the top-F set for draft rows
 * of ssd_saguaro_sample).  Greedy rows have lse = 0. */
typedef struct {
  double lse;
  float max;
  int32_t argmax;
} ssd_row_stats;

/* Speculation-cache descriptor shared by sampling and verification ([SSD-B]
 * core-mechanism section: the draft prepares K-token continuations keyed by
 * the possible verification outcomes (accepted length k, bonus token) while
 * the target verifies, and one lookup follows; part 1: F_k guesses at depth
 * k under the budget Bgt = sum F_k).  A host struct; `fanout` is host memory,
 * the other arrays device memory owned by the caller.
 *   fanout     host int32 [K+1]: F_k >= 0, each <= min(SSD_MAX_F, V)
 *              (e.g. from ssd_fanout); slots are depth-major, depth k at
 *              [off_k, off_k + F_k) with off_k = F_0 + ... + F_{k-1}
 *   keys       device int32 [B, Bgt]: ssd_saguaro_sample writes, for each
 *              row j, its top-F_j draft tokens (value desc, index asc) at
 *              depth j; ssd_verify reads them
 *   payload    device int32 [B, Bgt, K]: the K pre-speculated tokens of a slot
 *              (ssd_verify; may be NULL when K = 0)
 *   out_hit, out_slot  device int32 [B]; out_tokens device int32 [B, K]
 *              (ssd_verify): as ssd_cache_lookup.
 *   miss_fill  0 or 1 (ssd_verify): as ssd_cache_lookup, with the call's V
 *              and seed. */
typedef struct {
  const int32_t* fanout;
  int32_t* keys;
  const int32_t* payload;
  int32_t* out_hit;
  int32_t* out_slot;
  int32_t* out_tokens;
  int32_t miss_fill;
} ssd_cache;

/* Temperature softmax row statistics ([SSD-A] and [SSD-B] part 2 name the
 * sampling temperature; p = softmax(z / T)).
 *   logits      device [rows, ld] of dtype dt, V <= ld
 *   temperature device float [rows]
 *   out_stats   device ssd_row_stats [rows]
 *   out_probs   device float [rows, V] (dense, row stride V) or NULL; greedy
 *               rows get onehot(argmax).
 *   workspace   ssd_workspace_bytes(SSD_OP_SOFTMAX_T, rows, 0, V) bytes.
 * Errors: rows < 1, V < 1, V > SSD_MAX_V, ld < V, null pointers. */
ssd_status ssd_softmax_t(const void* logits, ssd_dtype dt, int64_t rows, int64_t V, int64_t ld,
                         const float* temperature, ssd_row_stats* out_stats, float* out_probs,
                         void* workspace, size_t ws_bytes, void* stream);

/* Top-F of the raw logits of each row, ordered by value descending then index
 * ascending ([SSD-A]: the bonus token is predicted from the draft's most
 * likely logits).
 *   out_idx device int32 [rows, F]; out_val device float [rows, F] (the exact
 *   logits) or NULL.  1 <= F <= min(SSD_MAX_F, V).
 *   workspace   ssd_workspace_bytes(SSD_OP_TOPF, rows, 0, V) bytes. */
ssd_status ssd_topf(const void* logits, ssd_dtype dt, int64_t rows, int64_t V, int64_t ld, int32_t F,
                    int32_t* out_idx, float* out_val, void* workspace, size_t ws_bytes, void* stream);

/* Draft side of one SSD round with Saguaro sampling sigma_{F,C} ([SSD-B] part
 * 2: the draft's most likely tokens are sampled less often so that the
 * residual mass, and with it the bonus token, lands in the cached set).
 * Reading of the lost formula: with S = top-F raw draft logits of the row,
 * w_x = C * q_x on S and q_x elsewhere, sigma = w / sum w, q = softmax(z/T).
 *   draft_logits device [B, K+1, ld] rows of dtype dt
 *   temperature  device float [B]
 *   F            size of S, 0 <= F <= min(SSD_MAX_F, V); C in (0, 1]
 *   F_out        entries of out_topf per row, F <= F_out <= min(SSD_MAX_F, V)
 *                (0 allowed when F = 0); the first F of them are S
 *   seed         Philox key
 * Outputs (device):
 *   out_tokens   int32 [B, K]: x_j ~ sigma_j for j < K (greedy: argmax)
 *   out_q        float [B, K]: sigma_j(x_j) (greedy: 1)
 *   out_stats    ssd_row_stats [B, K+1]: lse = ln sum w relative to max
 *   out_topf_idx int32 [B, K+1, F_out] or NULL when F_out = 0
 *   out_topf_val float [B, K+1, F_out] or NULL
 *   cache        NULL, or a cache descriptor whose `keys` receive each row j's
 *                top-F_j list (only fanout and keys are used here); row j then
 *                ranks max(F, F_out, F_j) entries
 * Row K is not sampled; its stats and top-F predict the bonus after K
 * acceptances.  workspace: ssd_workspace_bytes(SSD_OP_SAMPLE, B, K, V).
 * Errors: also a fan-out entry < 0 or > min(SSD_MAX_F, V), or cache without
 * keys. */
ssd_status ssd_saguaro_sample(const void* draft_logits, ssd_dtype dt, int32_t B, int32_t K, int64_t V,
                              int64_t ld, const float* temperature, int32_t F, float C, int32_t F_out,
                              uint64_t seed, int32_t* out_tokens, float* out_q, ssd_row_stats* out_stats,
                              int32_t* out_topf_idx, float* out_topf_val, const ssd_cache* cache,
                              void* workspace, size_t ws_bytes, void* stream);

/* Target side: lossless acceptance test, accepted prefix and bonus token
 * ([SSD-A]: the target accepts a prefix of the drafted tokens and samples one
 * extra bonus token after them, and the output follows the target's
 * distribution; [SSD-B] part 2: a rejected position's bonus comes from the
 * residual p - q).
 * For j = 0..K-1 in order: rho_j = p_j(x_j) / sigma_j(x_j) with p = softmax of
 * the target row at temperature T and sigma_j(x_j) = draft_q (the draft's own
 * probability of the token it sampled); u_j = Philox acceptance draw; accept
 * iff u_j < rho_j; k* = number of leading accepts.  The residual uses the
 * draft row k* through draft_stats, the first F entries of draft_topf_idx and
 * C (sigma rebuilt from the draft logits).
 * Bonus: k* < K -> sample the normalised residual max(0, p_k* - sigma_k*)
 * (p_k* if it has no mass); k* = K -> sample p_K.  Greedy sequences: accept
 * iff x_j = argmax of the target row; bonus = argmax of target row k*.
 *   target_logits, draft_logits  device [B, K+1, ld] rows of dtype dt
 *   temperature  device float [B]; F, C as used for sampling; seed
 *   draft_tokens device int32 [B, K]; ids outside [0, V) are rejected with
 *                p = 0
 *   draft_q      device float [B, K]: sigma_j(x_j) from ssd_saguaro_sample
 *                (a value <= 0 makes rho infinite when p > 0)
 *   draft_stats  device ssd_row_stats [B, K+1] from ssd_saguaro_sample
 *   draft_topf_idx device int32 [B, K+1, ld_topf], ld_topf >= F (NULL if F=0)
 * Outputs (device): out_accept_len int32 [B]; out_bonus int32 [B];
 *   out_p float [B, K] = p_j(x_j) for every j; out_target_stats
 *   ssd_row_stats [B, K+1] or NULL.
 *   cache  NULL, or a cache descriptor: the realised (k*, bonus) is looked up
 *          among depth k*'s keys as ssd_cache_lookup does, in the same
 *          kernel that draws the bonus.
 * workspace: ssd_workspace_bytes(SSD_OP_VERIFY, B, K, V).
 * Errors: also a bad fan-out (as for sampling) or a cache missing keys,
 * outputs, or the payload when K > 0 and Bgt > 0. */
ssd_status ssd_verify(const void* target_logits, const void* draft_logits, ssd_dtype dt, int32_t B, int32_t K,
                      int64_t V, int64_t ld, const float* temperature, int32_t F, float C, uint64_t seed,
                      const int32_t* draft_tokens, const float* draft_q, const ssd_row_stats* draft_stats,
                      const int32_t* draft_topf_idx, int32_t ld_topf, int32_t* out_accept_len,
                      int32_t* out_bonus, float* out_p, ssd_row_stats* out_target_stats, const ssd_cache* cache,
                      void* workspace, size_t ws_bytes, void* stream);

/* The arguments of ssd_saguaro_sample and ssd_verify as structs, in the same
 * order and with the same meaning (see those calls), for ssd_round. */
typedef struct {
  const void* draft_logits;
  ssd_dtype dt;
  int32_t B, K;
  int64_t V, ld;
  const float* temperature;
  int32_t F;
  float C;
  int32_t F_out;
  uint64_t seed;
  int32_t* out_tokens;
  float* out_q;
  ssd_row_stats* out_stats;
  int32_t* out_topf_idx;
  float* out_topf_val;
  const ssd_cache* cache;
  void* workspace;
  size_t ws_bytes;
} ssd_sample_args;

typedef struct {
  const void* target_logits;
  const void* draft_logits;
  ssd_dtype dt;
  int32_t B, K;
  int64_t V, ld;
  const float* temperature;
  int32_t F;
  float C;
  uint64_t seed;
  const int32_t* draft_tokens;
  const float* draft_q;
  const ssd_row_stats* draft_stats;
  const int32_t* draft_topf_idx;
  int32_t ld_topf;
  int32_t* out_accept_len;
  int32_t* out_bonus;
  float* out_p;
  ssd_row_stats* out_target_stats;
  const ssd_cache* cache;
  void* workspace;
  size_t ws_bytes;
} ssd_verify_args;

/* Verification with early exit ([SSD-A]: the target keeps the drafted tokens
 * only up to the first rejection, so no target row past it influences the
 * result): the same acceptance test, accepted length, bonus and cache lookup
 * as ssd_verify on the same arguments (`a`, as in ssd_verify), reading fewer
 * target rows.  Positions 0 .. J-1 are streamed for every sequence; positions
 * J .. K only for the sequences with no clear rejection below J (a decision
 * taken conservatively from the rows already read: u_j at least rho_j (1 +
 * 1e-4), a greedy token that is not the argmax, or a token outside [0, V)),
 * so a sequence whose acceptance test reaches row J always has its later
 * rows read.  1 <= J <= K+1 (J = K+1 reads every row).
 * Differences from ssd_verify: out_p[b, j] is p_j(x_j) for j <= k* and NaN
 * past it; out_target_stats must be NULL.  Workspace as for ssd_verify.
 * Errors: as ssd_verify; also SSD_ERR_INVALID_ARG for a NULL `a`, J outside
 * [1, K+1] or out_target_stats not NULL. */
ssd_status ssd_verify_early(const ssd_verify_args* a, int32_t J, void* stream);

/* One step of the SSD pipeline ([SSD-A] and [SSD-B] core mechanism: the draft
 * speculates the next round while the target verifies the current one):
 * verification of round i (`v`) and draft sampling of round i+1 (`s`), with
 * results identical to ssd_verify(v) followed by ssd_saguaro_sample(s).  The
 * sampling does not depend on the verification, so the library pairs each
 * latency-bound kernel of the verification with a kernel of the sampling in
 * one launch (acceptance and residual pass beside sampling's streaming pass;
 * bonus and cache lookup beside sampling's epilogue).  Either pointer may be
 * NULL (then this is the other call alone).  The two calls need separate
 * workspaces (SSD_ERR_WORKSPACE otherwise), and the sampling's outputs and
 * cache keys must not be the verification's inputs or outputs (round i+1's
 * buffers are not round i's).  When the element types or the 16-byte
 * alignment of the two differ, the calls run one after the other.
 * Errors: as the two calls; also SSD_ERR_INVALID_ARG when a sampling output
 * (tokens, q, stats, top-F indices) is the verification's input of the same
 * kind or both use the same cache keys (other aliasing is not detected). */
ssd_status ssd_round(const ssd_verify_args* v, const ssd_sample_args* s, void* stream);

/* One pipeline step with early-exit verification: ssd_round whose
 * verification is that of ssd_verify_early (target positions J .. K read
 * only for the sequences with no clear rejection below J; 1 <= J <= K+1).
 * For callers that need no p_j(x_j) past the first rejection: accepted
 * lengths, bonus tokens, cache lookup and every sampling output are those
 * of ssd_verify_early followed by ssd_saguaro_sample on the same arguments;
 * out_p is NaN past k* and out_target_stats must be NULL.  At large batches
 * most target rows past the first two positions are never read; at B (K+1)
 * <= 256 rows, or when the two calls' element types or alignments differ,
 * the two calls run in turn.  Errors: as ssd_round, and SSD_ERR_INVALID_ARG
 * for J outside [1, K+1] or out_target_stats not NULL. */
ssd_status ssd_round_early(const ssd_verify_args* v, const ssd_sample_args* s, int32_t J, void* stream);

/* ssd_round for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, checks and results as ssd_round, except that the
 * `workspace` and `ws_bytes` fields of v and s are ignored (they may be NULL
 * and 0).  The kernels use instead a scratch array the library holds in
 * device memory, SSD_NOALLOC_HALF_BYTES for the verification and as much for
 * the sampling, on every GPU it runs on, until the process ends; this call
 * allocates nothing.  The caller still passes every input and output.
 * The scratch needs no initialisation (every region is written before it is
 * read within a call) and keeps the last call's contents.  All calls of this
 * entry point on one GPU share that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give undefined results.
 * The device is the stream's (the current device for a NULL stream); its
 * scratch address is looked up on the first call there.
 * Errors: as ssd_round; SSD_ERR_SCRATCH_LIMIT when either call needs more
 * than SSD_NOALLOC_HALF_BYTES (ssd_workspace_bytes of its op; about 1 KB per
 * logit row and 2048 vocabulary entries), before any launch. */
#define SSD_NOALLOC_HALF_BYTES (8u << 20)
ssd_status ssd_round_noalloc(const ssd_verify_args* v, const ssd_sample_args* s, void* stream);

/* Token-tree verification ([SSD-A], closing paragraph of "SSD 如何實現草擬與
 * 驗證并行？": SSD combines naturally with token-tree speculation; the pages
 * give no algorithm).  Reading: the textbook multi-candidate rule, recursive
 * rejection sampling over each node's drafted children, lossless when the
 * children of a node are independent draws from sigma of that node's draft
 * row (e.g. ssd_saguaro_sample called once per child rank with its own
 * seed).  Walking from the root: at node n with children m_1 < m_2 < ...
 * (sibling rank i = 0, 1, ...) the residual starts as r = p_n; sibling i is
 * accepted iff u < r(x) / sigma_n(x), u the acceptance draw at (idx = i, b,
 * j = n); on acceptance the walk moves to it; on rejection r becomes
 * max(0, r - sigma_n) renormalised (unchanged when it has no mass).  When
 * every sibling is rejected the bonus is drawn from r, at a node without
 * children from p_n, both at (b, j = n) with the bonus streams.  Greedy
 * sequences accept the first child whose token is the target row's argmax;
 * their bonus is the argmax where the walk stops.  A path tree (parent[m] =
 * m - 1) gives exactly ssd_verify's accepted length and bonus.
 * Each rejection of a sibling costs one pass over the node's target and
 * draft rows (the residual's normaliser, needed before the next sibling).
 *   target_logits, draft_logits  device [B, N+1, ld] rows: row n holds the
 *                logits at node n (node 0 = the root)
 *   parent       host int32 [N+1]: parent[0] = -1, 0 <= parent[m] < m; the
 *                topology is shared by the batch; 0 <= N < SSD_MAX_TREE_NODES
 *   tokens       device int32 [B, N+1]: token of node m >= 1 (entry 0
 *                unused); ids outside [0, V) are rejected
 *   draft_q      device float [B, N+1]: sigma_{parent[m]}(token m) (a value
 *                <= 0 makes the ratio infinite when r > 0)
 *   draft_stats  device ssd_row_stats [B, N+1] of the draft rows (as from
 *                ssd_saguaro_sample with K = N); draft_topf_idx device int32
 *                [B, N+1, ld_topf] (their first F entries are each row's S;
 *                NULL if F = 0); temperature, F, C, seed as for ssd_verify
 * Outputs (device int32 [B]): out_accept_len = nodes accepted (the depth of
 *   out_last), out_last = the node where the walk stopped (its ancestors are
 *   the accepted path), out_bonus.
 * workspace: ssd_workspace_bytes(SSD_OP_VERIFY_TREE, B, N, V).
 * Errors: SSD_ERR_INVALID_ARG for a NULL `a` or pointer, sizes out of range,
 * a parent array that is not a tree in index order, bad F or C. */
typedef struct {
  const void* target_logits;
  const void* draft_logits;
  ssd_dtype dt;
  int32_t B, N;
  int64_t V, ld;
  const int32_t* parent;
  const float* temperature;
  int32_t F;
  float C;
  uint64_t seed;
  const int32_t* tokens;
  const float* draft_q;
  const ssd_row_stats* draft_stats;
  const int32_t* draft_topf_idx;
  int32_t ld_topf;
  int32_t* out_accept_len;
  int32_t* out_last;
  int32_t* out_bonus;
  void* workspace;
  size_t ws_bytes;
} ssd_tree_args;
ssd_status ssd_verify_tree(const ssd_tree_args* a, void* stream);

/* Speculation-cache lookup keyed by (accepted length, bonus token) ([SSD-B]
 * core-mechanism section: the draft builds a speculation cache while the
 * target verifies and a single lookup follows; [SSD-A]: on a hit the prepared
 * tokens go to the verifier at once).
 *   keys      device int32 [B, Bgt]: depth-major, depth k at
 *             [depth_off[k], depth_off[k+1])
 *   depth_off device int32 [K+2], non-decreasing, depth_off[K+1] <= Bgt
 *   payload   device int32 [B, Bgt, K]: the K pre-speculated tokens of a slot
 *   accept_len, bonus  device int32 [B] (from ssd_verify)
 * Outputs (device): out_hit int32 [B] (1/0); out_slot int32 [B] (lowest
 * matching slot or -1); out_tokens int32 [B, K] (payload on a hit).
 * On a miss ([SSD-B] part 3: past a critical batch size a miss is served by
 * a near-zero-latency speculator such as random tokens): miss_fill = 0 writes
 * -1 (the caller runs its own backup speculator); miss_fill = 1 writes K
 * random tokens in [0, V): token i of sequence b is floor(w * V / 2^32) with
 * w the Philox word of stream 5 at (idx = i, b, j = 0) under `seed` (V and
 * seed are read only when miss_fill = 1).
 * An accepted length outside [0, K] or offsets out of order give a miss.
 * Errors: also miss_fill not 0 or 1, or miss_fill = 1 with V outside
 * [1, SSD_MAX_V]. */
ssd_status ssd_cache_lookup(const int32_t* keys, const int32_t* depth_off, const int32_t* payload, int32_t B,
                            int32_t K, int32_t Bgt, const int32_t* accept_len, const int32_t* bonus,
                            int32_t* out_hit, int32_t* out_slot, int32_t* out_tokens, int32_t miss_fill,
                            int64_t V, uint64_t seed, void* stream);

/* Build cache keys from per-row top-F lists: keys[b, depth_off[k] + i] =
 * topf_idx[b, k, i] for i < F_k = depth_off[k+1] - depth_off[k] (F_k <=
 * ld_topf, else the key is -1).  topf_idx device int32 [B, K+1, ld_topf];
 * depth_off device int32 [K+2]; out_keys device int32 [B, Bgt]. */
ssd_status ssd_cache_keys(const int32_t* topf_idx, int32_t ld_topf, const int32_t* depth_off, int32_t B,
                          int32_t K, int32_t Bgt, int32_t* out_keys, void* stream);

/* Fan-out F_k, k = 0..K, under budget Bgt ([SSD-B] part 1: the optimal
 * per-depth fan-out is a truncated geometric series that shrinks with depth
 * because the chance of accepting k tokens decays exponentially).  Reading:
 * F_k proportional to ratio^k with sum exactly Bgt -- w_k = ratio^k by
 * repeated multiplication from 1, S = w_0 + ... + w_K in order, ideal_k =
 * Bgt * w_k / S (fp64), F_k = floor(ideal_k) and the remaining units go to
 * the largest fractional parts, ties to the smaller k; each F_k is capped at
 * V and the excess handed out in ascending k.  Pure host function.
 *   out_F host int32 [K+1].  Errors: Bgt < 0, K < 0 or > SSD_MAX_K, ratio not
 *   finite or <= 0, V < 1, Bgt > (K+1)*V. */
ssd_status ssd_fanout(int32_t Bgt, int32_t K, double ratio, int64_t V, int32_t* out_F);

/* Fan-out from measured statistics ([SSD-B] part 1: the budget goes where
 * acceptance stops most often; the pages' truncated geometric is the shape
 * this gives when the hit curves are the same power law at every depth).
 * Pure host function.
 *   a      host double [K+1]: measured P(k* = k), finite, >= 0
 *   h      host double [K+1][Fmax+1] row-major: h[k][F] = measured chance
 *          that the bonus after k acceptances is among the draft's top-F
 *          tokens of row k (h[k][0] = 0, non-decreasing in F), finite
 *   Fmax   1 .. SSD_MAX_F; Bgt <= (K+1) Fmax
 * Output out_F host int32 [K+1], sum Bgt: each slot in turn goes to the depth
 * with the largest a[k] (h[k][F_k+1] - h[k][F_k]) (ties to the smaller k;
 * depths at Fmax excluded); optimal for sum_k a[k] h[k][F_k] when every h[k]
 * is concave.  Errors: SSD_ERR_INVALID_ARG. */
ssd_status ssd_fanout_greedy(const double* a, const double* h, int32_t K, int32_t Fmax, int32_t Bgt,
                             int32_t* out_F);

/* Back-off rule for cache misses ([SSD-B] part 3: as the batch grows, the
 * chance that some sequence misses grows and the whole batch waits for the
 * backup speculator; below a critical batch size, set by the hit rate and the
 * latencies, an accurate slow backup pays, above it a near-zero-latency one
 * such as random tokens).  The pages give no formula; this rule compares
 * expected tokens per unit time.  With P = prod_b p_hit[b], the chance that
 * no sequence misses:
 *   accurate backup: B * e_acc tokens per t_round + (1 - P) * t_slow;
 *   fast backup:     sum_b (p_b e_acc + (1 - p_b) e_fast) tokens per
 *                    t_round + (1 - P) * t_fast.
 * Pure host function.
 *   p_hit  host double [B], each in [0, 1] (e.g. measured per-sequence hit
 *          rates)
 *   c      t_round > 0, t_slow >= 0, t_fast >= 0 (any one time unit),
 *          e_acc > 0, e_fast >= 0 (tokens per sequence and round), all finite
 * Outputs: *out_use_fast = 1 when the fast backup's rate is strictly higher
 * (else 0); *out_gain = its rate over the accurate backup's (out_gain may be
 * NULL).  Errors: SSD_ERR_INVALID_ARG for B < 1, null pointers or values out
 * of range. */
typedef struct {
  double t_round;  /* a round in which every sequence hits */
  double t_slow;   /* added wait for the accurate backup speculator */
  double t_fast;   /* added wait for the fast backup (random tokens) */
  double e_acc;    /* tokens per sequence and round from an accurate speculation */
  double e_fast;   /* tokens per sequence and round from the fast backup */
} ssd_backoff_cost;
ssd_status ssd_backoff(const double* p_hit, int32_t B, const ssd_backoff_cost* c, int32_t* out_use_fast,
                       double* out_gain);

/* Workspace bytes for `op`.  n = rows for SOFTMAX_T / TOPF (K ignored), n = B
 * for SAMPLE / VERIFY.  Returns 0 for invalid sizes. */
size_t ssd_workspace_bytes(ssd_op op, int64_t n, int32_t K, int64_t V);

/* Static string naming a status. */
const char* ssd_status_string(ssd_status s);

/* Streaming-read probe, a measurement aid (not part of the method): reads
 * `bytes` of device memory at `buf` (16-byte aligned) once with 16-byte loads
 * and folds them into one word per workgroup, in one of several launch
 * layouts, so that the read bandwidth the streaming passes can reach is
 * measured by this library on the same part.  variant: 0 one-shot grid of
 * 256-thread workgroups with 8 loads per thread in flight, nontemporal (the
 * streaming passes' layout); 1 the same with 16 loads; 2, 3 with 512 and
 * 1024 threads; 4 as 0 with ordinary loads; 5, 6 persistent grids of 8 x 256
 * and 4 x 512 threads per compute unit, the next chunk's loads issued before
 * the current one is folded; 7, 8 4 loads per thread with 256 and 1024
 * threads; 9 persistent, 2 x 1024 threads per compute unit, 4 loads; 10 as 0
 * with consecutive chunks kept on one XCD; 11 512 threads with 16 loads.
 *   out  device uint32 [out_len], out_len >= the grid (bytes / 16 / (threads
 *        x loads) workgroups for the one-shot variants); its contents are
 *        not meaningful.
 * Errors: SSD_ERR_INVALID_ARG for a bad pointer, size or variant;
 * SSD_ERR_UNSUPPORTED when out_len is too small. */
ssd_status ssd_read_probe(const void* buf, size_t bytes, int32_t variant, uint32_t* out, size_t out_len,
                          void* stream);

/* Phase stamps, a measurement aid of the instrumented build only (compiled
 * with -DSSD_PHASES; `python -m lossless_verify_sample_amd.build --phases`
 * writes libssd_phases.so): the latency-bound kernels record the 100 MHz
 * real-time counter (10 ns per tick) at fixed points, 8 slots per item:
 *   kind 0: sampling epilogue, item = row b*(K+1)+j: start, partials loaded,
 *           block weights summed, top-F list, sigma normaliser and outputs,
 *           block drawn, token drawn;
 *   kind 1: verification after the streaming pass, item = sequence: start,
 *           statistics of the K+1 rows, decisions, block of the bonus drawn
 *           (the lazy block race), bonus token, lookup done; slot 7 holds
 *           the number of blocks the lazy race evaluated (not a time).
 * ssd_phase_read copies the first n stamps of `kind` (item * 8 + slot, up to
 * 8192 items; slots an item does not reach keep older values) to host `out`.
 * Errors: SSD_ERR_UNSUPPORTED in the ordinary build; SSD_ERR_INVALID_ARG for
 * a bad kind, pointer or count. */
ssd_status ssd_phase_read(int32_t kind, uint64_t* out, int64_t n);

/* Kernel timer, a measurement aid (not part of the method).  While enabled,
 * every launch of the streaming pass -- the kernel that reads each logit row
 * once from HBM, in ssd_softmax_t, ssd_topf, ssd_saguaro_sample and
 * ssd_verify -- is timed by a pair of HIP events that the launch itself
 * records on the call's stream (hipExtLaunchKernelGGL), up to max_launches
 * launches per op.  In ssd_round the launch that carries the sampling's
 * streaming pass (beside the verification of each sequence, or at small
 * batches beside the verification's streaming pass) counts as SSD_OP_SAMPLE
 * and a launch of the verification's streaming pass alone as SSD_OP_VERIFY.
 *   ssd_timer_enable(n): n > 0 (re)creates the events and clears the counts;
 *     n = 0 destroys them.  Host-side state of the library, guarded by a
 *     mutex; launches from several threads interleave in one count, so time
 *     one thread's calls at a time.
 *     Errors: n < 0 or n > 1 << 20 (INVALID_ARG), event creation (HIP).
 *   ssd_timer_read(op, &launches, &total_ms): waits for the recorded events
 *     and returns how many launches of that op were timed and their summed
 *     duration in milliseconds.  Errors: bad op or null pointers. */
ssd_status ssd_timer_enable(int32_t max_launches);
ssd_status ssd_timer_read(ssd_op op, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
