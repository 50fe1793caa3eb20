/*
 * d3d.h -- C ABI of the MI355X (gfx950) hot path of asynchronous block-diffusion speculative
 * decoding: descriptor builder, packed draft attention, speculative-sampling verify, branch-cache
 * match.
 *
 * Pages cited: [D3D] = the summary page "D3D: Decoupled Diffusion Drafting for Asynchronous
 * Speculative Decoding"; [DScout] = the summary page "Factorization-Guided Training and Inference
 * for Diffusion-Drafted Speculative Decoding". Sections are named by their headings.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller unless marked (host). The library never
 *    allocates, frees or synchronises; GPU work is enqueued asynchronously on `stream`.
 *  - Tensors are dense, row-major (last index fastest), with the element type given by `dtype`
 *    (bf16 = IEEE bfloat16 bit patterns, f32 = IEEE binary32) unless stated otherwise.
 *  - Return value: D3D_OK (0) or a negative status. Argument errors are found on the host before
 *    anything is launched; d3d_status_string() describes a status. No C++ exception crosses the
 *    ABI. The library is thread-safe; two calls that share a workspace must not overlap in time.
 *    Its only global state is the static scratch of spec_verify_noalloc (one array per GPU, and
 *    the cached device address of that array).
 *  - A vocabulary size (vocab) is at most 2^28; larger values are argument errors.
 *  - Device-side contents (descriptors, page tables, token ids) are not validated on the host;
 *    kernels clamp every index they derive from them so that no access leaves its buffer.
 */
#ifndef D3D_H
#define D3D_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  D3D_OK = 0,
  D3D_EINVAL = -1,       /* bad shape or argument; nothing launched */
  D3D_EUNSUPPORTED = -2, /* valid but not implemented (head_dim, group size, ...) */
  D3D_EHIP = -3,         /* a HIP launch reported an error */
  D3D_EWORKSPACE = -4,   /* workspace missing or smaller than the *_workspace() size */
  D3D_ESCRATCH = -5      /* spec_verify_noalloc: the call needs more than D3D_VERIFY_SCRATCH_BYTES */
};

/* Element type of the tensor arguments. Only D3D_BF16 and D3D_F32 are valid; the two range
 * enumerators make every 32-bit value a value of the type, so that any other number a caller
 * passes (from C, or through a foreign-function interface) is refused with D3D_EINVAL rather than
 * being undefined in the library's C++. */
typedef enum {
  D3D_BF16 = 0,
  D3D_F32 = 1,
  D3D_DTYPE_RANGE_MIN_ = INT32_MIN,
  D3D_DTYPE_RANGE_MAX_ = INT32_MAX
} d3d_dtype;

/* flags bit of a block descriptor: the block is causal inside itself (else bidirectional). */
#define D3D_BLOCK_CAUSAL 1u

/* One packed block of B query rows: an anchor token followed by B-1 masked positions
 * ([D3D] 方法步骤详情 step 2 and step 4; [DScout] 前置知识: 块扩散草稿器).
 *  prefix_len : length of the request's shared, causally encoded prefix (informational).
 *  rej_pos    : r, the number of rows of the request's first block (the current block) this block
 *               also sees -- the accepted slice its branch assumes; 0 for the current block,
 *               k for the branch of rejection position k, B for the full-accept branch.
 *  anchor     : the anchor token id of the block.
 *  flags      : D3D_BLOCK_CAUSAL or 0. */
typedef struct {
  int32_t prefix_len;
  int32_t rej_pos;
  int32_t anchor;
  int32_t flags;
} d3d_block_desc;

/* ---------------------------------------------------------------------------------------------
 * Descriptor builder (host only) -- [D3D] 方法步骤详情 step 4 and 技术新颖性: one packed forward
 * pre-drafts, for each of the first C-1 rejection positions, F alternative anchors, plus the
 * full-accept case: N_async = B[(C-1)F + 2] tokens.
 *
 * Writes (C-1)F + 2 descriptors to `out` (host), in pack order: the current block
 * {prefix_len, 0, cur_anchor, CAUSAL}; then for k = 1..C-1 (major) and f = 0..F-1 the branch
 * {prefix_len, k, alt_anchors[(k-1)F + f], 0}; then the full-accept block
 * {prefix_len, B, alt_anchors[(C-1)F], 0}.
 *  block_size B in [1, 64]; coverage C in [2, B]; fanout F >= 1; prefix_len >= 0.
 *  alt_anchors (host): (C-1)F + 1 token ids.  cap: capacity of `out`.  n_out (host): count written.
 * Errors: D3D_EINVAL on a bad argument or cap < (C-1)F + 2 (nothing written).
 * ------------------------------------------------------------------------------------------- */
int d3d_build_branch_descs(int block_size, int coverage, int fanout, int prefix_len,
                           int32_t cur_anchor, const int32_t *alt_anchors,
                           d3d_block_desc *out, int cap, int *n_out);

/* The same for a batch of n_req requests with a common (B, C, F), as a serving scheduler builds
 * them each round: request i's (C-1)F + 2 descriptors are written at out[i * ((C-1)F + 2)], in the
 * order above, from prefix_len[i], cur_anchor[i] and the (C-1)F + 1 anchors at
 * alt_anchors[i * ((C-1)F + 1)] (all host arrays). req_block_off (host, n_req + 1 entries) receives
 * the packed block offsets draft_attn_packed takes.
 * Errors: D3D_EINVAL on a bad argument or cap < n_req ((C-1)F + 2) (out may be partly written). */
int d3d_build_branch_descs_batch(int n_req, int block_size, int coverage, int fanout,
                                 const int32_t *prefix_len, const int32_t *cur_anchor,
                                 const int32_t *alt_anchors, d3d_block_desc *out, int cap,
                                 int32_t *req_block_off);

/* The same batch built on the device from DEVICE arrays: in a serving loop the anchors come from
 * draft_topk on the GPU and the prefix lengths from kv_commit, so the descriptors need no round
 * trip through the host. Request i's (C-1)F + 2 descriptors go to out[i * ((C-1)F + 2)] (DEVICE), in
 * the order above, from prefix_len[i], cur_anchor[i] and the (C-1)F + 1 anchors at
 * alt_anchors[i * ((C-1)F + 1)]; req_block_off (DEVICE, n_req + 1 entries) receives i ((C-1)F + 2),
 * or is NULL. Device values are copied as they are (not validated). One launch on `stream`.
 * Errors: D3D_EINVAL on a bad argument or n_req ((C-1)F + 2) >= 2^31 - 256 (nothing launched). */
int d3d_build_branch_descs_device(int n_req, int block_size, int coverage, int fanout,
                                  const int32_t *prefix_len, const int32_t *cur_anchor,
                                  const int32_t *alt_anchors, d3d_block_desc *out,
                                  int32_t *req_block_off, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Packed draft attention -- one drafter attention layer of the packed forward ([D3D] 核心方法:
 * prefix shared and causally encoded, attention bidirectional inside a block; 方法步骤详情 step 4).
 *
 * Requests are packed one after another. Request i owns blocks [req_block_off[i],
 * req_block_off[i+1]) and query rows [B*req_block_off[i], B*req_block_off[i+1]); its first block
 * is its current block. Query row t of block b (position j = t mod B) with query head h attends to
 *   - every token of the request's prefix (req_prefix_len[i] tokens),
 *   - rows [0, r_b) of the request's current block, when b is not the current block,
 *   - the rows of its own block: all of them, or rows 0..j when the block is CAUSAL,
 * with softmax(scale * q.k) weights over key/value head g = h / (n_heads_q / n_heads_kv).
 *
 *  q      [total_q, n_heads_q, head_dim]     total_q = B * req_block_off[n_req]
 *  k_new, v_new [total_q, n_heads_kv, head_dim] the packed rows' own keys / values
 *  k_cache, v_cache: prefix keys / values.
 *     page_table == NULL: [n_req, kv_stride, n_heads_kv, head_dim]; request i's token p is at row
 *                         i*kv_stride + p; needs req_prefix_len[i] <= kv_stride.
 *     page_table != NULL: [num_pages, page_size, n_heads_kv, head_dim]; token p of request i is row
 *                         p mod page_size of page page_table[i*max_pages + p/page_size]; needs
 *                         req_prefix_len[i] <= max_pages*page_size. Page ids outside
 *                         [0, num_pages) are clamped into range (the result is then unspecified,
 *                         but no access leaves the cache).
 *  descs  [total_blocks] device descriptors (rej_pos and flags are used; rej_pos is clamped to
 *         [0, B]).
 *  req_block_off (host) [n_req+1], non-decreasing, req_block_off[0] == 0.
 *  req_prefix_len (host) [n_req], in [0, 2^30].
 *  dtype  D3D_BF16 (fp32 accumulation, bf16 output) or D3D_F32 (fp32 throughout).
 *  head_dim in {64, 128}; n_heads_q / n_heads_kv in {1, 2, 4, 8, 16}; 1 <= B <= 64;
 *  1 <= n_req <= D3D_ATTN_MAX_REQ.
 *  out    [total_q, n_heads_q, head_dim].
 *  ws     workspace of at least draft_attn_packed_workspace(...) bytes (may be NULL if that is 0);
 *         fp32 split-KV partial results; no initial contents are required.
 * ------------------------------------------------------------------------------------------- */
#define D3D_ATTN_MAX_REQ 64

/* Workspace bytes draft_attn_packed needs for this dtype, request layout and head shape on the
 * current device (the number of key splits depends on the device's compute-unit count); 0 when no
 * workspace is needed or the arguments are invalid. */
size_t draft_attn_packed_workspace(d3d_dtype dtype, const int32_t *req_block_off,
                                   const int32_t *req_prefix_len, int n_req, int block_size,
                                   int n_heads_q, int n_heads_kv, int head_dim);

int draft_attn_packed(d3d_dtype dtype, const void *q, const void *k_new, const void *v_new,
                      const void *k_cache, const void *v_cache, const int32_t *page_table,
                      int page_size, int max_pages, int num_pages, int kv_stride,
                      const d3d_block_desc *descs, const int32_t *req_block_off,
                      const int32_t *req_prefix_len, int n_req, int block_size, int n_heads_q,
                      int n_heads_kv, int head_dim, float scale, void *out, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* draft_attn_packed with a join: before its last launch (the split merge, when the call has one:
 * draft_attn_packed_workspace > 0; otherwise after the attention kernel) the stream waits for the
 * event `join` (hipStreamWaitEvent). A round that verifies on a second stream while the drafter
 * attends joins the two there, so that the merge is the round's last kernel. join == NULL is
 * draft_attn_packed. Same arguments, outputs and errors otherwise. */
int draft_attn_packed_join(d3d_dtype dtype, const void *q, const void *k_new, const void *v_new,
                           const void *k_cache, const void *v_cache, const int32_t *page_table,
                           int page_size, int max_pages, int num_pages, int kv_stride,
                           const d3d_block_desc *descs, const int32_t *req_block_off,
                           const int32_t *req_prefix_len, int n_req, int block_size, int n_heads_q,
                           int n_heads_kv, int head_dim, float scale, void *out, void *ws,
                           size_t ws_bytes, hipEvent_t join, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Speculative-sampling verify ([D3D] 前置知识: 投机解码; [DScout] 前置知识: 推测解码, 平均接受长度
 * MAT, 接受加权损失 AWL 与推测采样接受规则).
 *
 * For request i, target row j (j = 0..n_draft) and draft row j (j = 0..n_draft-1), with
 * P_j = softmax(z^P_j / T) and Q_j = softmax(z^Q_j / T):
 *   alpha_j = min(1, P_j(y_j) / Q_j(y_j))   (1 when Q_j(y_j) = 0)
 *   u_j     = Philox4x32-10 uniform, key = seed, counter = (j, i, round, 0)
 *   n_acc   = first j with u_j >= alpha_j, or n_draft when every draft is accepted
 *   next    = residual draw from max(0, P_n_acc - Q_n_acc) (rejection) or from P_n_draft (bonus),
 *             the smallest token v whose inclusive cumulative mass exceeds u' * Z, with
 *             u' = Philox uniform, counter = (0, i, round, 1)
 *   survival[k-1] = S(k) = prod_{j<k} alpha_j for k = 1..n_draft;  tau = 1 + sum_k S(k)
 * Uniforms take the top 27 bits of output word 0 and the top 26 of word 1: a double on the
 * 53-bit grid of [0, 1). temperature == 0 is greedy: alpha_j = [y_j == first argmax z^P_j], the
 * next token is the first argmax of the target row; draft logits are not read.
 * Precision: per-element exp in fp32 with fp64 accumulation for the acceptance statistics; the
 * sampled row is recomputed entirely in fp64.
 *
 *  target_logits [n_req, n_draft+1, vocab], draft_logits [n_req, n_draft, vocab]  (dtype)
 *  draft_tokens  [n_req, n_draft] int32 (ids outside [0, vocab) are clamped)
 *  1 <= n_draft <= 63; vocab >= 1; temperature >= 0 and finite.
 *  outputs: n_accepted [n_req] i32, next_token [n_req] i32, alpha [n_req, n_draft] f32,
 *           survival [n_req, n_draft] f32, tau [n_req] f32, flags [n_req] u32:
 *           bit0 some acceptance decision had |u_j - alpha_j| < 1e-6; bit1 the draw was within
 *           1e-6 Z of a cumulative boundary; bit2 the residual mass was zero and the draw fell back
 *           to P. Any output pointer except n_accepted and next_token may be NULL.
 *  ws: at least spec_verify_workspace(...) bytes; no initial contents are required.
 * ------------------------------------------------------------------------------------------- */
size_t spec_verify_workspace(int n_req, int n_draft, int vocab);

int spec_verify(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
                const int32_t *draft_tokens, int n_req, int n_draft, int vocab, float temperature,
                uint64_t seed, uint32_t round, int32_t *n_accepted, int32_t *next_token,
                float *alpha, float *survival, float *tau, uint32_t *flags, void *ws,
                size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * spec_verify for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments and outputs as spec_verify,
 * without ws / ws_bytes. The workspace is a file-scope device array of D3D_VERIFY_SCRATCH_BYTES on
 * each GPU, held until the process ends; the call allocates and frees nothing. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (different streams, or different
 * host threads without ordering) race and give undefined outputs. Its contents carry over from
 * call to call; none of them is read before it is written, so nothing is cleared.
 * Errors: as spec_verify; D3D_ESCRATCH (nothing launched) when spec_verify_workspace(n_req,
 * n_draft, vocab) exceeds D3D_VERIFY_SCRATCH_BYTES (e.g. about 1650 requests of B = 16 at
 * V = 151936); D3D_EHIP if the array's device address cannot be obtained.
 * ------------------------------------------------------------------------------------------- */
#define D3D_VERIFY_SCRATCH_BYTES ((size_t)6 << 20)

int spec_verify_noalloc(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
                        const int32_t *draft_tokens, int n_req, int n_draft, int vocab, float temperature,
                        uint64_t seed, uint32_t round, int32_t *n_accepted, int32_t *next_token,
                        float *alpha, float *survival, float *tau, uint32_t *flags, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Branch-cache match ([D3D] 前置知识: 异步起草与缓存命中): a verified outcome (n_acc accepted
 * drafts, then token t) hits the branch whose assumed accepted slice and anchor it reproduces:
 * the first block b after the request's current block, in pack order, with rej_pos == n_acc + 1
 * and anchor == t. hit_branch[i] = b - req_block_off[i] (the block's index inside the request), or
 * -1 on a miss. descs: [total_blocks]; req_block_off is a DEVICE array here, [n_req+1] (entries
 * are clamped to [0, total_blocks]); n_accepted, next_token, hit_branch: [n_req]; n_req >= 1.
 * ------------------------------------------------------------------------------------------- */
int branch_cache_match(const d3d_block_desc *descs, int total_blocks, const int32_t *req_block_off,
                       int n_req,
                       const int32_t *n_accepted, const int32_t *next_token, int32_t *hit_branch,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * spec_verify followed by branch_cache_match on its outcome, in the same launches: the match of a
 * request runs in the pass that settles its next token (greedy: the decide pass; sampling: the draw
 * pass). Arguments as spec_verify, then the branch_cache_match arguments (descs [total_blocks],
 * req_block_off DEVICE [n_req+1], hit_branch [n_req]). Outputs are identical to the two calls in
 * sequence. Errors: as spec_verify, and D3D_EINVAL on NULL descs / req_block_off / hit_branch or
 * total_blocks < 1.
 * ------------------------------------------------------------------------------------------- */
int spec_verify_match(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
                      const int32_t *draft_tokens, int n_req, int n_draft, int vocab, float temperature,
                      uint64_t seed, uint32_t round, int32_t *n_accepted, int32_t *next_token, float *alpha,
                      float *survival, float *tau, uint32_t *flags, void *ws, size_t ws_bytes,
                      const d3d_block_desc *descs, int total_blocks, const int32_t *req_block_off,
                      int32_t *hit_branch, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Drafter token selection ([D3D] 方法步骤详情 step 4, 前置知识: 异步起草与缓存命中): the k best
 * tokens of each logit row other than an excluded one. Order: larger logit first, ties to the lower
 * token id; NaN logits count as -inf. Uses: the greedy drafted token of every masked position of the
 * packed blocks (k = 1: argmax); the F alternative anchors of rejection position k = 1..C-1, i.e. the
 * F best tokens of draft row k-1 other than the rejected draft token d_k (its residual mass is zero,
 * so it can never be the replacement; k = F, exclude = d_k); the full-accept anchor (k = 1 over the
 * row after the block).
 *
 *  logits   [rows_in, vocab] (dtype), DEVICE; vocab >= 1
 *  rows     [n_rows] DEVICE row indexes into logits, or NULL for rows 0..n_rows-1
 *  exclude  [n_rows] DEVICE token to skip per row (any value outside [0, vocab): none), or NULL
 *  k        1..8; out DEVICE int32: row r's k tokens at out[out_off[r] .. + k-1] (out_off [n_rows]
 *           DEVICE, or NULL for r * k); -1 where a row has fewer than k candidates
 *  ws       at least draft_topk_workspace(n_rows, vocab, k) bytes; no initial contents required.
 * Errors: D3D_EINVAL on bad sizes (n_rows < 1, vocab < 1, k outside 1..8) or NULL pointers;
 * D3D_EWORKSPACE if ws is too small. Row indexes and offsets are not range-checked.
 * ------------------------------------------------------------------------------------------- */
size_t draft_topk_workspace(int n_rows, int vocab, int k);
int draft_topk(d3d_dtype dtype, const void *logits, int vocab, int n_rows, const int32_t *rows,
               const int32_t *exclude, int k, int32_t *out, const int32_t *out_off, void *ws,
               size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Sampled drafting at temperature T > 0 ([D3D] 方法步骤详情 step 4: the packed forward drafts every
 * masked position; [DScout] 实验结果 decodes at temperature 1): the token of each logit row is a draw
 * from softmax(z / T), taken by the Gumbel-max rule as the token with the largest
 * z_v / T - ln(-ln u_v), ties to the lower id, decided in fp64. u_v = ((w >> 8) + 1/2) / 2^24 with w
 * word (v mod 4) of Philox4x32-10 (Salmon et al., SC'11) at counter (v div 4, logits row index,
 * round, 2) under the key (seed low word, seed high word). NaN logits count as -inf; a row whose
 * logits are all -inf gets -1. Greedy drafting (T = 0) is draft_topk with k = 1.
 *
 *  logits       [rows_in, vocab] (dtype), DEVICE; vocab >= 1
 *  rows         [n_rows] DEVICE row indexes into logits, or NULL for rows 0..n_rows-1; the row index
 *               (rows[r], or r) is the generator's second counter word
 *  temperature  finite, > 0
 *  out          [n_rows] DEVICE int32: the drawn token of each row
 *  ws           at least draft_sample_workspace(n_rows, vocab) bytes; no initial contents required.
 * Errors: D3D_EINVAL on bad sizes (n_rows < 1, vocab < 1), a temperature that is not finite and
 * positive, or NULL pointers; D3D_EWORKSPACE if ws is too small. Row indexes are not range-checked.
 * ------------------------------------------------------------------------------------------- */
size_t draft_sample_workspace(int n_rows, int vocab);
int draft_sample(d3d_dtype dtype, const void *logits, int vocab, int n_rows, const int32_t *rows,
                 float temperature, uint64_t seed, uint32_t round, int32_t *out, void *ws, size_t ws_bytes,
                 hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * KV commit of the accepted slice and promotion of the hit branch ([D3D] 前置知识: 异步起草与缓存命中,
 * 方法步骤详情 step 4). After verification request i's prefix grows by its anchor and accepted drafts:
 * rows 0..n_acc_i of its block 0 in the packed k_new / v_new (causal in-block, so they are prefix
 * keys / values) are copied to the paged cache at token positions prefix_len[i] .. + n_acc_i, and
 * prefix_len[i] grows by n_acc_i + 1. With hit / packed_tokens / next_block given, next_block[i]
 * receives the B packed tokens of the hit branch (block hit_i of request i; the next round's current
 * block), or B times -1 on a miss.
 *
 *  k_new, v_new   [N_q, H_kv, d] (dtype), DEVICE, 16-byte aligned; the packed rows of the round
 *  k_cache, v_cache [num_pages, page_size, H_kv, d], DEVICE, 16-byte aligned
 *  page_table     [n_req, max_pages] int32 DEVICE
 *  req_block_off  [n_req + 1] int32 DEVICE (packed block offsets); prefix_len [n_req] int32 DEVICE,
 *                 read and updated; n_accepted [n_req] int32 DEVICE (clamped to [0, B-1])
 *  hit [n_req], packed_tokens [N_q], next_block [n_req, B] int32 DEVICE, all NULL or all given
 *  status [n_req] int32 DEVICE or NULL: 0 = committed; 1 = a slice row had no cache slot (page index
 *         past max_pages or page id outside [0, num_pages)): rows with a slot are still copied, and
 *         prefix_len grows only by the rows before the first row without one.
 * 1 <= B <= 256; H_kv * d * element size a multiple of 16. Errors: D3D_EINVAL on bad sizes or NULL
 * required pointers, D3D_EUNSUPPORTED on a row size that is not a multiple of 16 bytes.
 * ------------------------------------------------------------------------------------------- */
int kv_commit(d3d_dtype dtype, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
              const int32_t *page_table, int page_size, int max_pages, int num_pages,
              const int32_t *req_block_off, int32_t *prefix_len, const int32_t *n_accepted, int n_req,
              int block_size, int n_heads_kv, int head_dim, const int32_t *hit,
              const int32_t *packed_tokens, int32_t *next_block, int32_t *status, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Acceptance-weighted loss of drafter training ([DScout] 前置知识: 接受加权损失 AWL 与推测采样接受规则;
 * 方法步骤详情 step 4). For block r and future position k (0..n_pos-1), with P / Q the softmaxes of
 * the target / draft logits (temperature 1) and y the draft token:
 *   alpha_{r,k} = min(1, P(y) / Q(y))  (1 when Q(y) = 0);  w_{r,k} = prod_{j<k} alpha_{r,j}, w_{r,0} = 1
 *   L = sum I w CE / (sum I w + eps),  CE = -log Q(y*)
 * and, when grad is given, dL/dz^Q = I w / (sum I w + eps) * (Q - onehot(y*)) (w is a stop-gradient;
 * the target receives no gradient). Precision as in spec_verify: fp32 exp per element, fp64
 * accumulation, fp64 scalars; the gradient is computed in fp32 and stored in the logits' dtype.
 *
 *  target_logits, draft_logits [n_blocks, n_pos, vocab] (dtype) DEVICE; 1 <= n_pos <= 63
 *  draft_tokens, labels [n_blocks, n_pos] int32 DEVICE (clamped to [0, vocab)); include the same
 *  shape int32 DEVICE (0 = not in the loss) or NULL (all); eps >= 0 (the pages use 1e-6)
 *  outputs DEVICE: weights [n_blocks, n_pos] f32, ce the same or NULL, loss one double,
 *  grad [n_blocks, n_pos, vocab] (dtype) or NULL
 *  ws: at least awl_loss_workspace(n_blocks, n_pos, vocab) bytes; no initial contents required.
 * Errors: D3D_EINVAL on bad sizes, eps or NULL required pointers; D3D_EWORKSPACE.
 * ------------------------------------------------------------------------------------------- */
size_t awl_loss_workspace(int n_blocks, int n_pos, int vocab);
int awl_loss(d3d_dtype dtype, const void *target_logits, const void *draft_logits,
             const int32_t *draft_tokens, const int32_t *labels, const int32_t *include, int n_blocks,
             int n_pos, int vocab, double eps, float *weights, float *ce, double *loss, void *grad,
             void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Training-time packed attention ([D3D] 方法步骤详情 step 2, 核心方法; [DScout] 方法步骤详情 step 2).
 * One response of L tokens followed by n_blocks diffusion blocks of block_size rows (block i at
 * packed rows L + i*block_size .., its anchor at response position anchors[i]). A response row p
 * attends to response keys j <= p; a row of block i attends to response keys j < anchors[i]
 * (clamped to [0, L]) and to every row of block i; no row attends to another block. Query head h
 * uses key / value head h / (n_heads_q / n_heads_kv).
 *
 *  q, out, dout, dq [N, n_heads_q, head_dim], k, v, dk, dv [N, n_heads_kv, head_dim] (bf16, DEVICE),
 *  N = L + n_blocks * block_size; lse [N, n_heads_q] f32 DEVICE (natural log of the row's partition
 *  sum of scale * q.k); anchors [n_blocks] int32 DEVICE. Blocks packed in increasing anchor order
 *  run fastest (any order is computed correctly).
 *  Supported: bf16, head_dim 128, (n_heads_q / n_heads_kv) dividing 32, n_blocks <= 2048,
 *  N * n_heads_q * head_dim * 2 < 2^31 bytes; otherwise D3D_EUNSUPPORTED.
 *  train_attn_fwd writes out and lse. train_attn_bwd takes the forward's out and lse and the upstream
 *  gradient dout and writes dq, dk, dv (fp32 accumulation); ws: at least
 *  train_attn_workspace(L, n_blocks, block_size, n_heads_q, n_heads_kv) bytes (per-row
 *  rowsum(dout * out) and the fp32 partial key / value gradients of the query-tile chunks); no
 *  initial contents required. train_attn_workspace returns 0 for an unsupported shape.
 * Errors: D3D_EINVAL on bad sizes or NULL required pointers, D3D_EWORKSPACE, D3D_EUNSUPPORTED.
 * ------------------------------------------------------------------------------------------- */
size_t train_attn_workspace(int L, int n_blocks, int block_size, int n_heads_q, int n_heads_kv);
int train_attn_fwd(d3d_dtype dtype, const void *q, const void *k, const void *v, const int32_t *anchors, int L,
                   int n_blocks, int block_size, int n_heads_q, int n_heads_kv, int head_dim, float scale, void *out,
                   float *lse, hipStream_t stream);
int train_attn_bwd(d3d_dtype dtype, const void *q, const void *k, const void *v, const void *out, const void *dout,
                   const float *lse, const int32_t *anchors, int L, int n_blocks, int block_size, int n_heads_q,
                   int n_heads_kv, int head_dim, float scale, void *dq, void *dk, void *dv, void *ws,
                   size_t ws_bytes, hipStream_t stream);

const char *d3d_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* D3D_H */
