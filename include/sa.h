/*
 * sa.h -- C ABI of libsa.so: block-sparse attention forward on MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *  - "Sparse Attention" glossary (Ultralytics), section on common sparsity
 *    patterns: a query scores only a chosen subset of keys -- a causal
 *    sliding window, strided keys, global tokens, random links, attention
 *    sinks, or keys picked by content (DeepSeek Sparse Attention: an indexer
 *    scores every earlier token and the 2,048 best are attended).
 *  - same page, section on turning a pattern into savings: masking a dense
 *    score matrix still computes every score; speed comes from kernels that
 *    skip empty tiles; the mask is split into fixed blocks (128 x 128 in the
 *    example) and the sparsity is the share of blocks with no allowed pair.
 *  - blog "Sparse transformers: how to cut the O(n^2) of attention"
 *    (1gpt.online), section on how it looks in code: scores q.k^T/sqrt(d),
 *    disallowed pairs at -inf, softmax, product with V.
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller allocates and owns every buffer.  Pointers named
 *    "device" must be device memory of the current HIP device; the library
 *    keeps no device allocation of its own.
 *  - Asynchrony: all work is enqueued on `stream` (a hipStream_t; NULL is the
 *    null stream).  Nothing synchronises the host.
 *  - Errors: invalid arguments are rejected on the host before any launch
 *    (SA_ERR_INVALID_ARG / SA_ERR_UNSUPPORTED), so a rejected call writes
 *    nothing.  A failed launch returns SA_ERR_DEVICE.  sa_last_error()
 *    returns a thread-local description of the last non-OK status.  No call
 *    aborts or lets an exception escape.
 *  - Positions are absolute: query row r has position q_offset + r; key row
 *    s has position s.  All sizes and positions must fit in int32 (< 2^31);
 *    where a pattern is evaluated (sa_build_block_mask, sa_attn_fwd block
 *    mode), q_offset + n_q + n_kv must stay below 2^29.  In sa_attn_fwd,
 *    (n_kv + 256) times the larger K/V row stride in bytes must stay below
 *    2^31 (key rows are addressed with 32-bit byte offsets).
 *  - bfloat16 tensors are passed as raw 16-bit storage.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 2

typedef enum sa_status {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = 1,
    SA_ERR_UNSUPPORTED = 2,
    SA_ERR_DEVICE = 3
} sa_status;

enum { SA_DTYPE_BF16 = 0, SA_DTYPE_F32 = 1 };
enum { SA_MODE_BLOCKS = 0, SA_MODE_GATHER = 1, SA_MODE_STRIDED = 2 };

/*
 * Pattern descriptor.  A pair (q, kv) of absolute positions is allowed when
 *
 *     (!causal || kv <= q) && (local || sink || strided || global || unitband || random)
 *
 *   local    window_left >= 0 && q - kv <= window_left && kv - q <= window_right
 *   sink     kv < sinks
 *   strided  stride > 0 && q >= kv && (q - kv) % stride == stride_phase
 *   global   q < global_tokens || kv < global_tokens
 *   unitband unit > 0 && unit_window >= 0 && |q/unit - kv/unit| <= unit_window
 *   random   unit > 0 && kv/unit is one of rand_units[(q/unit)*n_rand + 0..n_rand-1]
 *            (rows q/unit >= rand_rows have no random units; -1 entries are empty)
 *
 * The terms are the glossary's fixed patterns (section on common sparsity
 * patterns) and the blog's templates (section on the main sparsity
 * templates; combining them is the norm, per the section that follows).
 * The glossary's example mask (causal, q - kv <= 1024 or kv < 4) is
 * causal=1, window_left=1024, window_right=0, sinks=4.
 *
 * rand_units is a DEVICE pointer (int32, rand_rows x n_rand, row-major),
 * NULL when n_rand == 0.  n_rand <= 4.
 */
typedef struct sa_pattern {
    int64_t causal;
    int64_t q_offset;
    int64_t window_left;
    int64_t window_right;
    int64_t sinks;
    int64_t stride;
    int64_t stride_phase;
    int64_t global_tokens;
    int64_t unit;
    int64_t unit_window;
    const int32_t *rand_units;
    int64_t n_rand;
    int64_t rand_rows;
} sa_pattern;

/*
 * sa_build_block_mask -- mask to per-query-block lists of live key blocks.
 * ("Sparse Attention" glossary, section on turning a pattern into savings:
 * the mask split into blocks, the blocks holding no allowed pair skipped.)
 *
 * The score matrix n_q x n_kv is cut into tiles of block_q x block_kv (the
 * last row/column of tiles clipped to the matrix).  For every tile the
 * number of allowed pairs is counted; a tile is live when the count is > 0,
 * full when it equals the clipped tile size, partial otherwise.
 *
 * Outputs (DEVICE pointers, caller-allocated, nqb = ceil(n_q/block_q),
 * nkb = ceil(n_kv/block_kv)):
 *   kv_count   int32 [nqb]         live key blocks of query block i
 *   kv_index   int32 [nqb * nkb]   row i: live key-block ids ascending, then -1
 *   kv_partial uint8 [nqb * nkb]   aligned with kv_index: 1 partial, 0 full/pad
 *   live_pairs int64 [1]           total allowed pairs over the whole matrix
 * block_q and block_kv must be multiples of 32 in [32, 1024].
 */
sa_status sa_build_block_mask(const sa_pattern *pattern, int64_t n_q, int64_t n_kv,
                              int32_t block_q, int32_t block_kv, int32_t *kv_count,
                              int32_t *kv_index, uint8_t *kv_partial, int64_t *live_pairs,
                              void *stream);

/*
 * Arguments of sa_attn_fwd.  All tensor pointers are DEVICE pointers.
 *
 *   q [batch, heads, n_q, head_dim], k/v [batch, heads, n_kv, head_dim]
 *     bfloat16, element strides {batch, head, row} in *_strides; the last
 *     dimension is contiguous; row strides and base addresses 16-byte aligned.
 *   o [batch, heads, n_q, head_dim] with o_strides, dtype o_dtype.
 *   lse float32 [batch, heads, n_q] contiguous, natural-log logsumexp of the
 *     scaled allowed scores (-inf for a row with no allowed key); may be NULL.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim) (the blog's scaling).
 *   head_dim is 64 or 128.
 *
 * mode SA_MODE_BLOCKS: block lists from sa_build_block_mask for the same
 *   pattern, n_q, n_kv, block_q, block_kv (shared by every batch and head).
 *   Only live tiles are visited; the pattern is evaluated per pair only on
 *   partial tiles (and on tiles clipped by n_kv).  block_q must be 64 or 128
 *   and block_kv 64 or 128.  With per_head_lists = 1 every (b, h) has lists
 *   of its own (as sa_select_blocks writes them): kv_count at
 *   (b*heads + h)*nqb, kv_index and kv_partial at (b*heads + h)*nqb*nkb;
 *   a pair is then attended when its tile is listed for the row's (b, h,
 *   query block) and, on a tile marked partial, the pattern allows it.
 * mode SA_MODE_GATHER: per-query key lists gather_idx int32 [n_q, topk]
 *   (row r lists key rows for query row r; entries < 0 or >= n_kv are
 *   skipped), shared by every batch and head when gather_bh_stride == 0,
 *   otherwise list of (b, h) starts at (b*heads + h) * gather_bh_stride.
 *   The pattern and block fields are ignored.  (Glossary, section on common
 *   sparsity patterns: full attention over the indexer's selected tokens.)
 * mode SA_MODE_STRIDED: the strided template of the blog "Sparse
 *   transformers: how to cut the O(n^2) of attention" (section on the main
 *   sparsity templates: near neighbours plus keys at a fixed step) --
 *   pattern causal, window_left = stride - 1, window_right = 0,
 *   stride_phase = stride - 1 and no other term, q_offset 0, n_q == n_kv a
 *   multiple of stride with n_q >= 3 * stride -- computed as two disjoint
 *   key sets per row: the local band through block lists, and the strided
 *   keys as plain causal attention between strided views of the same
 *   tensors (one per head and key residue; residue 0's view also holds the
 *   last row); the second part is merged into the first with log-sum-exp
 *   weights.  O must be float32 and
 *   lse non-NULL; block_q, block_kv and the list pointers are ignored: the
 *   block lists of the parts are read from `workspace` (at least
 *   sa_attn_workspace_bytes bytes, 256-byte aligned), where
 *   sa_attn_strided_plan has built them for the same pattern and n_q
 *   (batch, heads, head_dim, strides and tensors may differ between calls).
 *   Other patterns are rejected (SA_ERR_INVALID_ARG); they run in
 *   SA_MODE_BLOCKS.
 */
typedef struct sa_attn_args {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    int64_t batch;
    int64_t heads;
    int64_t n_q;
    int64_t n_kv;
    int64_t head_dim;
    int64_t o_dtype;
    int64_t q_strides[3];
    int64_t k_strides[3];
    int64_t v_strides[3];
    int64_t o_strides[3];
    double softmax_scale;
    int64_t mode;
    int64_t block_q;
    int64_t block_kv;
    const int32_t *kv_count;
    const int32_t *kv_index;
    const uint8_t *kv_partial;
    sa_pattern pattern;
    const int32_t *gather_idx;
    int64_t topk;
    int64_t gather_bh_stride;
    void *workspace;            /* DEVICE scratch or NULL, see sa_attn_workspace_bytes */
    int64_t workspace_bytes;
    int64_t per_head_lists;     /* SA_MODE_BLOCKS: 0 shared lists, 1 lists per (b, h) */
} sa_attn_args;

/*
 * Arguments of sa_select_blocks: content-selected key blocks, the glossary's
 * Native Sparse Attention "selection of the most relevant blocks" ("Sparse
 * Attention", section on common sparsity patterns), with a list per (b, h)
 * since heads differ in what they attend to (blog "Sparse transformers: how
 * to cut the O(n^2) of attention", section on combining templates).  The
 * pages give no formula; per (b, h, query block i) with query positions
 * p0 .. p1 (row r at q_offset + r):
 *   mean query qm_i and mean key km_j of key block j: fp64 sums of the
 *   block's rows in row order divided by the block size (rows past the end
 *   count as zero);  score(i, j) = qm_i . km_j, an fp64 fma chain over the
 *   head dim;
 *   kept: the key blocks holding positions p0 .. p1, plus the n_select
 *   blocks j with j*block_kv <= p1 (causally reachable) first in the order
 *   (score descending, block ascending).
 * Outputs (DEVICE, caller-allocated; nqb = ceil(n_q/block_q), nkb =
 * ceil(n_kv/block_kv) <= 1024):
 *   kv_count   int32 [batch*heads, nqb]
 *   kv_index   int32 [batch*heads, nqb, nkb]  kept blocks ascending, -1 pad
 *   kv_partial uint8 [batch*heads, nqb, nkb]  1: some pair of the clipped
 *              tile is not causal (key position > query position)
 *   live_pairs int64 [1]  causal pairs over all kept tiles
 * q, k: bfloat16 [batch, heads, n, head_dim] with element strides (b, h,
 * row), head_dim 64 or 128; block_q, block_kv 64 or 128.  workspace: at
 * least sa_select_blocks_workspace bytes, 256-byte aligned.  Attention over
 * the result: sa_attn_fwd, SA_MODE_BLOCKS, per_head_lists = 1, the same
 * block sizes and the pattern {causal = 1, q_offset, window_left = n_kv}.
 */
typedef struct sa_select_args {
    const void *q;
    const void *k;
    int64_t batch;
    int64_t heads;
    int64_t n_q;
    int64_t n_kv;
    int64_t head_dim;
    int64_t q_strides[3];
    int64_t k_strides[3];
    int64_t q_offset;
    int64_t block_q;
    int64_t block_kv;
    int64_t n_select;
    int32_t *kv_count;
    int32_t *kv_index;
    uint8_t *kv_partial;
    int64_t *live_pairs;
    void *workspace;
    int64_t workspace_bytes;
} sa_select_args;

/* Bytes of DEVICE scratch sa_select_blocks needs (the fp64 block means); 0
 * for sizes it does not take. */
size_t sa_select_blocks_workspace(const sa_select_args *args);

/* sa_select_blocks -- the content-selected lists above.  Asynchronous on
 * `stream`; invalid arguments are rejected before any launch. */
sa_status sa_select_blocks(const sa_select_args *args, void *stream);

/*
 * sa_attn_workspace_bytes -- bytes of device scratch that sa_attn_fwd needs
 * (SA_MODE_STRIDED: the block lists of its parts; 0 if the pattern is not
 * the strided template) or that let it take its split form (gather mode;
 * block mode with a long-row split), 0 when it has none.
 *
 * Block mode, lists shared by every (b, h), pattern not causal with
 * global_tokens > 0 and more than 8 key blocks: a query row below
 * global_tokens attends to every key (glossary, section on common sparsity
 * patterns: global tokens attend to all), so the query blocks holding such
 * rows list every key block.  Each of those blocks is walked in chunks of 8
 * list entries by separate workgroups, which write the chunk's normalised O
 * and LSE to the workspace ([batch*heads][blocks][chunks][block_q] rows of
 * head_dim floats, then one float per row); a second launch merges the
 * chunks of a row with log-sum-exp weights into O and LSE.  The result is
 * the same softmax; only the order of the float32 sums differs.
 *
 * Gather mode over a long key range (n_kv above 2^22 / (4 * head_dim)
 * keys, at most 256 ranges, batch * heads * ranges * n_q below 2^31) has a
 * split form: each key list is first partitioned by key range
 * (ranges of 4 MB of K and V per head), every range is then attended to
 * separately by workgroups that share it in one L2 cache, and the partial
 * results (running max, sum and unnormalised output per range) are merged.
 * The result is the same softmax; only the order of the float32 sums
 * differs.  The scratch holds the partitioned lists and the partial results.
 * With workspace == NULL sa_attn_fwd uses the single-pass form instead; a
 * non-NULL workspace smaller than this is an error.  The workspace is
 * overwritten by the call and must not overlap any other argument; calls
 * sharing one workspace must not run concurrently.
 */
size_t sa_attn_workspace_bytes(const sa_attn_args *args);

/*
 * sa_attn_strided_plan -- the block lists of SA_MODE_STRIDED's two parts
 * (band, residue views) into args->workspace, built once for a
 * pattern and length and read by every later sa_attn_fwd in that mode.  Uses
 * mode (must be SA_MODE_STRIDED), pattern, n_q, n_kv, the K/V row strides
 * (for the offset limit), workspace and workspace_bytes of `args`; rejects
 * what sa_attn_fwd would reject for these fields.  Asynchronous on `stream`.
 */
sa_status sa_attn_strided_plan(const sa_attn_args *args, void *stream);

/*
 * sa_attn_fwd -- O = softmax(Q K^T * scale restricted to allowed pairs) V, and LSE.
 * Computed in bfloat16 MFMA products with float32 accumulation; the softmax
 * runs in float32 (online over the visited tiles).  Returns as described in
 * the conventions above.
 */
sa_status sa_attn_fwd(const sa_attn_args *args, void *stream);

/*
 * sa_indexer_scores -- indexer score of query row r (position t = q_offset + r)
 * against every earlier key s <= t: a float32 fused-multiply-add chain over
 * the d_idx products in index order (the glossary's DeepSeek Sparse
 * Attention indexer, section on common sparsity patterns; the pages give no
 * formula, the plain dot product is used).
 *   q_idx bf16 [n_q, d_idx], k_idx bf16 [n_kv, d_idx] (DEVICE, contiguous)
 *   scores float32 [n_q, n_kv] (DEVICE): entries s <= min(t, n_kv-1) are
 *   written; the others are left untouched.
 * d_idx must be a multiple of 8 in [8, 256].
 */
sa_status sa_indexer_scores(const void *q_idx, const void *k_idx, int64_t n_q, int64_t n_kv,
                            int32_t d_idx, int64_t q_offset, float *scores, void *stream);

/*
 * sa_topk -- per query row, the topk candidates first in the total order
 * (score descending, key index ascending); candidates of row r are
 * s = 0 .. min(q_offset + r, n_kv - 1).  Output idx int32 [n_q, topk]
 * (DEVICE): the selected key indices in ascending order, -1 padded when a
 * row has fewer candidates.  -0.0 and +0.0 compare equal; a NaN score of
 * either sign ranks above every number, and NaNs tie with each other.
 * topk in [1, 4096], n_kv <= 65536.
 */
sa_status sa_topk(const float *scores, int64_t n_q, int64_t n_kv, int64_t q_offset, int32_t topk,
                  int32_t *idx_out, void *stream);

/*
 * sa_indexer_topk_workspace -- bytes of DEVICE scratch that sa_indexer_topk
 * needs when it streams (scores_out == NULL), 0 when these sizes have no
 * streaming form (n_q <= 0, n_kv <= 0, n_kv > 65536, topk outside
 * [1, 4096]).  At n_q = 1024, n_kv = 65536 it is about 66 MB, against 268 MB
 * for the score matrix the two-step form writes.
 */
size_t sa_indexer_topk_workspace(int64_t n_q, int64_t n_kv, int32_t topk);

/*
 * sa_indexer_topk -- the indexer and the top-k of DeepSeek Sparse Attention
 * ("Sparse Attention" glossary, section on common sparsity patterns: every
 * earlier token is scored, the topk best are attended) in one call.  Scores
 * and the order are exactly those of sa_indexer_scores and sa_topk, so the
 * selection is bit for bit the same either way.
 *
 *   scores_out != NULL: two steps, sa_indexer_scores into scores_out (float32
 *     [n_q, n_kv], DEVICE) followed by sa_topk; workspace is ignored.
 *   scores_out == NULL: streaming, no score matrix.  A 1/32 sample of each
 *     row's scores sets a threshold below the k-th best; one pass over the
 *     keys keeps the (score, index) of every candidate above it in the
 *     workspace; an exact selection among the kept candidates gives the
 *     top-k.  A row whose sample misleads (an adversarial order) is selected
 *     exactly from recomputed scores instead, so the result never depends on
 *     the data's order, only the time does.  workspace: DEVICE scratch of at
 *     least sa_indexer_topk_workspace(n_q, n_kv, topk) bytes, 256-byte
 *     aligned, owned by the caller, overwritten by the call; calls sharing
 *     one workspace must not run concurrently.
 * idx_out int32 [n_q, topk] (DEVICE): as sa_topk.  Limits: those of
 * sa_indexer_scores and sa_topk (d_idx a multiple of 8 in [8, 256], topk in
 * [1, 4096], n_kv <= 65536).
 */
sa_status sa_indexer_topk(const void *q_idx, const void *k_idx, int64_t n_q, int64_t n_kv,
                          int32_t d_idx, int64_t q_offset, int32_t topk, float *scores_out,
                          int32_t *idx_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sa_indexer_topk_noalloc -- the streaming sa_indexer_topk (scores_out NULL)
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Its
 * scratch is a fixed array of SA_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per device, held until the process ends; its address is
 * looked up on the first call on each device.  The call allocates nothing.
 * Sizes whose sa_indexer_topk_workspace exceeds the array are rejected with
 * SA_ERR_UNSUPPORTED (n_q = 1024, n_kv = 65536 fits).  Every call on one
 * device uses that device's one array and leaves its contents behind: calls
 * that overlap on a device (several streams or threads) race, so the caller
 * must order them.  Arguments, outputs and limits otherwise as
 * sa_indexer_topk.
 */
#define SA_NOALLOC_SCRATCH_BYTES (64ll << 20)
sa_status sa_indexer_topk_noalloc(const void *q_idx, const void *k_idx, int64_t n_q, int64_t n_kv,
                                  int32_t d_idx, int64_t q_offset, int32_t topk, int32_t *idx_out,
                                  void *stream);

/*
 * sa_merge_partial -- fold a second partial attention result into a first,
 * for key sets that are split into two disjoint parts per query row:
 *     O = (e^l1 O1 + e^l2 O2) / (e^l1 + e^l2),   LSE = log(e^l1 + e^l2)
 * (log-sum-exp algebra on the masked softmax of the blog "Sparse
 * transformers: how to cut the O(n^2) of attention", section on how it
 * looks in code; its strided template, section on the main sparsity
 * templates, splits into the local band and the strided keys).
 *   o      float32 (DEVICE), in/out: row (b, h, q) at
 *          o + b*o_strides[0] + h*o_strides[1] + q*o_strides[2], head_dim
 *          contiguous columns; the first part's O on entry, the merged O on
 *          return;
 *   lse    float32 [batch, heads, n] (DEVICE, contiguous), in/out, natural
 *          log; -inf marks a row without keys;
 *   o2     float32 (DEVICE), the second part's O at (b, h, q) with o2_strides;
 *          must not overlap o;
 *   lse2   float32 (DEVICE): row q = q_first + i*group + r (0 <= r < group,
 *          0 <= i < n2) has a second part, whose LSE is at
 *          lse2[((b*heads + h)*group + r)*n2 + i]; every other row is left
 *          unchanged (group = 1, q_first = 0, n2 = n: the natural
 *          [batch, heads, n] layout; group = stride: the layout that
 *          sa_attn_fwd writes for residue views of a strided pattern).
 * o and o2 16-byte aligned with strides that are multiples of 4 elements;
 * head_dim 64 or 128; group >= 1; q_first + (n2 - 1)*group < n.  A row where
 * both LSEs are -inf is left unchanged.  Asynchronous on `stream`;
 * allocates nothing.
 */
sa_status sa_merge_partial(float *o, float *lse, const float *o2, const float *lse2, int64_t batch,
                           int64_t heads, int64_t n, int32_t head_dim, const int64_t o_strides[3],
                           const int64_t o2_strides[3], int32_t group, int64_t q_first, int64_t n2,
                           void *stream);

/*
 * Arguments of sa_attn_bwd: the gradients of sa_attn_fwd's block mode with
 * respect to Q, K and V for an upstream gradient dO, by the chain rule on
 * the blog's masked attention ("Sparse transformers: how to cut the O(n^2)
 * of attention", section on how it looks in code; the "Sparse Attention"
 * glossary notes Native Sparse Attention is trained end to end):
 *   P = exp(s*scale - LSE) on allowed pairs,  D = rowsum(dO * O),
 *   dS = P * (dO . v - D),  dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q.
 * Every tensor is a contiguous DEVICE array [batch, heads, n, head_dim]:
 *   q, dout bfloat16 (n = n_q); k, v bfloat16 (n = n_kv);
 *   o float32 and lse float32 [batch, heads, n_q]: the forward's outputs for
 *   the same inputs, lists and pattern;
 *   dq float32 (n_q), dk, dv float32 (n_kv): written, every row (rows that
 *   no allowed pair touches get 0).
 * The block lists, pattern, block sizes and per_head_lists are those of the
 * forward call (block_q, block_kv 64 or 128; head_dim 64 or 128).  P and dS
 * enter the matrix products as bfloat16, products accumulate in float32.
 * workspace: at least sa_attn_bwd_workspace bytes, 256-byte aligned.
 */
typedef struct sa_attn_bwd_args {
    const void *q;
    const void *k;
    const void *v;
    const float *o;
    const float *lse;
    const void *dout;
    float *dq;
    float *dk;
    float *dv;
    int64_t batch;
    int64_t heads;
    int64_t n_q;
    int64_t n_kv;
    int64_t head_dim;
    double softmax_scale;
    int64_t block_q;
    int64_t block_kv;
    const int32_t *kv_count;
    const int32_t *kv_index;
    const uint8_t *kv_partial;
    int64_t per_head_lists;
    sa_pattern pattern;
    void *workspace;
    int64_t workspace_bytes;
} sa_attn_bwd_args;

/* Bytes of DEVICE scratch sa_attn_bwd needs (D per row and the block lists
 * transposed); 0 for sizes it does not take. */
size_t sa_attn_bwd_workspace(const sa_attn_bwd_args *args);

/* sa_attn_bwd -- dQ, dK, dV as above.  Asynchronous on `stream`; invalid
 * arguments are rejected before any launch. */
sa_status sa_attn_bwd(const sa_attn_bwd_args *args, void *stream);

/* Thread-local text of the last non-OK status of this thread ("" if none). */
const char *sa_last_error(void);

/* SA_ABI_VERSION of the library. */
int32_t sa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
