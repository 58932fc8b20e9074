// sa_internal.h -- device-side pattern evaluation and launcher declarations.
//
// The pattern is the union of fixed terms described in the "Sparse Attention"
// glossary (section on common sparsity patterns) and the sparse-transformer
// blog (section on the main sparsity templates), intersected with causality;
// its fields and their meaning are those of sa_pattern in include/sa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace sa {

// Exact unsigned division by an invariant divisor s >= 1 for 0 <= n < 2^31:
// with l = ceil(log2 s) and M = ceil(2^(31+l) / s), floor(n / s) equals
// (n * M) >> (31 + l).  (M*n/2^(31+l) = n/s + e*n/(s*2^(31+l)) with
// 0 <= e < s; the excess is below 2^-l <= 1/s, so the floor is unchanged.)
struct FastDiv {
    uint64_t mul;
    int32_t shift;
    int32_t div;
};

inline FastDiv make_fastdiv(int64_t s)
{
    FastDiv f{};
    if (s < 1) s = 1;
    int l = 0;
    while ((int64_t(1) << l) < s) ++l;
    f.shift = 31 + l;
    unsigned __int128 num = (unsigned __int128)1 << f.shift;
    f.mul = (uint64_t)((num + (unsigned __int128)s - 1) / (unsigned __int128)s);
    f.div = (int32_t)s;
    return f;
}

__device__ __forceinline__ int32_t fdiv(int32_t n, const FastDiv& f)
{
    return (int32_t)(((uint64_t)(uint32_t)n * f.mul) >> f.shift);
}

__device__ __forceinline__ int32_t fmod_(int32_t n, const FastDiv& f)
{
    return n - fdiv(n, f) * f.div;
}

// Pattern as the kernels see it: 32-bit positions, precomputed divisors.
struct DevPattern {
    int32_t causal;
    int32_t q_offset;
    int32_t window_left;   // < 0: local term off
    int32_t window_right;
    int32_t sinks;
    int32_t stride;        // <= 0: strided term off
    int32_t stride_phase;
    int32_t global_tokens;
    int32_t unit;          // <= 0: unit terms off
    int32_t unit_window;   // < 0: unit band off
    int32_t max_unit;      // larger unit indices cannot hold a key
    int32_t n_kv;          // keys at or past n_kv do not exist
    int32_t n_rand;
    int32_t rand_rows;
    const int32_t *rand_units;
    FastDiv stride_div;
    FastDiv unit_div;
    uint64_t stride_bits;  // bits at 0, stride, 2*stride, ... below 64
};

constexpr int kMaxRand = 4;

// Per-query quantities that do not change along a query row.
struct RowCtx {
    int32_t q;       // absolute query position
    int32_t qu;      // q / unit (0 if unit terms off)
    int32_t cap;     // keys >= cap are never allowed (causality, sequence end)
    int32_t wlo;     // local window [wlo, whi), already capped
    int32_t whi;
    int32_t rnd[kMaxRand];
};

__device__ __forceinline__ void row_ctx(const DevPattern& p, int32_t q, RowCtx& r)
{
    r.q = q;
    r.cap = p.causal ? min(q + 1, p.n_kv) : p.n_kv;
    r.wlo = q - p.window_left;
    r.whi = min(q + p.window_right + 1, r.cap);
    r.qu = p.unit > 0 ? fdiv(q, p.unit_div) : 0;
#pragma unroll
    for (int i = 0; i < kMaxRand; ++i) {
        const int32_t v = (i < p.n_rand && p.unit > 0 && r.qu < p.rand_rows)
                              ? p.rand_units[(int64_t)r.qu * p.n_rand + i]
                              : -1;
        r.rnd[i] = v > p.max_unit ? -1 : v;  // beyond every key: same as empty
    }
}

// (2^w - 1) << a for w, a in [0, 31] (one v_bfm_b32)
__device__ __forceinline__ uint32_t bit_field_mask(uint32_t w, uint32_t a)
{
    uint32_t r;
    asm("v_bfm_b32 %0, %1, %2" : "=v"(r) : "v"(w), "v"(a));
    return r;
}

// Bits [lo, hi) of the 32-key chunk [k0, k0 + 32), positions clamped to it;
// branch-free.  Callers keep lo, hi, k0 within int32 (the host clamps the
// pattern fields to the sequence sizes).
__device__ __forceinline__ uint32_t range_bits32(int32_t lo, int32_t hi, int32_t k0)
{
    const int32_t a = min(max(lo - k0, 0), 32);
    const int32_t b = min(max(hi - k0, 0), 32);
    const int32_t w = max(b - a, 0);  // w == 32 only when a == 0
    const uint32_t m = bit_field_mask((uint32_t)w & 31u, (uint32_t)a & 31u);
    return w >= 32 ? 0xFFFFFFFFu : m;
}

// Allowed keys among [k0, k0 + 32) for the query of `r`, as a bit mask (bit i
// = key k0 + i), keys past the sequence end excluded.  Every pattern term is
// an interval of keys for a fixed query, or for the strided term an
// arithmetic progression; each is cut at the row's causal / sequence cap, so
// the mask costs a few integer operations per term instead of 32 predicate
// evaluations.  Terms that are off cost nothing (uniform branches).
__device__ __forceinline__ uint32_t allowed_bits32(const DevPattern& p, const RowCtx& r, int32_t k0)
{
    const int32_t q = r.q;
    uint32_t m = 0;
    if (p.sinks > 0) m |= range_bits32(0, min(p.sinks, r.cap), k0);
    if (p.window_left >= 0) m |= range_bits32(r.wlo, r.whi, k0);
    if (p.global_tokens > 0) m |= range_bits32(0, q < p.global_tokens ? r.cap : min(p.global_tokens, r.cap), k0);
    if (p.stride > 0) {
        // keys kv <= q - phase with (q - phase - kv) % stride == 0: the largest
        // such key in the chunk is `first`; the others sit stride apart below it
        const int32_t qp = q - p.stride_phase;
        const int32_t top = min(qp, k0 + 31);
        const int32_t back = fmod_(max(qp - top, 0), p.stride_div);
        const int32_t first = top - (back == 0 ? 0 : p.stride - back);
        const int32_t o = first - k0;  // bit of `first`
        const int32_t base = fmod_(max(o, 0), p.stride_div);
        const uint32_t below = (uint32_t)((2ull << max(o, 0)) - 1ull);
        const uint32_t prog = (uint32_t)(p.stride_bits << base) & below;
        m |= o >= 0 ? prog & range_bits32(0, r.cap, k0) : 0u;
    }
    if (p.unit > 0) {
        if (p.unit_window >= 0)
            m |= range_bits32((r.qu - p.unit_window) * p.unit, min((r.qu + p.unit_window + 1) * p.unit, r.cap), k0);
#pragma unroll
        for (int i = 0; i < kMaxRand; ++i) {
            if (i < p.n_rand) {
                const uint32_t b = range_bits32(r.rnd[i] * p.unit, min((r.rnd[i] + 1) * p.unit, r.cap), k0);
                m |= r.rnd[i] >= 0 ? b : 0u;
            }
        }
    }
    return m;
}

// ---- launchers (defined in the .hip files) --------------------------------

hipError_t launch_zero_i64(int64_t* p, hipStream_t stream);
hipError_t launch_block_mask(const DevPattern& p, int32_t n_q, int32_t n_kv, int32_t block_q,
                             int32_t block_kv, int32_t* kv_count, int32_t* kv_index,
                             uint8_t* kv_partial, int64_t* live_pairs, hipStream_t stream);

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    void* o;
    float* lse;
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int64_t lse_sb, lse_sh, lse_sn;  // element strides of LSE (b, h, row)
    int32_t batch, heads, n_q, n_kv;
    int32_t merge;      // block mode, float32 O: fold into the O and LSE already there
    int32_t n_q_rest;   // block mode: rows of heads 1.. when it differs from head 0's n_q (0: n_q)
    float scale;        // softmax scale (natural units)
    float scale_log2;   // scale * log2(e)
    // block mode
    int32_t nqb, nkb;
    const int32_t* kv_count;
    const int32_t* kv_index;
    const uint8_t* kv_partial;
    int32_t per_head_lists;  // lists of (b, h) at (b*heads + h) * nqb [* nkb]
    int32_t last_first;      // dispatch a head's query blocks from the last one
    // long-row split (block mode, shared lists): query blocks [0, split_q) are
    // walked as split_c chunks of split_e list entries each by separate
    // workgroups, which write normalised partial O and LSE to part_o /
    // part_lse ([batch*heads][split_q][split_c][block_q] rows); a merge
    // launch folds them into O and LSE.  split_q = 0: no split.
    int32_t split_q, split_c, split_e;
    float* part_o;
    float* part_lse;
    DevPattern pat;
    // gather mode
    const int32_t* gidx;
    int32_t topk;
    int64_t g_bh_stride;
    // split gather form (scratch from the caller): key ranges of 2^g_shift
    // keys, lists partitioned by range, partial results per range
    int32_t g_shift;
    int32_t g_nchunk;
    int32_t* g_lists;   // [rows][topk], rows = n_q (shared lists) or batch*heads*n_q
    int32_t* g_offs;    // [rows][g_nchunk + 1]
    float* g_po;        // [batch*heads*n_q][g_nchunk][head_dim]
    float* g_pml;       // [batch*heads*n_q][g_nchunk][2]: max (log2 units), sum
};

// Long-row split of block mode: the query blocks every key is visible from.
// Without causality a query row below global_tokens attends to every key, so
// the blocks holding such rows list every key block; with more than
// kSplitEntries key blocks they are split.  Returns split_q (0: none) and
// the chunk count and size.  Chunks of 8 entries are about as long as the
// other rows' lists of a BigBird-style pattern (window, global and random
// blocks: 7-8 entries), so the dispatcher balances them with the rest; on
// the BigBird-style workload chunks of 4, 6, 8, 16 and 32 entries measured
// 150, 132, 124, 156 and 182 us.
constexpr int32_t kSplitEntries = 8;
inline int32_t long_row_split(int64_t causal, int64_t global_tokens, int64_t q_offset, int64_t n_q, int64_t nqb,
                              int64_t nkb, int64_t block_q, int32_t& chunks, int32_t& per_chunk)
{
    chunks = per_chunk = 0;
    if (causal || global_tokens <= 0 || nkb <= kSplitEntries || nqb <= 0) return 0;
    const int64_t rows = std::min(global_tokens - q_offset, n_q);
    if (rows <= 0) return 0;
    const int64_t gq = std::min((rows + block_q - 1) / block_q, nqb);
    per_chunk = kSplitEntries;
    chunks = (int32_t)((nkb + kSplitEntries - 1) / kSplitEntries);
    return (int32_t)gq;
}
hipError_t launch_split_merge(const AttnParams& a, int head_dim, int block_q, int o_f32, hipStream_t stream);

hipError_t launch_attn_blocks(const AttnParams& a, int head_dim, int block_q, int block_kv,
                              int o_f32, hipStream_t stream);
hipError_t launch_attn_gather(const AttnParams& a, int head_dim, int o_f32, hipStream_t stream);
hipError_t launch_attn_gather_split(const AttnParams& a, int head_dim, int o_f32, hipStream_t stream);

// Layout of the split-gather scratch (byte offsets, each 256-byte aligned).
struct GatherSplitLayout {
    int32_t shift, nchunk;
    int64_t rows;
    int64_t lists, offs, po, pml, total;
};
inline bool gather_split_layout(int64_t batch, int64_t heads, int64_t n_q, int64_t n_kv, int64_t head_dim,
                                int64_t topk, int64_t bh_stride, GatherSplitLayout& L)
{
    // 4 MB of K and V rows per range and head, the L2 of one XCD (on the
    // DeepSeek-style workload ranges of 1, 2, 4 and 8 MB measured 1,018,
    // 823, 796 and 867 us for the whole gather)
    int32_t shift = 0;
    while ((int64_t(1) << (shift + 1)) * 4 * head_dim <= (int64_t(1) << 22)) ++shift;
    const int64_t nchunk = (n_kv + (int64_t(1) << shift) - 1) >> shift;
    if (nchunk < 2 || nchunk > 256 || batch <= 0 || heads <= 0 || n_q <= 0) return false;
    if (batch * heads * nchunk * n_q >= (int64_t(1) << 31)) return false;  // 32-bit work items
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    L.shift = shift;
    L.nchunk = (int32_t)nchunk;
    L.rows = bh_stride == 0 ? n_q : batch * heads * n_q;
    const int64_t items = batch * heads * n_q;
    L.lists = 0;
    L.offs = up(L.lists + L.rows * topk * 4);
    L.po = up(L.offs + L.rows * (nchunk + 1) * 4);
    L.pml = up(L.po + items * nchunk * head_dim * 4);
    L.total = up(L.pml + items * nchunk * 2 * 4);
    return true;
}
// Second partial result folded into the first (merge.hip).  Row (b, h, q) of
// the first part: o + b*o_sb + h*o_sh + q*o_sn (float32, head_dim columns),
// lse[(b*heads + h)*n + q].  Row q = q_first + i*group + r (0 <= r < group,
// 0 <= i < n2) takes the second part: o2 at the same (b, h, q) with its
// strides, and its LSE at lse2[((b*heads + h)*group + r)*n2 + i]; the other
// rows are left unchanged.
struct MergeParams {
    float* o;
    float* lse;
    const float* o2;
    const float* lse2;
    int64_t rows;  // batch * heads * n
    int64_t n, n2, heads, q_first;
    int64_t o_sb, o_sh, o_sn, o2_sb, o2_sh, o2_sn;
    int32_t group;
};
hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t stream);

// Streaming indexer + top-k (indexer_topk.hip): no score matrix.  Scratch
// layout (byte offsets, each 256-byte aligned):
//   samp  uint32 [n_q][s_max]            order keys of the sampled tiles
//   lo    uint32 [n_q]                   per-row keep threshold (0: direct)
//   cnt   uint32 [n_q][nchunk][2]        kept candidates per (row, chunk) and half-wave
//   tnorm float  [n_tiles]               largest key norm of every 64-key tile
//   kept  uint32 [n_q][nchunk][cap]      kept candidates: approximate score with
//                                        its low 9 bits dropped, position within
//                                        the chunk in those 9 bits; half-wave 0
//                                        fills from the front, 1 from the back
constexpr int kStreamPeriod = 2048;  // one 64-key sample tile per this many keys
constexpr int kStreamChunk = 512;    // keys per filter chunk
constexpr int kStreamCap = 72;       // kept slots per (row, chunk)
constexpr int64_t kStreamMaxKv = 65536;
struct StreamTopkLayout {
    int32_t s_max, nchunk, ntile;
    int64_t samp, lo, cnt, tnorm, kept, total;
};
inline bool stream_topk_layout(int64_t n_q, int64_t n_kv, StreamTopkLayout& L)
{
    if (n_q <= 0 || n_kv <= 0 || n_kv > kStreamMaxKv) return false;
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    L.s_max = (int32_t)(64 * ((n_kv + kStreamPeriod - 1) / kStreamPeriod));
    L.nchunk = (int32_t)((n_kv + kStreamChunk - 1) / kStreamChunk);
    const int64_t regions = n_q * L.nchunk;
    L.samp = 0;
    L.lo = up(L.samp + n_q * L.s_max * 4);
    L.ntile = (int32_t)((n_kv + 63) / 64);
    L.cnt = up(L.lo + n_q * 4);
    L.tnorm = up(L.cnt + regions * 2 * 4);
    L.kept = up(L.tnorm + (int64_t)L.ntile * 4);
    L.total = up(L.kept + regions * kStreamCap * 4);
    return true;
}
hipError_t launch_indexer_topk_stream(const uint16_t* q_idx, const uint16_t* k_idx, int32_t n_q, int32_t n_kv,
                                      int32_t d_idx, int32_t q_offset, int32_t topk, int32_t* idx_out,
                                      uint8_t* ws, const StreamTopkLayout& L, hipStream_t stream);

// The fixed per-device scratch of sa_indexer_topk_noalloc (its address on
// the current device; looked up once per device).
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;
hipError_t noalloc_scratch(uint8_t** ptr);

// Content-selected key blocks (block_select.hip).  Scratch: the fp64 mean
// query of every (b, h, query block) and mean key of every (b, h, key block).
constexpr int kSelectMaxBlocks = 1024;  // key blocks per row
struct SelectParams {
    const uint16_t* q;
    const uint16_t* k;
    int64_t q_sb, q_sh, q_sn, k_sb, k_sh, k_sn;
    int32_t batch, heads, n_q, n_kv, d, q_offset, bq, bk, nqb, nkb, n_sel;
    int32_t* kv_count;
    int32_t* kv_index;
    uint8_t* kv_partial;
    int64_t* live_pairs;
    double* qm;  // [batch*heads][nqb][d]
    double* km;  // [batch*heads][d][nkb]
};
inline int64_t select_workspace_bytes(int64_t bh, int64_t nqb, int64_t nkb, int64_t d)
{
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    return up(bh * nqb * d * 8) + up(bh * nkb * d * 8);
}
hipError_t launch_select_blocks(const SelectParams& p, hipStream_t stream);

// Backward (attn_bwd.hip).  Tensors contiguous [batch, heads, n, head_dim];
// scratch: D [batch*heads*n_q] and the block lists transposed (per key block,
// the query blocks that list it).
struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* o;
    const float* lse;
    float* dq;
    float* dk;
    float* dv;
    int32_t batch, heads, n_q, n_kv;
    float scale, scale_log2;
    int32_t nqb, nkb, per_head_lists, n_lists;
    const int32_t* kv_count;
    const int32_t* kv_index;
    const uint8_t* kv_partial;
    DevPattern pat;
    float* dsum;        // [batch*heads*n_q]
    int32_t* q_count;   // [n_lists][nkb]
    int32_t* q_index;   // [n_lists][nkb][nqb]
    uint8_t* q_partial; // [n_lists][nkb][nqb]
    int32_t* order_q;   // [n_lists*nqb] list rows, longest first
    int32_t* order_k;   // [n_lists*nkb] transposed rows, longest first
};
struct BwdLayout {
    int64_t dsum, q_count, q_index, q_partial, order_q, order_k, total;
};
inline BwdLayout bwd_layout(int64_t rows, int64_t n_lists, int64_t nqb, int64_t nkb)
{
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    BwdLayout L;
    L.dsum = 0;
    L.q_count = up(rows * 4);
    L.q_index = up(L.q_count + n_lists * nkb * 4);
    L.q_partial = up(L.q_index + n_lists * nkb * nqb * 4);
    L.order_q = up(L.q_partial + n_lists * nkb * nqb);
    L.order_k = up(L.order_q + n_lists * nqb * 4);
    L.total = up(L.order_k + n_lists * nkb * 4);
    return L;
}
hipError_t launch_attn_bwd(const BwdParams& a, int head_dim, int block_q, int block_kv, hipStream_t stream);

hipError_t launch_indexer_scores(const uint16_t* q_idx, const uint16_t* k_idx, int32_t n_q,
                                 int32_t n_kv, int32_t d_idx, int32_t q_offset, float* scores,
                                 hipStream_t stream);
hipError_t launch_topk(const float* scores, int32_t n_q, int32_t n_kv, int32_t q_offset,
                       int32_t topk, int32_t* idx_out, hipStream_t stream);

}  // namespace sa
