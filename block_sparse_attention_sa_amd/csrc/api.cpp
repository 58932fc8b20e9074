// api.cpp -- the C ABI of libsa.so (declared in include/sa.h): argument
// validation on the host, conversion to the kernels' parameter blocks, and
// launches on the caller's stream.  No device memory is allocated here.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/sa.h"
#include "sa_internal.h"

namespace {

thread_local std::string g_err;

sa_status fail(sa_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

sa_status ok()
{
    return SA_OK;
}

constexpr int64_t kI32Max = 2147483647LL;

int32_t clamp32(int64_t v)
{
    if (v > kI32Max) return (int32_t)kI32Max;
    if (v < -kI32Max) return (int32_t)-kI32Max;
    return (int32_t)v;
}

bool aligned16(const void* p)
{
    return ((uintptr_t)p & 15u) == 0;
}

// Validates the pattern and fills the kernels' form of it.
sa_status make_pattern(const sa_pattern* p, int64_t n_q, int64_t n_kv, sa::DevPattern& d)
{
    if (!p) return fail(SA_ERR_INVALID_ARG, "pattern is NULL");
    if (p->q_offset < 0) return fail(SA_ERR_INVALID_ARG, "pattern.q_offset must be >= 0");
    // kernels do position arithmetic in int32: q + n_kv must stay in range
    if (p->q_offset + n_q + n_kv + 64 > (int64_t(1) << 29))
        return fail(SA_ERR_UNSUPPORTED, "query positions plus n_kv must stay below 2^29");
    if (p->window_left >= 0 && p->window_right < 0)
        return fail(SA_ERR_INVALID_ARG, "pattern.window_right must be >= 0 when the window is on");
    if (p->sinks < 0 || p->global_tokens < 0)
        return fail(SA_ERR_INVALID_ARG, "pattern.sinks and pattern.global_tokens must be >= 0");
    if (p->stride > 0 && (p->stride_phase < 0 || p->stride_phase >= p->stride))
        return fail(SA_ERR_INVALID_ARG, "pattern.stride_phase must be in [0, stride)");
    if (p->stride > kI32Max || p->unit > kI32Max)
        return fail(SA_ERR_UNSUPPORTED, "pattern.stride / pattern.unit must be below 2^31");
    if (p->n_rand < 0 || p->n_rand > sa::kMaxRand)
        return fail(SA_ERR_UNSUPPORTED, "pattern.n_rand must be in [0, %d]", sa::kMaxRand);
    if ((p->n_rand > 0 || p->unit_window >= 0) && p->unit <= 0)
        return fail(SA_ERR_INVALID_ARG, "pattern.unit must be > 0 for unit-level terms");
    if (p->n_rand > 0 && (!p->rand_units || p->rand_rows < 0))
        return fail(SA_ERR_INVALID_ARG, "pattern.rand_units is NULL or rand_rows < 0");
    d = sa::DevPattern{};
    // Values beyond the sequence extents are clamped to them: positions never
    // exceed q_max (queries) or n_kv (keys), so the predicate is unchanged and
    // int32 arithmetic in the kernels cannot overflow.
    const int64_t q_max = p->q_offset + n_q;
    const int64_t ext = (q_max > n_kv ? q_max : n_kv) + 1;
    d.causal = p->causal != 0;
    d.q_offset = (int32_t)p->q_offset;
    d.window_left = p->window_left < 0 ? -1 : (int32_t)(p->window_left < ext ? p->window_left : ext);
    d.window_right = (int32_t)(p->window_right < 0 ? 0 : (p->window_right < ext ? p->window_right : ext));
    d.sinks = (int32_t)(p->sinks < ext ? p->sinks : ext);
    d.stride = p->stride > 0 ? (int32_t)(p->stride < ext ? p->stride : ext) : 0;
    d.stride_phase = (int32_t)(p->stride > 0 ? p->stride_phase : 0);
    if (d.stride > 0 && d.stride_phase >= d.stride) d.stride_phase = d.stride;  // phase beyond every distance
    d.global_tokens = (int32_t)(p->global_tokens < ext ? p->global_tokens : ext);
    d.unit = p->unit > 0 ? (int32_t)(p->unit < ext ? p->unit : ext) : 0;
    d.max_unit = d.unit > 0 ? (int32_t)(ext / d.unit + 1) : 0;
    d.n_kv = (int32_t)n_kv;
    d.unit_window = d.unit > 0 && p->unit_window >= 0
                        ? (int32_t)(p->unit_window < d.max_unit ? p->unit_window : d.max_unit)
                        : -1;
    d.n_rand = d.unit > 0 ? (int32_t)p->n_rand : 0;
    d.rand_rows = d.n_rand > 0 ? clamp32(p->rand_rows) : 0;
    d.rand_units = d.n_rand > 0 ? p->rand_units : nullptr;
    d.stride_div = sa::make_fastdiv(d.stride > 0 ? d.stride : 1);
    d.stride_bits = 0;
    if (d.stride > 0)
        for (int64_t b = 0; b < 64; b += d.stride) d.stride_bits |= 1ull << b;
    d.unit_div = sa::make_fastdiv(d.unit > 0 ? d.unit : 1);
    return SA_OK;
}

sa_status launched(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(SA_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// The strided template that sa_attn_fwd's SA_MODE_STRIDED computes as
// disjoint key sets (causal; local band q - kv <= S - 1; strided keys
// (q - kv) % S == S - 1; no other term; q_offset 0; n_q == n_kv a multiple of
// S with at least three groups of S rows): S, else 0.
int64_t strided_template(const sa_attn_args* a)
{
    const sa_pattern& p = a->pattern;
    const int64_t S = p.stride;
    if (S <= 0 || p.stride_phase != S - 1 || !p.causal || p.window_left != S - 1 || p.window_right != 0) return 0;
    if (p.sinks || p.global_tokens || p.unit > 0 || p.n_rand || p.q_offset) return 0;
    if (a->n_q != a->n_kv || a->n_q % S || a->n_q / S < 3) return 0;
    return S;
}

// Scratch of the strided form: the block lists of its two parts (band on
// the natural layout; the residue views, n/S - 1 rows (the last of them
// exists for residue 0 only) against all n/S key groups -- the causal mask
// drops the groups past each row, and a key range that is a multiple of the
// sub-tile keeps the copies on the fast path).
struct StridedLayout {
    struct Lists {
        int64_t n_q, n_kv, nqb, nkb, count, index, partial, live;
    } band, res;
    int64_t total;
};
constexpr int kStridedBlock = 64;

StridedLayout strided_layout(int64_t n, int64_t S)
{
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    StridedLayout L{};
    const int64_t G = n / S;
    int64_t at = 0;
    auto lists = [&](StridedLayout::Lists& l, int64_t n_q, int64_t n_kv) {
        l.n_q = n_q;
        l.n_kv = n_kv;
        l.nqb = (n_q + kStridedBlock - 1) / kStridedBlock;
        l.nkb = (n_kv + kStridedBlock - 1) / kStridedBlock;
        l.count = at;
        l.index = up(l.count + 4 * l.nqb);
        l.partial = up(l.index + 4 * l.nqb * l.nkb);
        l.live = up(l.partial + l.nqb * l.nkb);
        at = up(l.live + 8);
    };
    lists(L.band, n, n);
    lists(L.res, G - 1, G);
    L.total = at;
    return L;
}

// SA_MODE_STRIDED: the strided template as two disjoint key sets per query
// row (the blog "Sparse transformers: how to cut the O(n^2) of attention",
// section on the main sparsity templates; the masked softmax's log-sum-exp
// splits over disjoint key sets):
//   band     kv in [q - (S - 1), q], block lists on the natural layout;
//   residue  kv = q - (S - 1) - S*m (m >= 1): for each key residue rho the
//            rows q = (i + 2)*S + rho - 1 against keys j*S + rho, j <= i --
//            plain causal attention between strided views of the same
//            tensors (no copy), one view per (head, residue).  The views
//            hold n/S - 2 rows, except residue 0's, whose row n/S - 2 is
//            query row n - 1.
// The residue part is folded into the band's O and LSE in the attention
// kernel's epilogue.  The block lists of both (the plan) are built into the
// workspace by sa_attn_strided_plan.
struct StridedParts {
    int64_t S, G;
    StridedLayout W;
    sa_pattern pat[2];
    sa::DevPattern dev[2];
};

sa_status strided_check(const sa_attn_args* a, StridedParts& P)
{
    P.S = strided_template(a);
    if (!P.S)
        return fail(SA_ERR_INVALID_ARG, "SA_MODE_STRIDED: the pattern is not the strided template "
                                        "(causal, window_left = stride - 1, stride_phase = stride - 1, "
                                        "no other term, n_q == n_kv a multiple of stride >= 3 * stride)");
    const int64_t n = a->n_q;
    P.G = n / P.S;
    P.W = strided_layout(n, P.S);
    if (!a->workspace || a->workspace_bytes < P.W.total)
        return fail(SA_ERR_INVALID_ARG, "SA_MODE_STRIDED needs a workspace of sa_attn_workspace_bytes (%lld bytes)",
                    (long long)P.W.total);
    if (((uintptr_t)a->workspace & 255u) != 0) return fail(SA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    // residue views step S rows per key: their 32-bit DMA offsets
    const int64_t row_b = 2 * std::max(a->k_strides[2], a->v_strides[2]);
    if ((n + 256 * P.S) * row_b > kI32Max)
        return fail(SA_ERR_UNSUPPORTED, "n_kv times the K/V row stride must stay below 2^31 bytes");
    const StridedLayout::Lists* ls[2] = {&P.W.band, &P.W.res};
    for (int i = 0; i < 2; ++i) P.pat[i] = sa_pattern{};
    P.pat[0].causal = 1; P.pat[0].window_left = P.S - 1; P.pat[0].unit_window = -1;
    P.pat[1].causal = 1; P.pat[1].window_left = P.G; P.pat[1].unit_window = -1;
    for (int i = 0; i < 2; ++i) {
        const sa_status st = make_pattern(&P.pat[i], ls[i]->n_q, ls[i]->n_kv, P.dev[i]);
        if (st != SA_OK) return st;
    }
    return SA_OK;
}

sa_status strided_plan(const sa_attn_args* a, hipStream_t s)
{
    StridedParts P;
    const sa_status st0 = strided_check(a, P);
    if (st0 != SA_OK) return st0;
    uint8_t* ws = (uint8_t*)a->workspace;
    const StridedLayout::Lists* ls[2] = {&P.W.band, &P.W.res};
    for (int i = 0; i < 2; ++i) {
        const sa_status st = launched(sa::launch_block_mask(P.dev[i], (int32_t)ls[i]->n_q, (int32_t)ls[i]->n_kv,
                                                            kStridedBlock, kStridedBlock, (int32_t*)(ws + ls[i]->count),
                                                            (int32_t*)(ws + ls[i]->index), ws + ls[i]->partial,
                                                            (int64_t*)(ws + ls[i]->live), s),
                                      "sa_attn_strided_plan");
        if (st != SA_OK) return st;
    }
    return ok();
}

sa_status strided_fwd(const sa_attn_args* a, const sa::AttnParams& base, hipStream_t s)
{
    StridedParts P;
    const sa_status st0 = strided_check(a, P);
    if (st0 != SA_OK) return st0;
    if (a->o_dtype != SA_DTYPE_F32) return fail(SA_ERR_UNSUPPORTED, "SA_MODE_STRIDED writes a float32 O");
    if (!a->lse) return fail(SA_ERR_INVALID_ARG, "SA_MODE_STRIDED needs lse (the parts are merged through it)");
    const int64_t n = a->n_q, S = P.S, G = P.G, B = a->batch, H = a->heads;
    uint8_t* ws = (uint8_t*)a->workspace;
    auto with_lists = [&](sa::AttnParams& p, int part, const StridedLayout::Lists& l) {
        p.pat = P.dev[part];
        p.nqb = (int32_t)l.nqb;
        p.nkb = (int32_t)l.nkb;
        p.kv_count = (const int32_t*)(ws + l.count);
        p.kv_index = (const int32_t*)(ws + l.index);
        p.kv_partial = ws + l.partial;
    };
    // band: the natural layout
    {
        sa::AttnParams p = base;
        with_lists(p, 0, P.W.band);
        const sa_status st =
            launched(sa::launch_attn_blocks(p, (int)a->head_dim, kStridedBlock, kStridedBlock, 1, s), "sa_attn_fwd");
        if (st != SA_OK) return st;
    }
    for (int64_t b = 0; b < B; ++b) {
        // residue views: "batch" = head, "head" = residue, row i; merged in place
        sa::AttnParams p = base;
        with_lists(p, 1, P.W.res);
        p.q = base.q + b * a->q_strides[0] + (2 * S - 1) * a->q_strides[2];
        p.k = base.k + b * a->k_strides[0];
        p.v = base.v + b * a->v_strides[0];
        p.o = (float*)base.o + b * a->o_strides[0] + (2 * S - 1) * a->o_strides[2];
        p.q_sb = a->q_strides[1]; p.q_sh = a->q_strides[2]; p.q_sn = S * a->q_strides[2];
        p.k_sb = a->k_strides[1]; p.k_sh = a->k_strides[2]; p.k_sn = S * a->k_strides[2];
        p.v_sb = a->v_strides[1]; p.v_sh = a->v_strides[2]; p.v_sn = S * a->v_strides[2];
        p.o_sb = a->o_strides[1]; p.o_sh = a->o_strides[2]; p.o_sn = S * a->o_strides[2];
        p.lse = a->lse + b * H * n + (2 * S - 1);
        p.lse_sb = n; p.lse_sh = 1; p.lse_sn = S;
        p.batch = (int32_t)H;
        p.heads = (int32_t)S;
        p.n_q = (int32_t)(G - 1);       // residue 0: its last row is query row n - 1
        p.n_q_rest = (int32_t)(G - 2);  // residues 1 .. S-1: that row would lie past n - 1
        p.n_kv = (int32_t)G;
        p.merge = 1;
        const sa_status st =
            launched(sa::launch_attn_blocks(p, (int)a->head_dim, kStridedBlock, kStridedBlock, 1, s), "sa_attn_fwd");
        if (st != SA_OK) return st;
    }
    return ok();
}

}  // namespace

extern "C" {

int32_t sa_abi_version(void)
{
    return SA_ABI_VERSION;
}

sa_status sa_merge_partial(float* o, float* lse, const float* o2, const float* lse2, int64_t batch,
                           int64_t heads, int64_t n, int32_t head_dim, const int64_t o_strides[3],
                           const int64_t o2_strides[3], int32_t group, int64_t q_first, int64_t n2,
                           void* stream)
{
    try {
        if (batch < 0 || heads < 0 || n < 0) return fail(SA_ERR_INVALID_ARG, "negative batch, heads or n");
        if (head_dim != 64 && head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
        if (group < 1) return fail(SA_ERR_INVALID_ARG, "group must be >= 1");
        if (batch > kI32Max || heads > kI32Max || n > kI32Max || batch * heads > kI32Max || batch * heads * n > (int64_t(1) << 40))
            return fail(SA_ERR_UNSUPPORTED, "batch, heads and n must stay below 2^31 and their product below 2^40");
        if (q_first < 0 || n2 < 0) return fail(SA_ERR_INVALID_ARG, "q_first and n2 must be >= 0");
        if (n2 > n || group > n + 1) return fail(SA_ERR_INVALID_ARG, "n2 and group must not exceed n");
        if (n2 > 0 && q_first + (n2 - 1) * group >= n)
            return fail(SA_ERR_INVALID_ARG, "rows q_first + i*group (i < n2) must stay below n");
        const int64_t rows = batch * heads * n;
        if (rows == 0) return ok();
        if (!o || !lse || !o2 || !lse2 || !o_strides || !o2_strides) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
        if (!aligned16(o) || !aligned16(o2)) return fail(SA_ERR_INVALID_ARG, "o and o2 must be 16-byte aligned");
        for (int j = 0; j < 3; ++j)
            if (o_strides[j] % 4 || o2_strides[j] % 4)
                return fail(SA_ERR_INVALID_ARG, "o and o2 strides must be multiples of 4 elements");
        sa::MergeParams p{};
        p.o = o;
        p.lse = lse;
        p.o2 = o2;
        p.lse2 = lse2;
        p.rows = rows;
        p.n = n;
        p.n2 = n2;
        p.q_first = q_first;
        p.heads = heads;
        p.o_sb = o_strides[0];
        p.o_sh = o_strides[1];
        p.o_sn = o_strides[2];
        p.o2_sb = o2_strides[0];
        p.o2_sh = o2_strides[1];
        p.o2_sn = o2_strides[2];
        p.group = group;
        return launched(sa::launch_merge(p, head_dim, (hipStream_t)stream), "sa_merge_partial");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_merge_partial: unexpected exception");
    }
}

const char* sa_last_error(void)
{
    return g_err.c_str();
}

sa_status sa_build_block_mask(const sa_pattern* pattern, int64_t n_q, int64_t n_kv, int32_t block_q,
                              int32_t block_kv, int32_t* kv_count, int32_t* kv_index,
                              uint8_t* kv_partial, int64_t* live_pairs, void* stream)
{
    try {
        if (n_q < 0 || n_kv < 0) return fail(SA_ERR_INVALID_ARG, "n_q and n_kv must be >= 0");
        if (n_kv > kI32Max) return fail(SA_ERR_UNSUPPORTED, "n_kv must be below 2^31");
        if (block_q < 32 || block_q > 1024 || block_q % 32 || block_kv < 32 || block_kv > 1024 ||
            block_kv % 32)
            return fail(SA_ERR_INVALID_ARG, "block_q/block_kv must be multiples of 32 in [32, 1024]");
        if (!live_pairs) return fail(SA_ERR_INVALID_ARG, "live_pairs is NULL");
        const int64_t nqb = (n_q + block_q - 1) / block_q, nkb = (n_kv + block_kv - 1) / block_kv;
        if (nqb > 0 && (!kv_count || (nkb > 0 && (!kv_index || !kv_partial))))
            return fail(SA_ERR_INVALID_ARG, "kv_count/kv_index/kv_partial is NULL");
        if (nkb > 16384) return fail(SA_ERR_UNSUPPORTED, "more than 16384 key blocks per row");
        if (nqb > kI32Max) return fail(SA_ERR_UNSUPPORTED, "too many query blocks");
        sa::DevPattern d;
        sa_status st = make_pattern(pattern, n_q, n_kv, d);
        if (st != SA_OK) return st;
        hipStream_t s = (hipStream_t)stream;
        if (nqb == 0) return launched(sa::launch_zero_i64(live_pairs, s), "sa_build_block_mask");
        return launched(sa::launch_block_mask(d, (int32_t)n_q, (int32_t)n_kv, block_q, block_kv,
                                              kv_count, kv_index, kv_partial, live_pairs, s),
                        "sa_build_block_mask");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_build_block_mask: unexpected exception");
    }
}

// Block mode's long-row split of the pattern's global-token query blocks
// (shared lists only) and the bytes of its partial results: normalised O
// rows, then one LSE per row.
static int32_t long_row_split_of(const sa_attn_args* a, int64_t nqb, int64_t nkb, int32_t& chunks, int32_t& per_chunk)
{
    chunks = per_chunk = 0;
    if (a->per_head_lists != 0) return 0;
    return sa::long_row_split(a->pattern.causal, a->pattern.global_tokens, a->pattern.q_offset, a->n_q, nqb, nkb,
                              a->block_q, chunks, per_chunk);
}

static int64_t split_bytes(const sa_attn_args* a, int32_t gq, int32_t chunks)
{
    const int64_t slots = a->batch * a->heads * gq * chunks * a->block_q;
    return ((slots * a->head_dim * 4 + 255) & ~int64_t(255)) + ((slots * 4 + 255) & ~int64_t(255));
}

size_t sa_attn_workspace_bytes(const sa_attn_args* a)
{
    if (a && a->mode == SA_MODE_BLOCKS) {
        if (a->batch <= 0 || a->heads <= 0 || a->n_q <= 0 || a->n_kv <= 0 || a->per_head_lists != 0 ||
            (a->head_dim != 64 && a->head_dim != 128) || (a->block_q != 64 && a->block_q != 128) ||
            (a->block_kv != 64 && a->block_kv != 128) || a->n_q > kI32Max || a->n_kv > kI32Max)
            return 0;
        const int64_t nqb = (a->n_q + a->block_q - 1) / a->block_q, nkb = (a->n_kv + a->block_kv - 1) / a->block_kv;
        int32_t chunks = 0, per_chunk = 0;
        const int32_t gq = long_row_split_of(a, nqb, nkb, chunks, per_chunk);
        return gq > 0 ? (size_t)split_bytes(a, gq, chunks) : 0;
    }
    if (a && a->mode == SA_MODE_STRIDED) {
        const int64_t S = strided_template(a);
        return S > 0 && a->n_q <= kI32Max ? (size_t)strided_layout(a->n_q, S).total : 0;
    }
    if (!a || a->mode != SA_MODE_GATHER || a->batch <= 0 || a->heads <= 0 || a->n_q <= 0 || a->n_kv <= 0 ||
        (a->head_dim != 64 && a->head_dim != 128) || a->topk < 1 || a->topk > 8192 || a->gather_bh_stride < 0)
        return 0;
    sa::GatherSplitLayout L;
    if (!sa::gather_split_layout(a->batch, a->heads, a->n_q, a->n_kv, a->head_dim, a->topk, a->gather_bh_stride, L))
        return 0;
    return (size_t)L.total;
}

sa_status sa_attn_fwd(const sa_attn_args* a, void* stream)
{
    try {
        if (!a) return fail(SA_ERR_INVALID_ARG, "args is NULL");
        if (a->batch < 0 || a->heads < 0 || a->n_q < 0 || a->n_kv < 0)
            return fail(SA_ERR_INVALID_ARG, "batch/heads/n_q/n_kv must be >= 0");
        if (a->head_dim != 64 && a->head_dim != 128)
            return fail(SA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
        if (a->o_dtype != SA_DTYPE_BF16 && a->o_dtype != SA_DTYPE_F32)
            return fail(SA_ERR_INVALID_ARG, "o_dtype must be SA_DTYPE_BF16 or SA_DTYPE_F32");
        if (a->mode != SA_MODE_BLOCKS && a->mode != SA_MODE_GATHER && a->mode != SA_MODE_STRIDED)
            return fail(SA_ERR_INVALID_ARG, "mode must be SA_MODE_BLOCKS, SA_MODE_GATHER or SA_MODE_STRIDED");
        if (a->n_q > kI32Max || a->n_kv > kI32Max || a->batch * a->heads > kI32Max)
            return fail(SA_ERR_UNSUPPORTED, "sizes must stay below 2^31");
        if (a->batch == 0 || a->heads == 0 || a->n_q == 0) return ok();
        if (!a->q || !a->o || (a->n_kv > 0 && (!a->k || !a->v)))
            return fail(SA_ERR_INVALID_ARG, "q/k/v/o is NULL");
        if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
            return fail(SA_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned");
        if (a->lse && ((uintptr_t)a->lse & 3u)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
        for (int i = 0; i < 3; ++i) {
            if (a->q_strides[i] < 0 || a->k_strides[i] < 0 || a->v_strides[i] < 0 || a->o_strides[i] < 0)
                return fail(SA_ERR_INVALID_ARG, "strides must be >= 0");
            if (a->q_strides[i] % 8 || a->k_strides[i] % 8 || a->v_strides[i] % 8)
                return fail(SA_ERR_INVALID_ARG, "q/k/v strides must be multiples of 8 elements");
            if (a->o_strides[i] % (a->o_dtype == SA_DTYPE_F32 ? 4 : 8))
                return fail(SA_ERR_INVALID_ARG, "o strides must keep 16-byte alignment");
        }
        if (a->q_strides[2] < a->head_dim || a->o_strides[2] < a->head_dim ||
            (a->n_kv > 0 && (a->k_strides[2] < a->head_dim || a->v_strides[2] < a->head_dim)))
            return fail(SA_ERR_INVALID_ARG, "row strides must be >= head_dim");
        double scale = a->softmax_scale > 0 ? a->softmax_scale : 1.0 / std::sqrt((double)a->head_dim);

        sa::AttnParams p{};
        p.q = (const uint16_t*)a->q;
        p.k = (const uint16_t*)a->k;
        p.v = (const uint16_t*)a->v;
        p.o = a->o;
        p.lse = a->lse;
        p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_sn = a->q_strides[2];
        p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_sn = a->k_strides[2];
        p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_sn = a->v_strides[2];
        p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1]; p.o_sn = a->o_strides[2];
        p.lse_sb = a->heads * a->n_q;
        p.lse_sh = a->n_q;
        p.lse_sn = 1;
        p.merge = 0;
        p.last_first = 1;
        p.batch = (int32_t)a->batch;
        p.heads = (int32_t)a->heads;
        p.n_q = (int32_t)a->n_q;
        p.n_kv = (int32_t)a->n_kv;
        p.scale = (float)scale;
        p.scale_log2 = (float)(scale * 1.4426950408889634);
        hipStream_t s = (hipStream_t)stream;
        const int o_f32 = a->o_dtype == SA_DTYPE_F32;

        if (a->mode == SA_MODE_STRIDED) return strided_fwd(a, p, s);
        if (a->mode == SA_MODE_BLOCKS) {
            if ((a->block_q != 64 && a->block_q != 128) || (a->block_kv != 64 && a->block_kv != 128))
                return fail(SA_ERR_UNSUPPORTED, "block_q and block_kv must be 64 or 128");
            if (!a->kv_count || (a->n_kv > 0 && (!a->kv_index || !a->kv_partial)))
                return fail(SA_ERR_INVALID_ARG, "block lists are NULL");
            sa_status st = make_pattern(&a->pattern, a->n_q, a->n_kv, p.pat);
            if (st != SA_OK) return st;
            p.nqb = (int32_t)((a->n_q + a->block_q - 1) / a->block_q);
            p.nkb = (int32_t)((a->n_kv + a->block_kv - 1) / a->block_kv);
            if ((int64_t)p.nqb * a->batch * a->heads > kI32Max)
                return fail(SA_ERR_UNSUPPORTED, "too many work items");
            p.kv_count = a->kv_count;
            p.kv_index = a->kv_index;
            p.kv_partial = a->kv_partial;
            if (a->per_head_lists != 0 && a->per_head_lists != 1)
                return fail(SA_ERR_INVALID_ARG, "per_head_lists must be 0 or 1");
            p.per_head_lists = (int32_t)a->per_head_lists;
            p.last_first = a->pattern.causal != 0;
            // key tiles are fetched with 32-bit byte offsets from the (batch, head) base
            const int64_t row_b = 2 * std::max(a->k_strides[2], a->v_strides[2]);
            if ((a->n_kv + 256) * row_b > kI32Max)
                return fail(SA_ERR_UNSUPPORTED, "n_kv times the K/V row stride must stay below 2^31 bytes");
            // long-row split (optional: with workspace == NULL the rows run whole)
            int32_t chunks = 0, per_chunk = 0;
            const int32_t gq = long_row_split_of(a, p.nqb, p.nkb, chunks, per_chunk);
            if (gq > 0 && a->workspace) {
                const int64_t need = split_bytes(a, gq, chunks);
                if (a->workspace_bytes < need)
                    return fail(SA_ERR_INVALID_ARG, "workspace smaller than sa_attn_workspace_bytes (%lld bytes)",
                                (long long)need);
                if (((uintptr_t)a->workspace & 255u) != 0)
                    return fail(SA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
                if (a->batch * a->heads * (p.nqb - gq + (int64_t)gq * chunks) > kI32Max)
                    return fail(SA_ERR_UNSUPPORTED, "too many work items");
                const int64_t slots = a->batch * a->heads * gq * chunks * a->block_q;
                p.split_q = gq;
                p.split_c = chunks;
                p.split_e = per_chunk;
                p.part_o = (float*)a->workspace;
                p.part_lse = (float*)((uint8_t*)a->workspace + ((slots * a->head_dim * 4 + 255) & ~int64_t(255)));
            }
            st = launched(sa::launch_attn_blocks(p, (int)a->head_dim, (int)a->block_q, (int)a->block_kv, o_f32, s),
                          "sa_attn_fwd");
            if (st != SA_OK || p.split_q == 0) return st;
            return launched(sa::launch_split_merge(p, (int)a->head_dim, (int)a->block_q, o_f32, s), "sa_attn_fwd");
        }
        if (!a->gather_idx) return fail(SA_ERR_INVALID_ARG, "gather_idx is NULL");
        {
            // gathered rows are addressed with 32-bit byte offsets from the (batch, head) base
            const int64_t row_b = 2 * std::max(a->k_strides[2], a->v_strides[2]);
            if ((a->n_kv + 256) * row_b > kI32Max)
                return fail(SA_ERR_UNSUPPORTED, "n_kv times the K/V row stride must stay below 2^31 bytes");
        }
        if (a->topk < 1 || a->topk > 8192) return fail(SA_ERR_UNSUPPORTED, "topk must be in [1, 8192]");
        if (a->gather_bh_stride < 0) return fail(SA_ERR_INVALID_ARG, "gather_bh_stride must be >= 0");
        p.gidx = a->gather_idx;
        p.topk = (int32_t)a->topk;
        p.g_bh_stride = a->gather_bh_stride;
        sa::GatherSplitLayout L;
        if (a->workspace &&
            sa::gather_split_layout(a->batch, a->heads, a->n_q, a->n_kv, a->head_dim, a->topk, a->gather_bh_stride, L)) {
            if (a->workspace_bytes < L.total)
                return fail(SA_ERR_INVALID_ARG, "workspace smaller than sa_attn_workspace_bytes (%lld bytes)",
                            (long long)L.total);
            if (((uintptr_t)a->workspace & 255u) != 0)
                return fail(SA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
            uint8_t* ws = (uint8_t*)a->workspace;
            p.g_shift = L.shift;
            p.g_nchunk = L.nchunk;
            p.g_lists = (int32_t*)(ws + L.lists);
            p.g_offs = (int32_t*)(ws + L.offs);
            p.g_po = (float*)(ws + L.po);
            p.g_pml = (float*)(ws + L.pml);
            return launched(sa::launch_attn_gather_split(p, (int)a->head_dim, o_f32, s), "sa_attn_fwd");
        }
        return launched(sa::launch_attn_gather(p, (int)a->head_dim, o_f32, s), "sa_attn_fwd");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_attn_fwd: unexpected exception");
    }
}

static sa_status check_indexer(const void* q_idx, const void* k_idx, int64_t n_q, int64_t n_kv,
                               int32_t d_idx, int64_t q_offset, const float* scores)
{
    if (n_q < 0 || n_kv < 0 || q_offset < 0) return fail(SA_ERR_INVALID_ARG, "negative size or offset");
    if (n_kv > kI32Max || q_offset + n_q > kI32Max) return fail(SA_ERR_UNSUPPORTED, "sizes must stay below 2^31");
    if (d_idx < 8 || d_idx > 256 || d_idx % 8) return fail(SA_ERR_UNSUPPORTED, "d_idx must be a multiple of 8 in [8, 256]");
    if (n_q > 0 && n_kv > 0 && (!q_idx || !k_idx)) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(scores))
        return fail(SA_ERR_INVALID_ARG, "q_idx/k_idx/scores must be 16-byte aligned");
    return SA_OK;
}

static sa_status check_topk(const float* scores, int64_t n_q, int64_t n_kv, int64_t q_offset, int32_t topk,
                            const int32_t* idx_out)
{
    if (n_q < 0 || n_kv < 0 || q_offset < 0) return fail(SA_ERR_INVALID_ARG, "negative size or offset");
    if (q_offset + n_q > kI32Max) return fail(SA_ERR_UNSUPPORTED, "positions must stay below 2^31");
    if (topk < 1 || topk > 4096) return fail(SA_ERR_UNSUPPORTED, "topk must be in [1, 4096]");
    if (n_kv > 65536) return fail(SA_ERR_UNSUPPORTED, "n_kv must be <= 65536");
    if (n_q > 0 && (!scores || !idx_out)) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(scores)) return fail(SA_ERR_INVALID_ARG, "scores must be 16-byte aligned");
    return SA_OK;
}

sa_status sa_indexer_scores(const void* q_idx, const void* k_idx, int64_t n_q, int64_t n_kv, int32_t d_idx,
                            int64_t q_offset, float* scores, void* stream)
{
    try {
        sa_status st = check_indexer(q_idx, k_idx, n_q, n_kv, d_idx, q_offset, scores);
        if (st != SA_OK) return st;
        if (n_q > 0 && n_kv > 0 && !scores) return fail(SA_ERR_INVALID_ARG, "scores is NULL");
        if (n_q == 0 || n_kv == 0) return ok();
        return launched(sa::launch_indexer_scores((const uint16_t*)q_idx, (const uint16_t*)k_idx, (int32_t)n_q,
                                                  (int32_t)n_kv, d_idx, (int32_t)q_offset, scores,
                                                  (hipStream_t)stream),
                        "sa_indexer_scores");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_indexer_scores: unexpected exception");
    }
}

sa_status sa_topk(const float* scores, int64_t n_q, int64_t n_kv, int64_t q_offset, int32_t topk,
                  int32_t* idx_out, void* stream)
{
    try {
        sa_status st = check_topk(scores, n_q, n_kv, q_offset, topk, idx_out);
        if (st != SA_OK) return st;
        if (n_q == 0) return ok();
        return launched(sa::launch_topk(scores, (int32_t)n_q, (int32_t)n_kv, (int32_t)q_offset, topk, idx_out,
                                        (hipStream_t)stream),
                        "sa_topk");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_topk: unexpected exception");
    }
}

size_t sa_indexer_topk_workspace(int64_t n_q, int64_t n_kv, int32_t topk)
{
    sa::StreamTopkLayout L;
    if (topk < 1 || topk > 4096 || !sa::stream_topk_layout(n_q, n_kv, L)) return 0;
    return (size_t)L.total;
}

sa_status sa_indexer_topk(const void* q_idx, const void* k_idx, int64_t n_q, int64_t n_kv, int32_t d_idx,
                          int64_t q_offset, int32_t topk, float* scores_out, int32_t* idx_out, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    try {
        if (scores_out) {
            // two steps through the caller's score matrix
            sa_status st = check_indexer(q_idx, k_idx, n_q, n_kv, d_idx, q_offset, scores_out);
            if (st != SA_OK) return st;
            st = check_topk(scores_out, n_q, n_kv, q_offset, topk, idx_out);
            if (st != SA_OK) return st;
            if (n_q == 0) return ok();
            if (n_kv > 0) {
                st = launched(sa::launch_indexer_scores((const uint16_t*)q_idx, (const uint16_t*)k_idx, (int32_t)n_q,
                                                        (int32_t)n_kv, d_idx, (int32_t)q_offset, scores_out,
                                                        (hipStream_t)stream),
                              "sa_indexer_topk");
                if (st != SA_OK) return st;
            }
            return launched(sa::launch_topk(scores_out, (int32_t)n_q, (int32_t)n_kv, (int32_t)q_offset, topk,
                                            idx_out, (hipStream_t)stream),
                            "sa_indexer_topk");
        }
        // streaming: no score matrix, scratch from the caller
        sa_status st = check_indexer(q_idx, k_idx, n_q, n_kv, d_idx, q_offset, nullptr);
        if (st != SA_OK) return st;
        if (topk < 1 || topk > 4096) return fail(SA_ERR_UNSUPPORTED, "topk must be in [1, 4096]");
        if (n_kv > sa::kStreamMaxKv) return fail(SA_ERR_UNSUPPORTED, "n_kv must be <= 65536");
        if (n_q > 0 && !idx_out) return fail(SA_ERR_INVALID_ARG, "idx_out is NULL");
        if (n_q == 0) return ok();
        if (n_kv == 0) return launched(sa::launch_topk(nullptr, (int32_t)n_q, 0, (int32_t)q_offset, topk, idx_out,
                                                       (hipStream_t)stream),
                                       "sa_indexer_topk");
        sa::StreamTopkLayout L;
        sa::stream_topk_layout(n_q, n_kv, L);
        if (!workspace) return fail(SA_ERR_INVALID_ARG, "workspace is NULL (sa_indexer_topk_workspace: %lld bytes)",
                                    (long long)L.total);
        if (workspace_bytes < (size_t)L.total)
            return fail(SA_ERR_INVALID_ARG, "workspace smaller than sa_indexer_topk_workspace (%lld bytes)",
                        (long long)L.total);
        if (((uintptr_t)workspace & 255u) != 0) return fail(SA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        return launched(sa::launch_indexer_topk_stream((const uint16_t*)q_idx, (const uint16_t*)k_idx, (int32_t)n_q,
                                                       (int32_t)n_kv, d_idx, (int32_t)q_offset, topk, idx_out,
                                                       (uint8_t*)workspace, L, (hipStream_t)stream),
                        "sa_indexer_topk");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_indexer_topk: unexpected exception");
    }
}

static sa_status check_select(const sa_select_args* a, sa::SelectParams& p)
{
    if (!a) return fail(SA_ERR_INVALID_ARG, "args is NULL");
    if (a->batch < 0 || a->heads < 0 || a->n_q < 0 || a->n_kv < 0 || a->q_offset < 0 || a->n_select < 0)
        return fail(SA_ERR_INVALID_ARG, "negative size, offset or n_select");
    if (a->head_dim != 64 && a->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if ((a->block_q != 64 && a->block_q != 128) || (a->block_kv != 64 && a->block_kv != 128))
        return fail(SA_ERR_UNSUPPORTED, "block_q and block_kv must be 64 or 128");
    if (a->n_q > kI32Max || a->n_kv > kI32Max || a->q_offset + a->n_q > kI32Max || a->batch * a->heads > 65535)
        return fail(SA_ERR_UNSUPPORTED, "sizes must stay below 2^31 and batch*heads below 65536");
    const int64_t nqb = (a->n_q + a->block_q - 1) / a->block_q, nkb = (a->n_kv + a->block_kv - 1) / a->block_kv;
    if (nkb > sa::kSelectMaxBlocks) return fail(SA_ERR_UNSUPPORTED, "more than %d key blocks", sa::kSelectMaxBlocks);
    if (nqb > 65535) return fail(SA_ERR_UNSUPPORTED, "more than 65535 query blocks");
    for (int i = 0; i < 3; ++i)
        if (a->q_strides[i] < 0 || a->k_strides[i] < 0) return fail(SA_ERR_INVALID_ARG, "strides must be >= 0");
    p = sa::SelectParams{};
    p.q = (const uint16_t*)a->q;
    p.k = (const uint16_t*)a->k;
    p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_sn = a->q_strides[2];
    p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_sn = a->k_strides[2];
    p.batch = (int32_t)a->batch;
    p.heads = (int32_t)a->heads;
    p.n_q = (int32_t)a->n_q;
    p.n_kv = (int32_t)a->n_kv;
    p.d = (int32_t)a->head_dim;
    p.q_offset = (int32_t)a->q_offset;
    p.bq = (int32_t)a->block_q;
    p.bk = (int32_t)a->block_kv;
    p.nqb = (int32_t)nqb;
    p.nkb = (int32_t)nkb;
    p.n_sel = (int32_t)std::min<int64_t>(a->n_select, nkb);
    p.kv_count = a->kv_count;
    p.kv_index = a->kv_index;
    p.kv_partial = a->kv_partial;
    p.live_pairs = a->live_pairs;
    return SA_OK;
}

size_t sa_select_blocks_workspace(const sa_select_args* a)
{
    sa::SelectParams p;
    const std::string keep = g_err;  // a size query leaves the last error alone
    const sa_status st = check_select(a, p);
    g_err = keep;
    if (st != SA_OK || a->batch * a->heads == 0 || p.nqb == 0 || p.nkb == 0) return 0;
    return (size_t)sa::select_workspace_bytes(a->batch * a->heads, p.nqb, p.nkb, p.d);
}

sa_status sa_select_blocks(const sa_select_args* a, void* stream)
{
    try {
        sa::SelectParams p;
        sa_status st = check_select(a, p);
        if (st != SA_OK) return st;
        if (!a->live_pairs) return fail(SA_ERR_INVALID_ARG, "live_pairs is NULL");
        hipStream_t s = (hipStream_t)stream;
        if (a->batch * a->heads == 0 || p.nqb == 0 || p.nkb == 0)
            return launched(sa::launch_zero_i64(a->live_pairs, s), "sa_select_blocks");
        if (!a->q || !a->k || !a->kv_count || !a->kv_index || !a->kv_partial)
            return fail(SA_ERR_INVALID_ARG, "NULL pointer");
        const int64_t need = sa::select_workspace_bytes(a->batch * a->heads, p.nqb, p.nkb, p.d);
        if (!a->workspace || a->workspace_bytes < need)
            return fail(SA_ERR_INVALID_ARG, "workspace smaller than sa_select_blocks_workspace (%lld bytes)",
                        (long long)need);
        if (((uintptr_t)a->workspace & 255u) != 0) return fail(SA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
        p.qm = (double*)a->workspace;
        p.km = (double*)((uint8_t*)a->workspace + up(a->batch * a->heads * p.nqb * p.d * 8));
        return launched(sa::launch_select_blocks(p, s), "sa_select_blocks");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_select_blocks: unexpected exception");
    }
}

static sa_status check_bwd(const sa_attn_bwd_args* a, sa::BwdParams& p, sa::BwdLayout& L)
{
    if (!a) return fail(SA_ERR_INVALID_ARG, "args is NULL");
    if (a->batch < 0 || a->heads < 0 || a->n_q < 0 || a->n_kv < 0)
        return fail(SA_ERR_INVALID_ARG, "batch/heads/n_q/n_kv must be >= 0");
    if (a->head_dim != 64 && a->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if ((a->block_q != 64 && a->block_q != 128) || (a->block_kv != 64 && a->block_kv != 128))
        return fail(SA_ERR_UNSUPPORTED, "block_q and block_kv must be 64 or 128");
    if (a->per_head_lists != 0 && a->per_head_lists != 1) return fail(SA_ERR_INVALID_ARG, "per_head_lists must be 0 or 1");
    if (a->n_q > kI32Max || a->n_kv > kI32Max || a->batch * a->heads > kI32Max)
        return fail(SA_ERR_UNSUPPORTED, "sizes must stay below 2^31");
    p = sa::BwdParams{};
    const sa_status st = make_pattern(&a->pattern, a->n_q, a->n_kv, p.pat);
    if (st != SA_OK) return st;
    p.batch = (int32_t)a->batch;
    p.heads = (int32_t)a->heads;
    p.n_q = (int32_t)a->n_q;
    p.n_kv = (int32_t)a->n_kv;
    const double scale = a->softmax_scale > 0 ? a->softmax_scale : 1.0 / std::sqrt((double)a->head_dim);
    p.scale = (float)scale;
    p.scale_log2 = (float)(scale * 1.4426950408889634);
    p.nqb = (int32_t)((a->n_q + a->block_q - 1) / a->block_q);
    p.nkb = (int32_t)((a->n_kv + a->block_kv - 1) / a->block_kv);
    p.per_head_lists = (int32_t)a->per_head_lists;
    p.n_lists = a->per_head_lists ? (int32_t)(a->batch * a->heads) : 1;
    if ((int64_t)p.nqb * a->batch * a->heads > kI32Max || (int64_t)p.nkb * a->batch * a->heads > kI32Max)
        return fail(SA_ERR_UNSUPPORTED, "too many work items");
    L = sa::bwd_layout(a->batch * a->heads * a->n_q, p.n_lists, p.nqb, p.nkb);
    return SA_OK;
}

size_t sa_attn_bwd_workspace(const sa_attn_bwd_args* a)
{
    sa::BwdParams p;
    sa::BwdLayout L;
    const std::string keep = g_err;  // a size query leaves the last error alone
    const sa_status st = check_bwd(a, p, L);
    g_err = keep;
    return st == SA_OK ? (size_t)L.total : 0;
}

sa_status sa_attn_bwd(const sa_attn_bwd_args* a, void* stream)
{
    try {
        sa::BwdParams p;
        sa::BwdLayout L;
        sa_status st = check_bwd(a, p, L);
        if (st != SA_OK) return st;
        if (a->batch == 0 || a->heads == 0 || (a->n_q == 0 && a->n_kv == 0)) return ok();
        if (!a->q || !a->k || !a->v || !a->o || !a->lse || !a->dout || !a->dq || !a->dk || !a->dv || !a->kv_count ||
            (p.nkb > 0 && (!a->kv_index || !a->kv_partial)))
            return fail(SA_ERR_INVALID_ARG, "NULL pointer");
        if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->dout))
            return fail(SA_ERR_INVALID_ARG, "q/k/v/dout must be 16-byte aligned");
        if (!a->workspace || a->workspace_bytes < L.total)
            return fail(SA_ERR_INVALID_ARG, "workspace smaller than sa_attn_bwd_workspace (%lld bytes)",
                        (long long)L.total);
        if (((uintptr_t)a->workspace & 255u) != 0) return fail(SA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        p.q = (const uint16_t*)a->q;
        p.k = (const uint16_t*)a->k;
        p.v = (const uint16_t*)a->v;
        p.dout = (const uint16_t*)a->dout;
        p.o = a->o;
        p.lse = a->lse;
        p.dq = a->dq;
        p.dk = a->dk;
        p.dv = a->dv;
        p.kv_count = a->kv_count;
        p.kv_index = a->kv_index;
        p.kv_partial = a->kv_partial;
        uint8_t* ws = (uint8_t*)a->workspace;
        p.dsum = (float*)(ws + L.dsum);
        p.q_count = (int32_t*)(ws + L.q_count);
        p.q_index = (int32_t*)(ws + L.q_index);
        p.q_partial = ws + L.q_partial;
        p.order_q = (int32_t*)(ws + L.order_q);
        p.order_k = (int32_t*)(ws + L.order_k);
        return launched(sa::launch_attn_bwd(p, (int)a->head_dim, (int)a->block_q, (int)a->block_kv,
                                            (hipStream_t)stream),
                        "sa_attn_bwd");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_attn_bwd: unexpected exception");
    }
}

sa_status sa_attn_strided_plan(const sa_attn_args* a, void* stream)
{
    try {
        if (!a) return fail(SA_ERR_INVALID_ARG, "args is NULL");
        if (a->mode != SA_MODE_STRIDED) return fail(SA_ERR_INVALID_ARG, "mode must be SA_MODE_STRIDED");
        if (a->n_q < 0 || a->n_q > kI32Max) return fail(SA_ERR_UNSUPPORTED, "n_q must be in [0, 2^31)");
        return strided_plan(a, (hipStream_t)stream);
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_attn_strided_plan: unexpected exception");
    }
}

sa_status sa_indexer_topk_noalloc(const void* q_idx, const void* k_idx, int64_t n_q, int64_t n_kv, int32_t d_idx,
                                  int64_t q_offset, int32_t topk, int32_t* idx_out, void* stream)
{
    try {
        sa::StreamTopkLayout L;
        if (n_q > 0 && n_kv > 0 && n_kv <= sa::kStreamMaxKv && sa::stream_topk_layout(n_q, n_kv, L) &&
            L.total > sa::kNoAllocScratchBytes)
            return fail(SA_ERR_UNSUPPORTED,
                        "sa_indexer_topk_noalloc: these sizes need %lld bytes of scratch, above the fixed %lld",
                        (long long)L.total, (long long)sa::kNoAllocScratchBytes);
        uint8_t* ws = nullptr;
        if (n_q > 0 && n_kv > 0) {
            const hipError_t e = sa::noalloc_scratch(&ws);
            if (e != hipSuccess)
                return fail(SA_ERR_DEVICE, "sa_indexer_topk_noalloc: scratch address: %s", hipGetErrorString(e));
        }
        return sa_indexer_topk(q_idx, k_idx, n_q, n_kv, d_idx, q_offset, topk, nullptr, idx_out, ws,
                               (size_t)sa::kNoAllocScratchBytes, stream);
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_indexer_topk_noalloc: unexpected exception");
    }
}

}  // extern "C"
