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

size_t sa_attn_workspace_bytes(const sa_attn_args* a)
{
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
        if (a->mode != SA_MODE_BLOCKS && a->mode != SA_MODE_GATHER)
            return fail(SA_ERR_INVALID_ARG, "mode must be SA_MODE_BLOCKS or SA_MODE_GATHER");
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
        p.batch = (int32_t)a->batch;
        p.heads = (int32_t)a->heads;
        p.n_q = (int32_t)a->n_q;
        p.n_kv = (int32_t)a->n_kv;
        p.scale = (float)scale;
        p.scale_log2 = (float)(scale * 1.4426950408889634);
        hipStream_t s = (hipStream_t)stream;
        const int o_f32 = a->o_dtype == SA_DTYPE_F32;

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
            // key tiles are fetched with 32-bit byte offsets from the (batch, head) base
            const int64_t row_b = 2 * std::max(a->k_strides[2], a->v_strides[2]);
            if ((a->n_kv + 256) * row_b > kI32Max)
                return fail(SA_ERR_UNSUPPORTED, "n_kv times the K/V row stride must stay below 2^31 bytes");
            return launched(sa::launch_attn_blocks(p, (int)a->head_dim, (int)a->block_q,
                                                   (int)a->block_kv, o_f32, s),
                            "sa_attn_fwd");
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
    if (n_q > 0 && n_kv > 0 && (!q_idx || !k_idx || !scores)) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
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

sa_status sa_indexer_topk(const void* q_idx, const void* k_idx, int64_t n_q, int64_t n_kv, int32_t d_idx,
                          int64_t q_offset, int32_t topk, float* scores, int32_t* idx_out, void* stream)
{
    try {
        sa_status st = check_indexer(q_idx, k_idx, n_q, n_kv, d_idx, q_offset, scores);
        if (st != SA_OK) return st;
        st = check_topk(scores, n_q, n_kv, q_offset, topk, idx_out);
        if (st != SA_OK) return st;
        if (n_q == 0) return ok();
        if (n_kv > 0) {
            st = launched(sa::launch_indexer_scores((const uint16_t*)q_idx, (const uint16_t*)k_idx, (int32_t)n_q,
                                                    (int32_t)n_kv, d_idx, (int32_t)q_offset, scores,
                                                    (hipStream_t)stream),
                          "sa_indexer_topk");
            if (st != SA_OK) return st;
        }
        return launched(sa::launch_topk(scores, (int32_t)n_q, (int32_t)n_kv, (int32_t)q_offset, topk, idx_out,
                                        (hipStream_t)stream),
                        "sa_indexer_topk");
    } catch (...) {
        return fail(SA_ERR_DEVICE, "sa_indexer_topk: unexpected exception");
    }
}

}  // extern "C"
