// attn_bwd.hip -- gradients of the block-sparse attention (dQ, dK, dV).
//
// What is computed: for the masked attention of the blog "Sparse
// transformers: how to cut the O(n^2) of attention" (section on how it looks
// in code: scores q.k^T/sqrt(d), disallowed pairs at -inf, softmax, times V)
// and an upstream gradient dO, the chain rule gives, per allowed pair,
//   P = exp(s*scale - LSE),  dP = dO . v,  D = sum over the row of P*dP
//     = dO . O,  dS = P * (dP - D),
//   dV = sum_q P dO,  dQ = scale * sum_kv dS k,  dK = scale * sum_q dS q.
// ("Sparse Attention" glossary, section on common sparsity patterns: Native
// Sparse Attention is trained end to end.)  Only the live tiles of the block
// lists are visited, and the pattern is evaluated on partial tiles only, as
// in the forward kernel.
//
// gfx950 mapping: every product is a v_mfma_f32_32x32x16_bf16 on 32 x 32
// tiles with bf16 operands (P and dS rounded to bf16) and float32
// accumulation.  The contraction index of an MFMA may be permuted freely as
// long as both operands use the same order; the backward uses this so that
// P and dS feed the second product straight from the accumulator registers
// of the first: lane half h of an output tile holds rows 8m + 4h + c
// (m, c < 4), so the k-slots 8h .. 8h+7 of chunk ks carry rows
// 16ks + 4h + {0..3} and 16ks + 8 + 4h + {0..3}, and the other operand is
// read with the same order: at head_dim 128 by transposing 16-bit reads
// (ds_read_b64_tr_b16) of the one, swizzled row-major LDS copy, at head_dim
// 64 from a second, transposed copy (two 8-byte reads).
//   * bwd_dq_kernel: a wave owns 32 queries (Q and dO in registers) and walks
//     the live key tiles 32 keys at a time; the workgroup stages K and V in
//     LDS, double-buffered, the next tile's loads in
//     flight while the current one is computed, one barrier per step.  It
//     also forms D = rowsum(dO * O) for its queries.
//   * bwd_dkdv_kernel: two waves own each 32 keys (K, and V for dP, in
//     registers), one accumulating dV and one dK, and walk the query tiles
//     whose lists hold their key block (the lists transposed by
//     bwd_transpose_kernel), staging Q and dO the same way.
//   * Work items start longest list first (bwd_order_kernel), so that key
//     blocks every query sees (attention sinks, global tokens) do not finish
//     last.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
// u16 stride of a transposed [dim][32 rows] tile: 18 dwords, so the 8-byte
// reads of 32 lanes at 32 consecutive dims cover the 64 banks once, and the
// transposing u32 stores of a wave (16 row pairs x 4 chunks) do as well
constexpr int kTS = 36;

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// At head_dim 128 the staged tiles are kept once, row-major and unpadded,
// and the transposed operands are read from them with transposing 16-bit
// reads (ds_read_b64_tr_b16) instead of from a second, transposed copy:
// 16-byte chunk c of row r is stored at
// chunk c ^ tswz(r).  The swizzle is a bijection on a row's chunks and takes
// distinct values on any 16 consecutive rows (row reads: 16 lanes, one chunk,
// 16 rows); on four rows from a multiple of four it sends four consecutive
// chunks to sixteen distinct ones (transposing reads: 32 lanes, 4 rows x 4
// chunks), so both reads hit distinct banks.
template <int D>
__device__ __forceinline__ int tswz(int r)
{
    return D == 128 ? ((r & 15) ^ ((r & 3) << 2)) : (((r >> 1) & 7) ^ (((r >> 1) & 1) << 2));
}
// Byte offsets of a lane's reads.  Row reads (A operand, lane row l32,
// chunks 2c + hh): chunk (2c + hh) ^ tswz(l32) = (hh ^ tswz(l32)) ^ 2c, so
// the read of chunk pair c is at row_off ^ (c << 5).  Transposing reads (rows
// 16ks + rof and 16ks + rof + 8, 8 bytes at column 32db + cof): the swizzle of
// those rows does not depend on ks (rof < 8), and chunk 4db + cof/8 XOR the
// swizzle is (cof/8 ^ swizzle) ^ 4db, so the read is at
// 16ks rows + (tr_off[h] ^ (db << 6)).
template <int D>
struct LaneOffs {
    int row_off, tr_off0, tr_off1;
    __device__ __forceinline__ LaneOffs(int lane)
    {
        const int l32 = lane & 31, hh = lane >> 5;
        const int rof = 4 * (lane >> 5) + ((lane & 15) >> 2), cof = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        row_off = l32 * 2 * D + ((hh ^ tswz<D>(l32)) << 4);
        tr_off0 = rof * 2 * D + (((cof >> 3) ^ tswz<D>(rof)) << 4) + 2 * (cof & 7);
        tr_off1 = (rof + 8) * 2 * D + (((cof >> 3) ^ tswz<D>(rof + 8)) << 4) + 2 * (cof & 7);
    }
    // keep the XORed addresses from being hoisted out of the step loop (they
    // would take a register each)
    __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(row_off), "+v"(tr_off0), "+v"(tr_off1)); }
};
__device__ __forceinline__ bf16x8 row_op(const uint16_t* t, int off)
{
    return lds8(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(t) + off));
}
// B operand with the permuted contraction order (rows 16ks + 4hh .. + 3 and
// 16ks + 8 + 4hh .. + 3 of column 32db + l32) by transposing 16-bit reads of
// the row-major tile
template <int D>
__device__ __forceinline__ bf16x8 trr_op(const uint16_t* t, int ks, int db, const LaneOffs<D>& o)
{
    const char* b = reinterpret_cast<const char*>(t + 16 * ks * D);
    const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b + (o.tr_off0 ^ (db << 6))));
    const bf16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b + (o.tr_off1 ^ (db << 6))));
    return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// B operand with the permuted contraction order: rows r0 .. r0+3 and
// r0+8 .. r0+11 of column `dim` of a transposed tile
__device__ __forceinline__ bf16x8 tr_op(const uint16_t* tr, int dim, int r0)
{
    const u32x2 lo = *reinterpret_cast<const u32x2*>(tr + dim * kTS + r0);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(tr + dim * kTS + r0 + 8);
    const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
    return __builtin_bit_cast(bf16x8, w);
}

// A operand from accumulator elements base .. base+7 (bf16, nearest even)
__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base)
{
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)v[base + j];
    return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// 32 rows [row0, row0 + 32) of a [n, D] bf16 tensor, staged through
// registers: load() issues the global reads (rows at or past n read as zero),
// store() writes the row-major copy ([32][D + 8], 16-byte rows padded so that
// 16 lanes reading one chunk of 16 rows hit distinct banks) and, when T, the
// transposed copy ([D][kTS]).  A thread moves row pairs (2p, 2p + 1) of one
// 8-column chunk so that the transposed stores are whole dwords.
template <int D, int NT, bool T>
struct Stage32 {
    static constexpr int CH = D / 8, ITEMS = 16 * CH, PER = (ITEMS + NT - 1) / NT, RS = D + 8;
    u32x4 r0[PER], r1[PER];

    __device__ __forceinline__ void clear()
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) r0[i] = r1[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int row0, int n, int tid)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int it = tid + i * NT;
            const int p = it & 15, ch = it >> 4;
            const int64_t r = (int64_t)row0 + 2 * p;
            r0[i] = r1[i] = u32x4{0u, 0u, 0u, 0u};
            if (it < ITEMS) {
                if (r < n) r0[i] = *reinterpret_cast<const u32x4*>(src + r * D + 8 * ch);
                if (r + 1 < n) r1[i] = *reinterpret_cast<const u32x4*>(src + (r + 1) * D + 8 * ch);
            }
        }
    }
    // the unpadded, swizzled row-major copy only
    __device__ __forceinline__ void store_swz(uint16_t* t, int tid) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int it = tid + i * NT;
            if (it >= ITEMS) continue;
            const int p = it & 15, ch = it >> 4;
            *reinterpret_cast<u32x4*>(t + (2 * p) * D + ((ch ^ tswz<D>(2 * p)) << 3)) = r0[i];
            *reinterpret_cast<u32x4*>(t + (2 * p + 1) * D + ((ch ^ tswz<D>(2 * p + 1)) << 3)) = r1[i];
        }
    }
    __device__ __forceinline__ void store(uint16_t* rm, uint16_t* tr, int tid) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int it = tid + i * NT;
            if (it >= ITEMS) continue;
            const int p = it & 15, ch = it >> 4;
            *reinterpret_cast<u32x4*>(rm + (2 * p) * RS + 8 * ch) = r0[i];
            *reinterpret_cast<u32x4*>(rm + (2 * p + 1) * RS + 8 * ch) = r1[i];
            if (T) {
                uint32_t* t32 = reinterpret_cast<uint32_t*>(tr);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int dim = 8 * ch + 2 * x;
                    t32[dim * (kTS / 2) + p] = (r0[i][x] & 0xFFFFu) | (r1[i][x] << 16);
                    t32[(dim + 1) * (kTS / 2) + p] = (r0[i][x] >> 16) | (r1[i][x] & 0xFFFF0000u);
                }
            }
        }
    }
};

// For every list row L and key block j: the query blocks whose list holds j,
// ascending, with the list's partial flag.  One wave per (L, j); lane i
// binary-searches row i's ascending list, a ballot keeps the order.
__global__ void __launch_bounds__(256) bwd_transpose_kernel(const int32_t* __restrict__ kv_count,
                                                            const int32_t* __restrict__ kv_index,
                                                            const uint8_t* __restrict__ kv_partial, int32_t n_lists,
                                                            int32_t nqb, int32_t nkb, int32_t* __restrict__ q_count,
                                                            int32_t* __restrict__ q_index,
                                                            uint8_t* __restrict__ q_partial)
{
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wv >= (int64_t)n_lists * nkb) return;
    const int64_t L = wv / nkb;
    const int j = (int)(wv % nkb);
    int n = 0;
    for (int i0 = 0; i0 < nqb; i0 += 64) {
        const int i = i0 + lane;
        bool found = false;
        uint8_t part = 0;
        if (i < nqb) {
            const int64_t row = L * nqb + i;
            const int cnt = max(0, min(kv_count[row], nkb));
            const int32_t* ix = kv_index + row * nkb;
            int lo = 0, hi = cnt;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (ix[mid] < j) lo = mid + 1;
                else hi = mid;
            }
            if (lo < cnt && ix[lo] == j) {
                found = true;
                part = kv_partial[row * nkb + lo];
            }
        }
        const uint64_t m = __ballot(found);
        if (found) {
            const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
            q_index[wv * nqb + pos] = i;
            q_partial[wv * nqb + pos] = part;
        }
        n += __popcll(m);
    }
    if (lane == 0) q_count[wv] = n;
}

__device__ __forceinline__ int order_bucket(int32_t c, int32_t maxc)
{
    c = max(0, min(c, maxc));
    return (int)(((int64_t)c * 1023) / max(maxc, 1));
}

// order[rank] = item, items by list length descending (equal lengths in any
// order): a schedule only, every item writes its own outputs.  Block 0 orders
// the query-block lists, block 1 the transposed key-block lists.
__global__ void __launch_bounds__(1024) bwd_order_kernel(const int32_t* __restrict__ cq, int32_t nq_items,
                                                         int32_t maxq, int32_t* __restrict__ oq,
                                                         const int32_t* __restrict__ ck, int32_t nk_items,
                                                         int32_t maxk, int32_t* __restrict__ ok)
{
    const int32_t* cnt = blockIdx.x ? ck : cq;
    const int32_t T = blockIdx.x ? nk_items : nq_items;
    const int32_t maxc = blockIdx.x ? maxk : maxq;
    int32_t* order = blockIdx.x ? ok : oq;
    __shared__ int32_t slot[1024];
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x;
    slot[tid] = 0;
    __syncthreads();
    for (int32_t t = tid; t < T; t += 1024) atomicAdd(&slot[1023 - order_bucket(cnt[t], maxc)], 1);
    __syncthreads();
    const int v = slot[tid];
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if ((tid & 63) >= off) x += y;
    }
    if ((tid & 63) == 63) wsum[tid >> 6] = x;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < (tid >> 6); ++i) before += wsum[i];
    slot[tid] = before + x - v;
    __syncthreads();
    for (int32_t t = tid; t < T; t += 1024) {
        const int pos = atomicAdd(&slot[1023 - order_bucket(cnt[t], maxc)], 1);
        order[pos] = t;
    }
}

template <int D, int BQ, int BK>
__global__ void __launch_bounds__(BQ * 2, 2)
bwd_dq_kernel(BwdParams a)
{
    constexpr int NT = BQ * 2, NDC = D / 16, NDB = D / 32, RS = D + 8, SUB = BK / 32;
    // head_dim 128: K once, swizzled, Kᵀ operands by transposing reads; head_dim
    // 64: padded row-major and transposed copies (the swizzled form measured
    // slower there on the BigBird-style workload)
    constexpr bool SW = D == 128;
    using KStage = Stage32<D, NT, !SW>;
    using VStage = Stage32<D, NT, false>;
    __shared__ __attribute__((aligned(16))) uint16_t k_rm[2][32 * (SW ? D : RS)];
    __shared__ __attribute__((aligned(16))) uint16_t k_tr[2][SW ? 8 : D * kTS];
    __shared__ __attribute__((aligned(16))) uint16_t v_rm[2][32 * RS];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
    const int BH = a.batch * a.heads;
    int bh, qb;
    int64_t lrow;
    if (a.per_head_lists) {
        const int t = a.order_q[blockIdx.x];
        bh = t / a.nqb;
        qb = t % a.nqb;
        lrow = t;
    } else {
        bh = (int)(blockIdx.x % (unsigned)BH);
        qb = a.order_q[blockIdx.x / (unsigned)BH];
        lrow = qb;
    }
    const int q = qb * BQ + 32 * w + l32;  // this lane's query row
    LaneOffs<D> lo(lane);
    const bool q_ok = q < a.n_q;
    const int64_t qrow = (int64_t)bh * a.n_q + q;
    // B operands Q^T and dO^T: lane holds row q, dims 16s + 8hh .. + 7; and
    // the row's D = dO . O from the same dims plus the other half's
    bf16x8 qop[NDC], gop[NDC];
    float dpart = 0.f;
#pragma unroll
    for (int s = 0; s < NDC; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (q_ok) {
            x = *reinterpret_cast<const u32x4*>(a.q + qrow * D + 16 * s + 8 * hh);
            y = *reinterpret_cast<const u32x4*>(a.dout + qrow * D + 16 * s + 8 * hh);
            const f32x4 o0 = *reinterpret_cast<const f32x4*>(a.o + qrow * D + 16 * s + 8 * hh);
            const f32x4 o1 = *reinterpret_cast<const f32x4*>(a.o + qrow * D + 16 * s + 8 * hh + 4);
            dpart += bf16_lo(y.x) * o0.x + bf16_hi(y.x) * o0.y + bf16_lo(y.y) * o0.z + bf16_hi(y.y) * o0.w;
            dpart += bf16_lo(y.z) * o1.x + bf16_hi(y.z) * o1.y + bf16_lo(y.w) * o1.z + bf16_hi(y.w) * o1.w;
        }
        qop[s] = __builtin_bit_cast(bf16x8, x);
        gop[s] = __builtin_bit_cast(bf16x8, y);
    }
    const float dsum = dpart + __shfl_xor(dpart, 32);
    if (q_ok && hh == 0) a.dsum[qrow] = dsum;
    const float lse = q_ok ? a.lse[qrow] : INFINITY;
    const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;  // a row without keys has no pair
    RowCtx rc;
    row_ctx(a.pat, q + a.pat.q_offset, rc);
    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

    const int cnt = max(0, min(a.kv_count[lrow], a.nkb));
    const int nsteps = cnt * SUB;
    const int32_t* idx = a.kv_index + lrow * a.nkb;
    const uint8_t* prt = a.kv_partial + lrow * a.nkb;
    const uint16_t* kg = a.k + (int64_t)bh * a.n_kv * D;
    const uint16_t* vg = a.v + (int64_t)bh * a.n_kv * D;
    // A list of up to 64 entries sits in lane registers (lane e: entry e) and
    // is read with readlane, so a step issues no load before its own.
    const bool list_regs = cnt <= 64;
    int l_idx = 0, l_prt = 0;
    if (list_regs && lane < cnt) {
        l_idx = idx[lane];
        l_prt = prt[lane];
    }
    auto entry = [&](int e) { return list_regs ? __builtin_amdgcn_readlane(l_idx, e) : idx[e]; };
    auto partial = [&](int e) { return (list_regs ? __builtin_amdgcn_readlane(l_prt, e) : (int)prt[e]) != 0; };
    // first key of step s, or -1 when the step holds no key
    auto step_k0 = [&](int s) -> int {
        const int j = entry(s / SUB);
        if ((unsigned)j >= (unsigned)a.nkb) return -1;
        const int k0 = j * BK + 32 * (s % SUB);
        return k0 < a.n_kv ? k0 : -1;
    };
    // K and V rows of a step, loaded into registers two steps ahead of their
    // use and written to LDS one step ahead
    struct Fetched {
        KStage k;
        VStage v;
    };
    auto fetch = [&](Fetched& f, int s) {
        const int k0 = step_k0(s);
        if (k0 >= 0) {
            f.k.load(kg, k0, a.n_kv, tid);
            f.v.load(vg, k0, a.n_kv, tid);
        }
    };
    auto put = [&](const Fetched& f, int s, int b) {
        if (step_k0(s) >= 0) {
            if constexpr (SW) f.k.store_swz(k_rm[b], tid);
            else f.k.store(k_rm[b], k_tr[b], tid);
            f.v.store(v_rm[b], nullptr, tid);
        }
    };
    auto compute = [&](int s, int b) {
        const int k0 = step_k0(s);
        if (k0 >= 0) {
            if constexpr (SW) lo.opaque();
            // S^T = K Q^T and dP^T = V dO^T: lane = query, element i = key 8(i/4) + 4hh + i%4
            f32x16 st, dpt;
#pragma unroll
            for (int i = 0; i < 16; ++i) st[i] = dpt[i] = 0.f;
            const uint16_t* kr = k_rm[b] + l32 * RS + 8 * hh;
            const uint16_t* vr = v_rm[b] + l32 * RS + 8 * hh;
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16((SW ? row_op(k_rm[b], lo.row_off ^ (c << 5)) : lds8(kr + 16 * c)), qop[c], st, 0, 0, 0);
                dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(vr + 16 * c), gop[c], dpt, 0, 0, 0);
            }
            uint32_t mbits = 0xFFFFFFFFu;
            if (partial(s / SUB) || k0 + 32 > a.n_kv) mbits = allowed_bits32(a.pat, rc, k0) >> (4 * hh);
            f32x16 ds;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const bool ok = (mbits >> (8 * (i >> 2) + (i & 3))) & 1u;
                const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[i], a.scale_log2, -lse2)) : 0.f;
                ds[i] = p * (dpt[i] - dsum);
            }
            // dQ (queries x d) += dS (queries x keys) K (keys x d)
            const bf16x8 a0 = pack8(ds, 0), a1 = pack8(ds, 8);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 b0 = SW ? trr_op<D>(k_rm[b], 0, db, lo) : tr_op(k_tr[b], 32 * db + l32, 4 * hh);
                const bf16x8 b1 = SW ? trr_op<D>(k_rm[b], 1, db, lo) : tr_op(k_tr[b], 32 * db + l32, 16 + 4 * hh);
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, dq[db], 0, 0, 0);
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, dq[db], 0, 0, 0);
            }
        }
    };
    Fetched f0, f1;
    if (nsteps > 0) {
        fetch(f0, 0);
        put(f0, 0, 0);
    }
    if constexpr (KStage::PER == 1 && D == 128) {
        // Two register sets alternate, so the loop is unrolled by two and
        // names them statically: at step s, set s%2 (whose data went to LDS
        // last step) takes the loads of step s+2 and set (s+1)%2 goes to LDS
        // buffer (s+1)%2.
        if (nsteps > 1) fetch(f1, 1);
        __syncthreads();
        for (int s0 = 0; s0 < nsteps; s0 += 2) {
            if (s0 + 2 < nsteps) fetch(f0, s0 + 2);
            compute(s0, 0);
            if (s0 + 1 < nsteps) put(f1, s0 + 1, 1);
            __syncthreads();
            if (s0 + 1 < nsteps) {
                if (s0 + 3 < nsteps) fetch(f1, s0 + 3);
                compute(s0 + 1, 1);
                if (s0 + 2 < nsteps) put(f0, s0 + 2, 0);
                __syncthreads();
            }
        }
    } else {
        // with more rows a thread (64-query blocks), or at head_dim 64 where a
        // second set would cost a wave of occupancy: one set, one step ahead
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
            if (s + 1 < nsteps) fetch(f0, s + 1);
            compute(s, s & 1);
            if (s + 1 < nsteps) put(f0, s + 1, (s + 1) & 1);
            __syncthreads();
        }
    }
    // dq element (db, i): query row 8(i/4) + 4hh + i%4 of the wave, dim 32 db + l32
    float* dqg = a.dq + (int64_t)bh * a.n_q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int qr = qb * BQ + 32 * w + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (qr < a.n_q) dqg[(int64_t)qr * D + 32 * db + l32] = dq[db][i] * a.scale;
        }
}

template <int D, int BQ, int BK>
__global__ void __launch_bounds__(BK * 4, 1)
bwd_dkdv_kernel(BwdParams a)
{
    // Two waves per 32-key group: the first BK/32 waves accumulate dV, the
    // others dK.  A dV wave forms S and P of step s, leaves P in LDS and adds
    // P^T dO; the dK wave of its group runs one step behind, forming dP of
    // step s - 1, dS from the P left there, and adding dS^T Q.  Each wave
    // holds one 32 x D accumulator (64 registers a lane), so two waves fit
    // per SIMD and one wave's vector work runs beside the other's matrix
    // instructions.  The staged tiles of three steps are live at once (the
    // dK waves' step, the dV waves' step, the next step being written).
    constexpr int NT = BK * 4, NW = BK / 32, NDC = D / 16, NDB = D / 32, RS = D + 8, SUB = BQ / 32;
    // the dV waves stage the Q tile, the dK waves the dO tile
    // head_dim 128: each tile once, swizzled, transposed operands by
    // transposing reads (as in bwd_dq_kernel)
    constexpr bool SW = D == 128;
    using QStage = Stage32<D, NT / 2, !SW>;
    __shared__ __attribute__((aligned(16))) uint16_t q_rm[3][32 * (SW ? D : RS)];
    __shared__ __attribute__((aligned(16))) uint16_t q_tr[3][SW ? 8 : D * kTS];
    __shared__ __attribute__((aligned(16))) uint16_t g_rm[3][32 * (SW ? D : RS)];
    __shared__ __attribute__((aligned(16))) uint16_t g_tr[3][SW ? 8 : D * kTS];
    __shared__ __attribute__((aligned(16))) float lse_s[3][32];
    __shared__ __attribute__((aligned(16))) float dsum_s[3][32];
    __shared__ __attribute__((aligned(16))) uint32_t mw_s[3][NW][32];
    __shared__ __attribute__((aligned(16))) f32x4 p_s[2][NW][4][64];  // P of a step: [group][i/4][lane]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
    const int grp = w % NW;          // the wave's 32 keys
    const bool dk_wave = w >= NW;    // wave-uniform role
    const int BH = a.batch * a.heads;
    int bh, kb;
    int64_t lrow;
    if (a.per_head_lists) {
        const int t = a.order_k[blockIdx.x];
        bh = t / a.nkb;
        kb = t % a.nkb;
        lrow = t;
    } else {
        bh = (int)(blockIdx.x % (unsigned)BH);
        kb = a.order_k[blockIdx.x / (unsigned)BH];
        lrow = kb;
    }
    const int kbase = kb * BK + 32 * grp;  // this wave's keys
    LaneOffs<D> lo(lane);
    const int kv = kbase + l32;            // this lane's key row
    const bool k_ok = kv < a.n_kv;
    const int64_t krow = (int64_t)bh * a.n_kv + kv;
    // B operands K^T (and V^T in the dK waves): lane holds key row kv, dims 16s + 8hh .. + 7
    auto load_op = [&](const uint16_t* src, bf16x8* op) {
#pragma unroll
        for (int s = 0; s < NDC; ++s) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (k_ok) x = *reinterpret_cast<const u32x4*>(src + krow * D + 16 * s + 8 * hh);
            op[s] = __builtin_bit_cast(bf16x8, x);
        }
    };
    // zero accumulators made by a matrix instruction (0 * 0 + 0), so that they
    // are born in the registers the loop's matrix instructions accumulate in
    auto zero_acc = [&](f32x16* acc) {
        const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        f32x16 zacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) zacc[i] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, zacc, 0, 0, 0);
    };

    const int cnt = max(0, min(a.q_count[lrow], a.nqb));
    const int nsteps = cnt * SUB;
    const int32_t* idx = a.q_index + lrow * a.nqb;
    const uint8_t* prt = a.q_partial + lrow * a.nqb;
    // A list of up to 64 entries sits in lane registers (lane e: entry e) and
    // is read with readlane, so a step issues no load before its own.
    const bool list_regs = cnt <= 64;
    int l_idx = 0, l_prt = 0;
    if (list_regs && lane < cnt) {
        l_idx = idx[lane];
        l_prt = prt[lane];
    }
    auto entry = [&](int e) { return list_regs ? __builtin_amdgcn_readlane(l_idx, e) : idx[e]; };
    auto partial = [&](int e) { return (list_regs ? __builtin_amdgcn_readlane(l_prt, e) : (int)prt[e]) != 0; };
    const uint16_t* qg = a.q + (int64_t)bh * a.n_q * D;
    const uint16_t* gg = a.dout + (int64_t)bh * a.n_q * D;
    const float* lseg = a.lse + (int64_t)bh * a.n_q;
    const float* dsg = a.dsum + (int64_t)bh * a.n_q;
    // first query of step s; a step past the last query (the ragged end of the
    // last block) stages zero rows with LSE = +inf, so it adds nothing
    auto step_q0 = [&](int s) -> int { return entry(s / SUB) * BQ + 32 * (s % SUB); };
    // Staged data of one step (rows, LSE, D, mask words), loaded into
    // registers two steps ahead of its use and written to LDS one step ahead.
    // Nothing loaded is used before the step is written to LDS (a use would
    // wait for every load in flight).
    struct Fetched {
        QStage x;  // Q rows (dV waves) or dO rows (dK waves)
        float lse, dsum;
        uint32_t mword;
    };
    const int stid = tid % (NT / 2);
    auto fetch = [&](Fetched& f, int s) {
        const int q0 = step_q0(s);
        f.x.load(dk_wave ? gg : qg, q0, a.n_q, stid);
        f.lse = INFINITY;
        f.dsum = 0.f;
        if ((unsigned)(tid - NT / 2) < 32u) {
            // rows past n_q read the last row's values; put() gives them
            // LSE = +inf (P = 0), so their D never counts
            const int qr = min(q0 + (tid - NT / 2), a.n_q - 1);
            f.lse = lseg[qr];
            f.dsum = dsg[qr];
        }
        f.mword = 0u;
        // the mask words and the row values come from the dK waves, whose
        // step is the shorter one
        if (dk_wave && partial(s / SUB)) {
            // bit l of word r: key kbase + l is allowed for query q0 + r
            const int qr = q0 + l32;
            RowCtx rc;
            row_ctx(a.pat, qr + a.pat.q_offset, rc);
            f.mword = qr < a.n_q ? allowed_bits32(a.pat, rc, kbase) : 0u;
        }
    };
    auto put = [&](const Fetched& f, int s, int buf) {
        if constexpr (SW) f.x.store_swz(dk_wave ? g_rm[buf] : q_rm[buf], stid);
        else if (dk_wave) f.x.store(g_rm[buf], g_tr[buf], stid);
        else f.x.store(q_rm[buf], q_tr[buf], stid);
        if ((unsigned)(tid - NT / 2) < 32u) {
            // a row without keys (LSE = -inf) or past n_q has no pair
            const int r = tid - NT / 2;
            const bool row_ok = step_q0(s) + r < a.n_q;
            lse_s[buf][r] = (!row_ok || f.lse == -INFINITY) ? INFINITY : f.lse * kLog2e;
            dsum_s[buf][r] = f.dsum;
        }
        if (dk_wave && partial(s / SUB) && hh == 0) mw_s[buf][grp][l32] = f.mword;
    };
    // X Y^T for row-major X (32 rows in LDS) and Y in registers: S = Q K^T,
    // dP = dO V^T; lane = key, element i = query 8(i/4) + 4hh + i%4
    auto product = [&](const uint16_t* xrm, const bf16x8* yop, f32x16& acc) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
        const uint16_t* xr = xrm + l32 * RS + 8 * hh;
        if constexpr (SW) lo.opaque();
        auto x_op = [&](int c) { return SW ? row_op(xrm, lo.row_off ^ (c << 5)) : lds8(xr + 16 * c); };
        // LDS operands are requested two k-steps ahead (a ring of three)
        bf16x8 xa[3];
        xa[0] = x_op(0);
        xa[1] = x_op(1);
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            if (c + 2 < NDC) xa[(c + 2) % 3] = x_op(c + 2);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[c % 3], yop[c], acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // acc (keys x d) += X^T (keys x queries) Y with X from the softmax and Y
    // read transposed from LDS (ytr: the transposed copy, or at head_dim 128
    // the swizzled row-major tile); step it = ks * NDB + db reads rows
    // 16ks + 4hh.. of dim 32db + l32
    auto accumulate = [&](const uint16_t* ytr, const f32x16& x, f32x16* acc) {
        bf16x8 yb[3];
        auto ld_b = [&](int slot, int it) {
            const int ks = it / NDB, dim = 32 * (it % NDB) + l32;
            yb[slot] = SW ? trr_op<D>(ytr, ks, it % NDB, lo) : tr_op(ytr, dim, 16 * ks + 4 * hh);
        };
        ld_b(0, 0);
        ld_b(1, 1);
        const bf16x8 xa[2] = {pack8(x, 0), pack8(x, 8)};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < 2 * NDB; ++it) {
            if (it + 2 < 2 * NDB) ld_b((it + 2) % 3, it + 2);
            const int ks = it / NDB, db = it % NDB;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[ks], yb[it % 3], acc[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // P of one step (masked keys 0)
    auto softmax = [&](int s, int b, const f32x16& sv, f32x16& pv) {
        const bool masked = partial(s / SUB);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[b][8 * m + 4 * hh]);
            u32x4 w4 = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
            if (masked) w4 = *reinterpret_cast<const u32x4*>(&mw_s[b][grp][8 * m + 4 * hh]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int i = 4 * m + c;
                const bool ok = (w4[c] >> l32) & 1u;
                pv[i] = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], a.scale_log2, -l4[c])) : 0.f;
            }
        }
    };
    // Iteration j (0 .. nsteps) computes step j in the dV waves and step
    // j - 1 in the dK waves; step s is staged in LDS buffer s % 3.  Two
    // register sets alternate, so the loop is unrolled by two and names them
    // statically: at iteration j, set j%2 (whose data went to LDS last
    // iteration) takes the loads of step j+2 and set (j+1)%2 goes to LDS.
    auto run = [&](auto&& compute) {
        Fetched f0, f1;
        if (nsteps > 0) {
            fetch(f0, 0);
            put(f0, 0, 0);
        }
        if (nsteps > 1) fetch(f1, 1);
        __syncthreads();
        for (int j0 = 0; j0 <= nsteps; j0 += 2) {
            if (j0 + 2 < nsteps) fetch(f0, j0 + 2);
            compute(j0);
            if (j0 + 1 < nsteps) put(f1, j0 + 1, (j0 + 1) % 3);
            __syncthreads();
            if (j0 + 1 <= nsteps) {
                if (j0 + 3 < nsteps) fetch(f1, j0 + 3);
                compute(j0 + 1);
                if (j0 + 2 < nsteps) put(f0, j0 + 2, (j0 + 2) % 3);
                __syncthreads();
            }
        }
    };
    // element (db, i): key row 8(i/4) + 4hh + i%4 of the wave, dim 32 db + l32
    auto write = [&](float* dst, const f32x16* acc, float mul) {
        float* g = dst + (int64_t)bh * a.n_kv * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kr = kbase + 8 * (i >> 2) + 4 * hh + (i & 3);
                if (kr < a.n_kv) g[(int64_t)kr * D + 32 * db + l32] = acc[db][i] * mul;
            }
    };
    f32x4* pmine = &p_s[0][grp][0][lane];  // this lane's P of the group, buffer 0
    constexpr int PB = NW * 4 * 64;          // f32x4 per P buffer
    if (!dk_wave) {
        // S, P of step j; P to LDS; dV += P^T dO
        bf16x8 kop[NDC];
        load_op(a.k, kop);
        f32x16 dv[NDB];
        zero_acc(dv);
        run([&](int j) {
            if (j >= nsteps) return;
            const int b = j % 3;
            f32x16 sv, pv;
            product(q_rm[b], kop, sv);
            softmax(j, b, sv, pv);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                pmine[(j & 1) * PB + 64 * m] = f32x4{pv[4 * m], pv[4 * m + 1], pv[4 * m + 2], pv[4 * m + 3]};
            accumulate(SW ? g_rm[b] : g_tr[b], pv, dv);
        });
        write(a.dv, dv, 1.f);
    } else {
        // dP of step j - 1, dS = P (dP - D) with that step's P; dK += dS^T Q
        bf16x8 vop[NDC];
        load_op(a.v, vop);
        f32x16 dk[NDB];
        zero_acc(dk);
        run([&](int j) {
            if (j < 1) return;
            const int s = j - 1, b = s % 3;
            f32x16 dp, ds;
            product(g_rm[b], vop, dp);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 p4 = pmine[(s & 1) * PB + 64 * m];
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dsum_s[b][8 * m + 4 * hh]);
#pragma unroll
                for (int c = 0; c < 4; ++c) ds[4 * m + c] = p4[c] * (dp[4 * m + c] - d4[c]);
            }
            accumulate(SW ? q_rm[b] : q_tr[b], ds, dk);
        });
        write(a.dk, dk, a.scale);
    }
}

template <int D, int BQ, int BK>
hipError_t launch_bwd_t(const BwdParams& a, hipStream_t stream)
{
    const int64_t bh = (int64_t)a.batch * a.heads;
    if (bh * a.nqb > 0)
        hipLaunchKernelGGL((bwd_dq_kernel<D, BQ, BK>), dim3((unsigned)(bh * a.nqb)), dim3(BQ * 2), 0, stream, a);
    if (bh * a.nkb > 0)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, BQ, BK>), dim3((unsigned)(bh * a.nkb)), dim3(BK * 4), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& a, int bq, int bk, hipStream_t stream)
{
    if (bq == 128 && bk == 128) return launch_bwd_t<D, 128, 128>(a, stream);
    if (bq == 128 && bk == 64) return launch_bwd_t<D, 128, 64>(a, stream);
    if (bq == 64 && bk == 128) return launch_bwd_t<D, 64, 128>(a, stream);
    if (bq == 64 && bk == 64) return launch_bwd_t<D, 64, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& a, int head_dim, int block_q, int block_kv, hipStream_t stream)
{
    if (head_dim != 128 && head_dim != 64) return hipErrorInvalidValue;
    const int64_t nt = (int64_t)a.n_lists * a.nkb;
    if (nt > 0)
        hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)((nt + 3) / 4)), dim3(256), 0, stream, a.kv_count,
                           a.kv_index, a.kv_partial, a.n_lists, a.nqb, a.nkb, a.q_count, a.q_index, a.q_partial);
    hipLaunchKernelGGL(bwd_order_kernel, dim3(2), dim3(1024), 0, stream, a.kv_count, a.n_lists * a.nqb, a.nkb,
                       a.order_q, a.q_count, a.n_lists * a.nkb, a.nqb, a.order_k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (head_dim == 128) return launch_bwd_d<128>(a, block_q, block_kv, stream);
    return launch_bwd_d<64>(a, block_q, block_kv, stream);
}

}  // namespace sa
