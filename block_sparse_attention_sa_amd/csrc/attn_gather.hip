// attn_gather.hip -- attention of each query over its own key list.
//
// "Sparse Attention" glossary, section on common sparsity patterns: under
// DeepSeek Sparse Attention full attention is computed only over the tokens
// the indexer selected for that query, so the cost per query is constant.
// The softmax is the one of the blog's masked attention (section on how it
// looks in code) restricted to the listed keys.
//
// Each query has a different key set, so there is no K/V tile shared by
// several queries and no matrix product to put on MFMA: the work is two
// gathered matrix-vector products, about one flop per byte moved, bound by
// the latency of the row gathers and the vector work per key.  One wave works
// on one query's list (or, in the split form, on the part of it that falls in
// one key range) in blocks of 128 keys with an online softmax:
//   * the block's key indices are read once (two per lane) and turned into the
//     byte offsets of their K and V rows, kept in LDS (a key out of range reads
//     row 0 with its score forced to -inf);
//   * scores: D/32 lanes per K row, 64 contiguous bytes each, pair dot
//     products against the query's bfloat16 pairs, summed over the row's
//     lanes with DPP moves; four steps of row loads are issued before any is
//     used, so a block costs a few memory round trips, not one per key;
//   * values: D/8 lanes per V row, 16 bytes each; a lane group takes two keys
//     per step and adds both with one pair dot product per column pair;
//   * scores and then probabilities sit in 128 floats of LDS per wave; a
//     short last block runs only the load batches that hold keys.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWaves = 4;

// workgroup id -> work block, so that consecutive blocks (one head's key
// range) run on the same XCD when workgroups are dealt round-robin over the
// 8 XCDs; a bijection for any grid size
__device__ __forceinline__ int xcd_remap(int wg, int nwg)
{
    const int c = nwg / 8, r = nwg % 8;
    const int x = wg % 8, slot = wg / 8;
    const int base = x < r ? x * (c + 1) : r * (c + 1) + (x - r) * c;
    return base + slot;
}

constexpr int kBlk = 128;  // keys per block of the online softmax
constexpr int kVF = 4;     // value steps whose row loads are issued together
constexpr int kPartItems = 1;  // (head, range, query) items per wave in the split form

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Cross-lane steps on the vector unit (DPP) instead of LDS permutes:
// quad_perm [1,0,3,2] and [2,3,0,1] exchange with lane ^ 1 and lane ^ 2;
// row_ror 4 and 8 rotate within 16-lane rows, which for an operation that is
// associative and commutative, applied to values already equal within each
// quad, combines the four quads of the row in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_sum(float x)
{
    x += dpp<0xB1>(x);
    return x + dpp<0x4E>(x);
}
// sum over the 16-lane row, in every lane of it
__device__ __forceinline__ float row_sum(float x)
{
    x = quad_sum(x);
    x += dpp<0x124>(x);
    return x + dpp<0x128>(x);
}

// a.x * b.x + a.y * b.y + c on bfloat16 pairs (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// How the lanes of a wave read K rows for the scores: LQ lanes per row, each
// taking PC pieces of 16 bytes, and QF steps of row loads issued together.
//   packed: a lane's pieces are contiguous (lane s of a row reads bytes
//           [s*PB, (s+1)*PB) with PB = 2*D/LQ), so one load instruction
//           touches each row in LQ places;
//   spread: piece x of lane s is bytes [16*(s + LQ*x), +16), so the LQ lanes
//           of a row read 16*LQ contiguous bytes per instruction (a whole
//           128-byte line at D = 128, LQ = 8).
// The split form's waves share one key range in L2, and there the number of
// lines an instruction touches sets the rate (spread, 8 lanes per row at
// D = 128: 1,049 -> 816 us for 1024 queries x 16 heads x top-2048 over a
// 64K context); the single pass, whose rows mostly miss L2, is faster packed.
template <int D, int LQ_, bool SPREAD, int QF_>
struct ScoreShape {
    static constexpr int LQ = LQ_, QF = QF_;
    static constexpr int PB = 2 * D / LQ, PC = PB / 16;
    static_assert(PB % 16 == 0 && LQ >= 2 && 64 % LQ == 0, "score lane split");
    __device__ static constexpr uint32_t off(int s, int x) { return SPREAD ? 16u * (s + LQ * x) : PB * s + 16u * x; }
};
template <int D> using ScorePacked = ScoreShape<D, D / 32, false, 4>;
template <int D> using ScoreSpread = ScoreShape<D, D / 16, true, 8>;

// The query's bfloat16 pairs that match this lane's K pieces: q2[4x + j] pairs
// with word j of piece x.
template <int D, class SS>
__device__ __forceinline__ void load_q2(const uint16_t* qrow, int lane, uint32_t (&q2)[4 * SS::PC])
{
    const int qs = lane % SS::LQ;
#pragma unroll
    for (int x = 0; x < SS::PC; ++x) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(qrow) + SS::off(qs, x));
#pragma unroll
        for (int j = 0; j < 4; ++j) q2[4 * x + j] = w[j];
    }
}

// Online softmax of one query over the n keys keys[0..n): m (max, log2
// units, scale folded in), l (sum of exp2(s - m)) and acc (sum of
// exp2(s - m) v over this lane's 8 columns [8*(lane % (D/8)), +8)).  With
// `check`, entries outside [0, n_kv) are skipped.
//   scores: SS::LQ lanes per key row, each PC pieces of 16 bytes (see
//           ScoreShape), bf16 pair dot products, then a sum over the row's
//           lanes;
//   values: D/8 lanes per row, each 16 bytes; a lane group takes two keys
//           per step, their values are interleaved into (key0, key1) pairs
//           and one pair dot product with (p0, p1) adds both keys' terms.
template <int D, class SS>
__device__ __forceinline__ void gather_online(const int32_t* keys, int n, bool check, int n_kv,
                                              const uint16_t* kg, uint32_t krow_b, const uint16_t* vg, uint32_t vrow_b,
                                              const uint32_t (&q2)[4 * SS::PC], float c, float* sc, uint32_t* ro, int lane,
                                              float& m, float& l, float (&acc)[8])
{
    constexpr int LQ = SS::LQ, KQ = 64 / LQ, PC = SS::PC, kQF = SS::QF;  // scores: lanes per row, rows per step
    constexpr int QSTEPS = kBlk / KQ;
    constexpr int LPK = D / 8, GP = 64 / LPK;  // values: lanes per row, row groups
    constexpr int KPV = 2 * GP;                // keys per value step
    constexpr int VSTEPS = kBlk / KPV;
    static_assert(QSTEPS % kQF == 0 && VSTEPS % kVF == 0, "block split");
    const int qs = lane % LQ, qg = lane / LQ;
    const int sub = lane % LPK, vgr = lane / LPK;
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int b0 = 0; b0 < n; b0 += kBlk) {
        const int nb = min(kBlk, n - b0);
        // byte offsets of the block's K rows (bit 31 set: no key; the row
        // read is then row 0, whose score is dropped) and V rows (row 0 for
        // no key, whose probability is 0), two entries per lane, in LDS
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int e = b0 + 64 * r + lane;
            const int s = e < n ? keys[e] : -1;
            const bool ok = e < n && !(check && (s < 0 || s >= n_kv));
            ro[64 * r + lane] = ok ? (uint32_t)s * krow_b : 0x80000000u;
            ro[kBlk + 64 * r + lane] = ok ? (uint32_t)s * vrow_b : 0u;
        }
        wave_lds_sync();
        // ---- scores (a short last block runs only the batches that hold keys)
        const int qlim = (nb + KQ - 1) / KQ;
        float bmax = -INFINITY;
#pragma unroll 1
        for (int g = 0; g < qlim; g += kQF) {
            u32x4 w[kQF][PC];
            bool okk[kQF];
#pragma unroll
            for (int i = 0; i < kQF; ++i) {
                const uint32_t off = ro[(g + i) * KQ + qg];
                okk[i] = (int32_t)off >= 0;
                const char* row = reinterpret_cast<const char*>(kg) + (uint64_t)(off & 0x7FFFFFFFu);
#pragma unroll
                for (int x = 0; x < PC; ++x) w[i][x] = *reinterpret_cast<const u32x4*>(row + SS::off(qs, x));
            }
#pragma unroll
            for (int i = 0; i < kQF; ++i) {
                float d0 = 0.f, d1 = 0.f;
#pragma unroll
                for (int x = 0; x < PC; ++x) {
                    d0 = dot2(w[i][x][0], q2[4 * x + 0], d0);
                    d1 = dot2(w[i][x][1], q2[4 * x + 1], d1);
                    d0 = dot2(w[i][x][2], q2[4 * x + 2], d0);
                    d1 = dot2(w[i][x][3], q2[4 * x + 3], d1);
                }
                float d = d0 + d1;
                if (LQ == 4 || LQ == 8) {
                    d = quad_sum(d);
                    // 8 lanes per row: lanes 4..7 of the row's group add the
                    // quad below theirs (row_ror 4); lanes 0..3 then hold no
                    // row's score and stay out of the maximum
                    if (LQ == 8) d += dpp<0x124>(d);
                } else {
#pragma unroll
                    for (int off = 1; off < LQ; off <<= 1) d += __shfl_xor(d, off, 64);
                }
                const float sv = okk[i] ? d * c : -INFINITY;
                bmax = fmaxf(bmax, LQ == 8 && qs < 4 ? -INFINITY : sv);
                if (qs == (LQ == 8 ? 4 : 0)) sc[(g + i) * KQ + qg] = sv;
            }
        }
        if (LQ == 4 || LQ == 8) {
            // equal within quads already (or -inf in a whole quad): fold the
            // row's quads, then the rows
            bmax = fmaxf(bmax, dpp<0x124>(bmax));
            bmax = fmaxf(bmax, dpp<0x128>(bmax));
            for (int off = 16; off < 64; off <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, off, 64));
        } else {
            for (int off = LQ; off < 64; off <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, off, 64));
        }
        const float m_new = fmaxf(m, bmax);
        if (m_new != -INFINITY && m_new > m) {
            const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] *= alpha;
            m = m_new;
        }
        wave_lds_sync();
        // ---- probabilities (two per lane) and their sum
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int e = 64 * r + lane;
            const float sv = sc[e];
            const float pv = (e < nb && sv != -INFINITY) ? __builtin_amdgcn_exp2f(sv - m) : 0.f;
            sc[e] = pv;
            ps += pv;
        }
        ps = row_sum(ps);
        for (int off = 16; off < 64; off <<= 1) ps += __shfl_xor(ps, off, 64);
        l += ps;
        wave_lds_sync();
        // ---- acc += p v, two keys per lane group and step (probabilities past
        // nb are 0 and their offsets point at row 0)
        const int vlim = (nb + KPV - 1) / KPV;
#pragma unroll 1
        for (int g = 0; g < vlim; g += kVF) {
            u32x4 w0[kVF], w1[kVF];
#pragma unroll
            for (int i = 0; i < kVF; ++i) {
                const int e0 = (g + i) * KPV + 2 * vgr;
                const u32x2 vo = *reinterpret_cast<const u32x2*>(ro + kBlk + e0);
                const char* vb = reinterpret_cast<const char*>(vg);
                w0[i] = *reinterpret_cast<const u32x4*>(vb + (uint64_t)(vo[0] + 16u * sub));
                w1[i] = *reinterpret_cast<const u32x4*>(vb + (uint64_t)(vo[1] + 16u * sub));
            }
#pragma unroll
            for (int i = 0; i < kVF; ++i) {
                const int e0 = (g + i) * KPV + 2 * vgr;
                const bf16x2 pp = {(__bf16)sc[e0], (__bf16)sc[e0 + 1]};
                const uint32_t p2 = __builtin_bit_cast(uint32_t, pp);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // (key0, key1) pairs of columns 2j and 2j+1
                    const uint32_t lo = __builtin_amdgcn_perm(w1[i][j], w0[i][j], 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(w1[i][j], w0[i][j], 0x07060302u);
                    acc[2 * j] = dot2(lo, p2, acc[2 * j]);
                    acc[2 * j + 1] = dot2(hi, p2, acc[2 * j + 1]);
                }
            }
        }
        wave_lds_sync();
    }
    // the keys of a step were spread over the lane groups: sum the groups
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int off = LPK; off < 64; off <<= 1) acc[i] += __shfl_xor(acc[i], off, 64);
}

template <int D, bool OF32>
__global__ void __launch_bounds__(kWaves * 64) attn_gather_kernel(AttnParams a)
{
    constexpr int LPK = D / 8;
    __shared__ float sc_all[kWaves][kBlk];
    __shared__ __attribute__((aligned(16))) uint32_t ro_all[kWaves][2 * kBlk];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
    if (item >= (int64_t)a.batch * a.heads * a.n_q) return;
    // head-major order: item = bh * n_q + t
    const int t = (int)(item % a.n_q);
    const int bh = (int)(item / a.n_q);
    const int b = bh / a.heads, h = bh % a.heads;
    const int sub = lane % LPK, kgrp = lane / LPK;
    typedef ScorePacked<D> SS;
    uint32_t q2[4 * SS::PC];
    load_q2<D, SS>(a.q + b * a.q_sb + h * a.q_sh + (int64_t)t * a.q_sn, lane, q2);
    float m, l, acc[8];
    gather_online<D, SS>(a.gidx + bh * a.g_bh_stride + (int64_t)t * a.topk, a.topk, true, a.n_kv,
                     a.k + b * a.k_sb + h * a.k_sh, (uint32_t)(2 * a.k_sn), a.v + b * a.v_sb + h * a.v_sh,
                     (uint32_t)(2 * a.v_sn), q2, a.scale_log2, sc_all[wave], ro_all[wave], lane, m, l, acc);
    if (kgrp == 0) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int64_t obase = b * a.o_sb + h * a.o_sh + (int64_t)t * a.o_sn + sub * 8;
        if (OF32) {
            float* op = reinterpret_cast<float*>(a.o) + obase;
            *reinterpret_cast<float4*>(op) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
            *reinterpret_cast<float4*>(op + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
        } else {
            typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
            u32x4 w;
            for (int i = 0; i < 4; ++i) {
                const bf16x2 pr = {(__bf16)(acc[2 * i] * inv), (__bf16)(acc[2 * i + 1] * inv)};
                w[i] = __builtin_bit_cast(uint32_t, pr);
            }
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.o) + obase) = w;
        }
        if (a.lse && lane == 0)
            a.lse[item] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Split form.  With the lists of all queries in hand, the work is regrouped
// by key range so that the K and V rows a workgroup gathers come from one
// 4 MB range per head, which the workgroups of one XCD share in its L2:
//   partition: every list is reordered by key range (list order kept inside
//              a range) and the range starts are recorded;
//   part:      one wave per (batch*head, range, query) attends to the keys
//              of its range and writes the unnormalised output, the max (log2
//              units) and the sum of its partial softmax;
//   merge:     one wave per (batch*head, query) rescales the partials to the
//              common max and normalises.
// Same softmax as the single pass; only float32 summation order differs.

__global__ void __launch_bounds__(kWaves * 64) gather_partition_kernel(AttnParams a)
{
    __shared__ int32_t cnt_all[kWaves][256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t rows = a.g_bh_stride == 0 ? (int64_t)a.n_q : (int64_t)a.batch * a.heads * a.n_q;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= rows) return;  // wave-level work only: no workgroup barrier below
    const int32_t* src = a.g_bh_stride == 0
                             ? a.gidx + row * a.topk
                             : a.gidx + (row / a.n_q) * a.g_bh_stride + (row % a.n_q) * a.topk;
    int32_t* dst = a.g_lists + row * a.topk;
    int32_t* offs = a.g_offs + row * (a.g_nchunk + 1);
    int32_t* cnt = cnt_all[wave];
    const int nch = a.g_nchunk;

    for (int i = lane; i < 256; i += 64) cnt[i] = 0;
    wave_lds_sync();
    // list entries are read eight per lane at a time, so that a row costs a
    // few memory latencies instead of one per 64 entries
    constexpr int EB = 8;
    for (int e0 = 0; e0 < a.topk; e0 += 64 * EB) {
        int sv[EB];
#pragma unroll
        for (int j = 0; j < EB; ++j) {
            const int e = e0 + 64 * j + lane;
            sv[j] = e < a.topk ? src[e] : -1;
        }
#pragma unroll
        for (int j = 0; j < EB; ++j)
            if (sv[j] >= 0 && sv[j] < a.n_kv) atomicAdd(&cnt[sv[j] >> a.g_shift], 1);
    }
    wave_lds_sync();
    // exclusive scan of the range counts (lane owns ranges 4*lane .. 4*lane+3)
    int v[4], tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = 4 * lane + k;
        v[k] = i < nch ? cnt[i] : 0;
        tot += v[k];
    }
    int incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    int run = incl - tot;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = 4 * lane + k;
        if (i < nch) {
            offs[i] = run;
            cnt[i] = run;  // from here on: next free slot of range i
        }
        run += v[k];
    }
    if (lane == 63) offs[nch] = incl;
    wave_lds_sync();
    // stable scatter, 64 entries at a time: a lane's slot is its range's next
    // free slot plus the number of lower lanes with the same range (found
    // with one ballot per bit of the range index)
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int sv[EB];
    for (int e0 = 0; e0 < a.topk; e0 += 64) {
        const int jb = (e0 / 64) % EB;
        if (jb == 0) {
#pragma unroll
            for (int j = 0; j < EB; ++j) {
                const int e = e0 + 64 * j + lane;
                sv[j] = e < a.topk ? src[e] : -1;
            }
        }
        int s = sv[0];
#pragma unroll
        for (int j = 1; j < EB; ++j) s = jb == j ? sv[j] : s;
        const bool ok = s >= 0 && s < a.n_kv;
        const int ch = ok ? (s >> a.g_shift) : 0;
        uint64_t m = __builtin_amdgcn_ballot_w64(ok);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = ((ch >> bit) & 1) != 0;
            const uint64_t bb = __builtin_amdgcn_ballot_w64(on);
            m &= on ? bb : ~bb;
        }
        const int rank = __popcll(m & below);
        const int base = cnt[ch];
        wave_lds_sync();
        if (ok) {
            dst[base + rank] = s;
            if ((m >> lane) == 1ull) cnt[ch] = base + rank + 1;  // the group's highest lane
        }
        wave_lds_sync();
    }
}

template <int D>
__global__ void __launch_bounds__(kWaves * 64) gather_part_kernel(AttnParams a)
{
    constexpr int LPK = D / 8;
    __shared__ float sc_all[kWaves][kBlk];
    __shared__ __attribute__((aligned(16))) uint32_t ro_all[kWaves][2 * kBlk];
    const int lane = threadIdx.x & 63;
    // uniform over the wave: the item decode and addressing below run on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // sizes fit in 32 bits (the host checks batch*heads*n_q and the range count)
    const uint32_t nq = (uint32_t)a.n_q, nch = (uint32_t)a.g_nchunk;
    const uint32_t n_items = (uint32_t)(a.batch * a.heads) * nch * nq;
    // kPartItems consecutive items per wave: item = ((bh * nchunk) + range) *
    // n_q + t, so a wave's items share their head and key range, and the waves
    // working on one key range of one head are neighbours on the same XCD
    const uint32_t first = ((uint32_t)xcd_remap(blockIdx.x, gridDim.x) * kWaves + wave) * kPartItems;
    const int sub = lane % LPK, kgrp = lane / LPK;
    int cur_rest = -1;
    int b = 0, h = 0, bh = 0, rg = 0;
    const uint16_t* kg = nullptr;
    const uint16_t* vg = nullptr;
    for (uint32_t u = 0; u < (uint32_t)kPartItems; ++u) {
        const uint32_t item = first + u;
        if (item >= n_items) break;  // uniform
        const uint32_t t = item % nq;
        const int rest = (int)(item / nq);
        if (rest != cur_rest) {  // uniform: head and range of this item
            cur_rest = rest;
            rg = rest % (int)nch;
            bh = rest / (int)nch;
            b = bh / a.heads;
            h = bh % a.heads;
            kg = a.k + b * a.k_sb + h * a.k_sh;
            vg = a.v + b * a.v_sb + h * a.v_sh;
        }
        const int64_t row = a.g_bh_stride == 0 ? (int64_t)t : (int64_t)bh * nq + t;
        const int32_t* offs = a.g_offs + row * (nch + 1);
        const int o0 = offs[rg], o1 = offs[rg + 1];
        typedef ScoreSpread<D> SS;
        uint32_t q2[4 * SS::PC];
        load_q2<D, SS>(a.q + b * a.q_sb + h * a.q_sh + (int64_t)t * a.q_sn, lane, q2);
        float m, l, acc[8];
        gather_online<D, SS>(a.g_lists + row * a.topk + o0, o1 - o0, false, a.n_kv, kg, (uint32_t)(2 * a.k_sn), vg,
                         (uint32_t)(2 * a.v_sn), q2, a.scale_log2, sc_all[wave], ro_all[wave], lane, m, l, acc);
        const int64_t pidx = ((int64_t)bh * nq + t) * nch + rg;
        if (kgrp == 0) {
            float* po = a.g_po + pidx * D + sub * 8;
            *reinterpret_cast<float4*>(po) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4*>(po + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
        if (lane == 0) {
            a.g_pml[pidx * 2] = m;  // -inf for an empty range
            a.g_pml[pidx * 2 + 1] = l;
        }
    }
}

template <int D, bool OF32>
__global__ void __launch_bounds__(kWaves * 64) gather_merge_kernel(AttnParams a)
{
    constexpr int PER = D / 64;  // output columns per lane
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (item >= (int64_t)a.batch * a.heads * a.n_q) return;
    const int t = (int)(item % a.n_q);
    const int bh = (int)(item / a.n_q);
    const int b = bh / a.heads, h = bh % a.heads;
    const float* pml = a.g_pml + item * a.g_nchunk * 2;
    const float* po = a.g_po + item * a.g_nchunk * D;
    // one online pass over the ranges, sixteen at a time: a batch's partial
    // rows, maxima and sums are all requested before any is used, then the
    // running result is rescaled to the batch's max and the batch added
    constexpr int RB = 16;
    float m = -INFINITY, l = 0.f, acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    for (int r0 = 0; r0 < a.g_nchunk; r0 += RB) {
        float mr[RB], lr[RB], pv[RB][PER];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const int r = r0 + j;
            const bool in = r < a.g_nchunk;
            mr[j] = in ? pml[2 * r] : -INFINITY;
            lr[j] = in ? pml[2 * r + 1] : 0.f;
#pragma unroll
            for (int i = 0; i < PER; ++i) pv[j][i] = in ? po[r * D + lane * PER + i] : 0.f;
        }
        float bm = mr[0];
#pragma unroll
        for (int j = 1; j < RB; ++j) bm = fmaxf(bm, mr[j]);
        if (bm == -INFINITY) continue;  // every range of the batch is empty
        if (bm > m) {
            // m == -inf: nothing accumulated yet, factor 0
            const float g = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - bm);
            l *= g;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] *= g;
            m = bm;
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            // an empty range has max -inf: factor 0
            const float f = mr[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mr[j] - m);
            l = __builtin_fmaf(lr[j], f, l);
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(pv[j][i], f, acc[i]);
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t obase = b * a.o_sb + h * a.o_sh + (int64_t)t * a.o_sn + lane * PER;
    if (OF32) {
        float* op = reinterpret_cast<float*>(a.o) + obase;
#pragma unroll
        for (int i = 0; i < PER; ++i) op[i] = acc[i] * inv;
    } else {
        uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + obase;
#pragma unroll
        for (int i = 0; i < PER; ++i) op[i] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] * inv));
    }
    if (a.lse && lane == 0)
        a.lse[item] = l > 0.f ? (m + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

template <int D, bool OF32>
hipError_t launch_one(const AttnParams& a, hipStream_t stream)
{
    const int64_t items = (int64_t)a.batch * a.heads * a.n_q;
    const int64_t wgs = (items + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((attn_gather_kernel<D, OF32>), dim3((unsigned)wgs), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool OF32>
hipError_t launch_split(const AttnParams& a, hipStream_t stream)
{
    const int64_t rows = a.g_bh_stride == 0 ? (int64_t)a.n_q : (int64_t)a.batch * a.heads * a.n_q;
    hipLaunchKernelGGL(gather_partition_kernel, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kWaves * 64), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t parts = (int64_t)a.batch * a.heads * a.g_nchunk * a.n_q;
    const int64_t per_wg = (int64_t)kWaves * kPartItems;
    hipLaunchKernelGGL((gather_part_kernel<D>), dim3((unsigned)((parts + per_wg - 1) / per_wg)), dim3(kWaves * 64),
                       0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)a.batch * a.heads * a.n_q;
    hipLaunchKernelGGL((gather_merge_kernel<D, OF32>), dim3((unsigned)((items + kWaves - 1) / kWaves)),
                       dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_gather_split(const AttnParams& a, int head_dim, int o_f32, hipStream_t stream)
{
    if (head_dim == 128) return o_f32 ? launch_split<128, true>(a, stream) : launch_split<128, false>(a, stream);
    if (head_dim == 64) return o_f32 ? launch_split<64, true>(a, stream) : launch_split<64, false>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_attn_gather(const AttnParams& a, int head_dim, int o_f32, hipStream_t stream)
{
    if (head_dim == 128) return o_f32 ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
    if (head_dim == 64) return o_f32 ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace sa
