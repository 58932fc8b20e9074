// indexer_topk.hip -- indexer scores and per-query top-k selection.
//
// "Sparse Attention" glossary, section on common sparsity patterns: DeepSeek
// Sparse Attention runs a small indexer that scores every earlier token for
// each query, then attends only to the 2,048 best-scored tokens.  The pages
// give no indexer formula; the score used here is the plain dot product of
// the indexer query and key, accumulated in float32 as one fused
// multiply-add chain in dimension order (a fixed order makes the selection
// reproducible bit for bit); the chain runs on the float32 matrix cores.
// Ties in the selection go to the lower index.
#include "sa_internal.h"

#include <mutex>

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------------------
// Indexer on the float32 matrix cores.  v_mfma_f32_32x32x1_2b_f32 takes one
// dimension per instruction: every output gets exactly one multiply-add per
// step, and the product of two bfloat16 values is exact in float32, so a
// chain of these instructions in dimension order rounds exactly like the
// sequential fused-multiply-add chain (checked bit for bit, denormal sums
// included).  Operands: A = the lane's key (lanes 0-31 keys 0-31 of the
// tile, lanes 32-63 keys 32-63), B = the lane's query (both halves hold the
// same 32 queries), so the two 32 x 32 blocks cover 32 queries x 64 keys.
// Result element (reg r, lane l): query l % 32, key 32*(r/16) + 8*((r%16)/4)
// + 4*(l/32) + r%4, i.e. runs of four consecutive keys of one query row.
// A wave owns 32 queries and walks a 512-key chunk in 64-key tiles; the next
// tile's key rows are loaded while the current tile's chain runs.
typedef __attribute__((ext_vector_type(32))) float f32x32;
constexpr int XQ = 32;    // queries per wave
constexpr int XW = 4;     // waves per workgroup
constexpr int XT = 64;    // keys per tile
constexpr int XKC = 512;  // keys per workgroup

__device__ __forceinline__ float bf16_at(const uint32_t (&p)[32], int j)
{
    return __uint_as_float((j & 1) ? (p[j >> 1] & 0xFFFF0000u) : (p[j >> 1] << 16));
}

__device__ __forceinline__ void load_row64(const uint16_t* row, bool ok, int nd, uint32_t (&p)[32])
{
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ok && 8 * g < nd) w = *reinterpret_cast<const u32x4*>(row + 8 * g);
        p[4 * g + 0] = w[0];
        p[4 * g + 1] = w[1];
        p[4 * g + 2] = w[2];
        p[4 * g + 3] = w[3];
    }
}

// The chain over the tiles [s_begin, s_end) (64 keys each) for the wave's 32
// query rows r0 .. r0 + 31: emit(s0, acc) receives each tile's 32 x 64
// scores in the layout above.  Key rows past n_kv read as row n_kv - 1 (the
// caller drops those entries).
template <class Emit>
__device__ __forceinline__ void indexer_walk(const uint16_t* __restrict__ qi, const uint16_t* __restrict__ ki,
                                             int32_t n_q, int32_t n_kv, int32_t d, int r0, int s_begin,
                                             int s_end, Emit&& emit)
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int r = r0 + col;  // this lane's query
    const bool r_ok = r < n_q;
    const uint16_t* qrow = qi + (int64_t)(r_ok ? r : 0) * d;
    const int nch = (d + 63) >> 6;

    uint32_t qp[32], kp[32], kn[32];
    float qv[64];
    if (nch == 1) {
        load_row64(qrow, r_ok, d, qp);
#pragma unroll
        for (int j = 0; j < 64; ++j) qv[j] = bf16_at(qp, j);
    }
    auto key_row = [&](int s0) { return ki + (int64_t)min(s0 + lane, n_kv - 1) * d; };
    if (nch == 1) load_row64(key_row(s_begin), s_begin + lane < n_kv, d, kn);

    for (int s0 = s_begin; s0 < s_end; s0 += XT) {
        f32x32 acc;
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] = 0.f;
        if (nch == 1) {
#pragma unroll
            for (int i = 0; i < 32; ++i) kp[i] = kn[i];
            if (s0 + XT < s_end) load_row64(key_row(s0 + XT), s0 + XT + lane < n_kv, d, kn);
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                if (8 * g >= d) break;  // uniform
#pragma unroll
                for (int x = 0; x < 8; ++x)
                    acc = __builtin_amdgcn_mfma_f32_32x32x1f32(bf16_at(kp, 8 * g + x), qv[8 * g + x], acc, 0, 0, 0);
            }
        } else {
            const uint16_t* krow = key_row(s0);
            const bool s_ok = s0 + lane < n_kv;
            for (int c = 0; c < nch; ++c) {
                const int c0 = 64 * c, nd = min(64, d - c0);
                load_row64(qrow + c0, r_ok, nd, qp);
                load_row64(krow + c0, s_ok, nd, kp);
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    if (8 * g >= nd) break;  // uniform
#pragma unroll
                    for (int x = 0; x < 8; ++x)
                        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(bf16_at(kp, 8 * g + x), bf16_at(qp, 8 * g + x), acc, 0, 0, 0);
                }
            }
        }
        emit(s0, acc);
    }
}

__global__ void __launch_bounds__(64 * XW, 2)
indexer_kernel(const uint16_t* __restrict__ qi, const uint16_t* __restrict__ ki, int32_t n_q,
               int32_t n_kv, int32_t d, int32_t q_offset, float* __restrict__ scores)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int hh = lane >> 5, col = lane & 31;
    const int r0 = (blockIdx.y * XW + w) * XQ;
    if (r0 >= n_q) return;  // no barriers in this kernel: waves leave on their own
    const int s_begin = blockIdx.x * XKC;
    const int t_max = q_offset + min(r0 + XQ, n_q) - 1;  // last query position of the wave
    const int s_end = min(min(s_begin + XKC, n_kv), t_max + 1);
    if (s_begin >= s_end) return;

    const int r = r0 + col;  // this lane's query
    const bool r_ok = r < n_q;
    const int t = q_offset + r;
    float* orow = scores + (int64_t)(r_ok ? r : 0) * n_kv;
    const bool vec_ok = (n_kv & 3) == 0;

    indexer_walk(qi, ki, n_q, n_kv, d, r0, s_begin, s_end, [&](int s0, const f32x32& acc) {
        if (!r_ok) return;
        // entries s <= t of this query row, s < n_kv
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int sk = s0 + 32 * b + 8 * m + 4 * hh;
                const float v0 = acc[16 * b + 4 * m + 0], v1 = acc[16 * b + 4 * m + 1];
                const float v2 = acc[16 * b + 4 * m + 2], v3 = acc[16 * b + 4 * m + 3];
                if (vec_ok && sk + 3 <= t && sk + 3 < n_kv) {
                    *reinterpret_cast<float4*>(orow + sk) = make_float4(v0, v1, v2, v3);
                } else {
                    if (sk + 0 <= t && sk + 0 < n_kv) orow[sk + 0] = v0;
                    if (sk + 1 <= t && sk + 1 < n_kv) orow[sk + 1] = v1;
                    if (sk + 2 <= t && sk + 2 < n_kv) orow[sk + 2] = v2;
                    if (sk + 3 <= t && sk + 3 < n_kv) orow[sk + 3] = v3;
                }
            }
    });
}

// ---------------------------------------------------------------------------
// Top-k: one workgroup of 256 threads per query row, several rows per CU.
//
// The row is read from HBM once.  The first eighth of that pass -- 128 runs
// of 64 keys spread evenly over the row -- is a sample that brackets the key T of the k-th
// largest candidate: two 11-bit digit levels of sample histograms give keys
// LO <= HI whose sample ranks lie a few standard deviations either side of
// the rank k maps to.  One pass over the row then marks every candidate with
// key >= HI as selected (bitmap in LDS), counts them, and keeps the candidates
// in [LO, HI) -- about 1,200 for k = 2,048 of 65,536 -- in LDS.  If the
// counts show that T lies in the bracket, an exact radix selection on the
// kept keys (relative to LO, 11-bit digits) finds T and how many of the
// candidates equal to T are taken; otherwise (ties, adversarial orders) the
// same exact selection runs over the whole row from memory.  A bitmap of
// selected positions plus one of ties then gives each thread its output slots
// after one block scan, and the indices leave in ascending order through an
// LDS staging buffer with coalesced stores.
constexpr int KTH = 256;                   // threads per row
constexpr int KWAVES = KTH / 64;
constexpr int KMAXN = 65536;               // candidates per row at most
constexpr int KWORDS = KMAXN / 32;         // bitmap words
constexpr int KWCAP = 512;                 // kept keys per wave
constexpr int KCAP = KWCAP * KWAVES;       // kept keys per row
constexpr int KBINS = 2048;                // 11-bit digits
constexpr int KBATCH = 8;                  // float4 loads in flight per thread

// Order-preserving 32-bit key: larger float, larger key; -0.0 and +0.0 map to
// one key; every NaN maps to the largest key.
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t k = (u >> 31) ? ~u : (u | 0x80000000u);
    k = a == 0u ? 0x80000000u : k;
    return a > 0x7F800000u ? 0xFFFFFFFFu : k;
}

struct __attribute__((aligned(16))) TopkLds {
    uint32_t sel[KWORDS];    // bit p: candidate p is selected
    uint32_t hist[KBINS];    // digit histogram; tie bitmap once T is known
    uint32_t mid[2 * KCAP];  // kept keys [KCAP], their positions [KCAP]; output staging
    uint32_t wsum[KWAVES];
    uint32_t wcnt[KWAVES];
    uint32_t state[4];
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Exclusive scan over the KTH threads; *total gets the sum.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v, lane);
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < KWAVES; ++i) {
        const uint32_t s = wsum[i];
        before += i < w ? s : 0u;
        tot += s;
    }
    *total = tot;
    __syncthreads();
    return x - v + before;
}

// Maximum over the KTH threads (every thread gets it).
__device__ uint32_t block_max(uint32_t v, uint32_t* wmax)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor(v, off, 64));
    if (lane == 0) wmax[w] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < KWAVES; ++i) m = max(m, wmax[i]);
    __syncthreads();
    return m;
}

// For ranks r0, r1 (1-based from the largest digit down; 0 = not asked), the
// digit whose bin holds the rank and the rank left inside that bin, into
// state[0..1] and state[2..3].  Ends with a barrier.
template <class Lds>
__device__ void find_digits(Lds& L, uint32_t r0, uint32_t r1)
{
    const int tid = threadIdx.x;
    // thread t owns bins KBINS-1-8t down to KBINS-8-8t
    const uint4 a = *reinterpret_cast<const uint4*>(&L.hist[KBINS - 8 - 8 * tid]);
    const uint4 b = *reinterpret_cast<const uint4*>(&L.hist[KBINS - 4 - 8 * tid]);
    const uint32_t c[8] = {b.w, b.z, b.y, b.x, a.w, a.z, a.y, a.x};
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += c[j];
    uint32_t total;
    const uint32_t excl = block_excl_scan(sum, L.wsum, &total);
    const uint32_t rs[2] = {r0, r1};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint32_t r = rs[q];
        if (r > excl && r <= excl + sum) {
            uint32_t run = excl;
            for (int j = 0; j < 8; ++j) {
                if (run + c[j] >= r) {
                    L.state[2 * q] = (uint32_t)(KBINS - 1 - 8 * tid - j);
                    L.state[2 * q + 1] = r - run;
                    break;
                }
                run += c[j];
            }
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void zero_words(uint32_t* p, int n)
{
    for (int i = threadIdx.x * 4; i < n; i += KTH * 4)
        *reinterpret_cast<uint4*>(p + i) = make_uint4(0u, 0u, 0u, 0u);
}

// Exact selection: among the keys v (of `width` significant bits) that
// for_each(f) hands to f, the r-th largest.  Returns its value and how many
// of the keys equal to it rank within the first r.
template <class Lds, class ForEach>
__device__ void radix_select(Lds& L, ForEach&& for_each, uint32_t width, uint32_t r,
                             uint32_t& value, uint32_t& rem)
{
    uint32_t P = 0, done = 0;
    rem = r;
    while (done < width) {
        const uint32_t nb = min(11u, width - done);
        const uint32_t s = width - done - nb;
        const uint32_t top = s + nb;
        const uint32_t msk = (1u << nb) - 1u;
        zero_words(L.hist, KBINS);
        __syncthreads();
        for_each([&](uint32_t v) {
            if (((uint64_t)v >> top) == (uint64_t)P) atomicAdd(&L.hist[(v >> s) & msk], 1u);
        });
        __syncthreads();
        find_digits(L, rem, 0u);
        P = (P << nb) | L.state[0];
        rem = L.state[1];
        done += nb;
    }
    value = P;
}

// The selected keys leave in ascending position order: every position whose
// bit is set in `sel`, plus the first need_eq positions (lowest first) whose
// bit is set in `tie` (bitmaps of KMAXN positions).  Thread t owns positions
// [256t, 256t + 256); `stage` (k words of LDS) orders the output so the
// stores are coalesced.
template <class Lds>
__device__ void emit_ascending(Lds& L, const uint32_t* sel, const uint32_t* tie, uint32_t need_eq, int32_t k,
                               uint32_t* stage, int32_t* __restrict__ out)
{
    const int tid = threadIdx.x;
    uint32_t sw[8], tw[8];
    {
        const uint4 s0 = *reinterpret_cast<const uint4*>(&sel[8 * tid]);
        const uint4 s1 = *reinterpret_cast<const uint4*>(&sel[8 * tid + 4]);
        const uint4 t0 = *reinterpret_cast<const uint4*>(&tie[8 * tid]);
        const uint4 t1 = *reinterpret_cast<const uint4*>(&tie[8 * tid + 4]);
        sw[0] = s0.x; sw[1] = s0.y; sw[2] = s0.z; sw[3] = s0.w;
        sw[4] = s1.x; sw[5] = s1.y; sw[6] = s1.z; sw[7] = s1.w;
        tw[0] = t0.x; tw[1] = t0.y; tw[2] = t0.z; tw[3] = t0.w;
        tw[4] = t1.x; tw[5] = t1.y; tw[6] = t1.z; tw[7] = t1.w;
    }
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        n_gt += (uint32_t)__popc(sw[i]);
        n_eq += (uint32_t)__popc(tw[i]);
    }
    // one scan of (n_gt << 16 | n_eq): neither prefix reaches 2^16.  Ties are
    // taken in position order, so the ties taken before this thread number
    // min(need_eq, ties before it).
    uint32_t tot;
    const uint32_t ex = block_excl_scan((n_gt << 16) | n_eq, L.wsum, &tot);
    // (No conditional unsigned difference here: written as need_eq > e ?
    // need_eq - e : 0, the subtraction gets hoisted with a no-wrap flag and
    // the minimum below folds as if need_eq >= e always held.)
    const uint32_t eq_before = ex & 0xFFFFu;
    const uint32_t taken_before = min(need_eq, eq_before);
    uint32_t take = min(need_eq, eq_before + n_eq) - taken_before;
    uint32_t pos = (ex >> 16) + taken_before;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t m = sw[i], te = tw[i];
        while (te && take) {  // lowest-index ties first
            const uint32_t low = te & (0u - te);
            m |= low;
            te ^= low;
            --take;
        }
        while (m) {
            if (pos < (uint32_t)k) stage[pos] = (uint32_t)(256 * tid + 32 * i + __builtin_ctz(m));
            ++pos;
            m &= m - 1u;
        }
    }
    __syncthreads();
    for (int e = tid; e < k; e += KTH) out[e] = (int32_t)stage[e];
}

template <bool ALIGNED>
__global__ void __launch_bounds__(KTH)
topk_kernel(const float* __restrict__ scores, int32_t n_q, int32_t n_kv, int32_t q_offset,
            int32_t k, int32_t* __restrict__ idx_out)
{
    __shared__ TopkLds L;
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int64_t t = (int64_t)q_offset + r;
    const int n_cand = (int)min((int64_t)n_kv, t + 1);
    const float* row = scores + (int64_t)r * n_kv;
    int32_t* out = idx_out + (int64_t)r * k;

    if (n_cand <= k) {
        for (int e = tid; e < k; e += KTH) out[e] = e < n_cand ? e : -1;
        return;
    }

    // Thread t reads, at step `it`, the float4 of positions 4g .. 4g+3 with
    // g = 1024*(t/16) + 16*it + t%16: each step covers 16 runs of 64 keys, one
    // in each sixteenth of the row.  Steps are taken in the order 0, 8, ..,
    // 56, 1, 9, .., so the first batch of eight -- keys p with p % 512 < 64,
    // an eighth of the row spread evenly over it -- is the sample.
    auto pos_of = [&](int it) { return 4 * (((tid >> 4) << 10) + (it << 4) + (tid & 15)); };
    auto load1 = [&](int it) {
        const int base = pos_of(it);
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ALIGNED) {
            if (base < n_cand) f = *reinterpret_cast<const float4*>(row + base);
        } else {
            if (base + 0 < n_cand) f.x = row[base + 0];
            if (base + 1 < n_cand) f.y = row[base + 1];
            if (base + 2 < n_cand) f.z = row[base + 2];
            if (base + 3 < n_cand) f.w = row[base + 3];
        }
        return f;
    };
    float4 nxt[KBATCH], cur[KBATCH];
#pragma unroll
    for (int j = 0; j < KBATCH; ++j) nxt[j] = load1(KBATCH * j);
#pragma unroll
    for (int j = 0; j < KBATCH; ++j) cur[j] = nxt[j];
#pragma unroll
    for (int j = 0; j < KBATCH; ++j) nxt[j] = load1(KBATCH * j + 1);  // in flight meanwhile
    zero_words(L.sel, KWORDS);
    zero_words(L.hist, KBINS);
    __syncthreads();

    // ---- bracket from the sample ----
    uint32_t skey[KBATCH][4];
    uint32_t svalid = 0;  // bit 4j + x
#pragma unroll
    for (int j = 0; j < KBATCH; ++j) {
        const int base = pos_of(KBATCH * j);
        skey[j][0] = order_key(cur[j].x);
        skey[j][1] = order_key(cur[j].y);
        skey[j][2] = order_key(cur[j].z);
        skey[j][3] = order_key(cur[j].w);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const bool v = base + x < n_cand;
            svalid |= (v ? 1u : 0u) << (4 * j + x);
            if (v) atomicAdd(&L.hist[skey[j][x] >> 21], 1u);
        }
    }
    __syncthreads();
    const uint32_t s_n = (uint32_t)((n_cand >> 9) * 64 + min(n_cand & 511, 64));
    // sample ranks a few standard deviations either side of k's image
    const float rho = (float)k * (float)s_n / (float)n_cand;
    const float delta = 4.0f * sqrtf(rho) + 8.0f;
    const float fhi = floorf(rho - delta), flo = ceilf(rho + delta);
    const uint32_t r_hi = fhi < 1.0f ? 0u : (uint32_t)fhi;
    const uint32_t r_lo = flo > (float)s_n ? 0u : (uint32_t)flo;
    find_digits(L, r_hi, r_lo);
    const uint32_t b_hi = L.state[0], q_hi = L.state[1];
    const uint32_t b_lo = L.state[2], q_lo = L.state[3];
    uint64_t HI = uint64_t(1) << 32;  // keys >= HI: selected for sure
    uint32_t LO = 0;                  // keys in [LO, HI): kept
#pragma unroll
    for (int side = 0; side < 2; ++side) {
        const uint32_t rk = side == 0 ? r_hi : r_lo;
        if (rk == 0) continue;  // uniform
        const uint32_t b1 = side == 0 ? b_hi : b_lo;
        zero_words(L.hist, KBINS);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KBATCH; ++j)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (((svalid >> (4 * j + x)) & 1u) && (skey[j][x] >> 21) == b1)
                    atomicAdd(&L.hist[(skey[j][x] >> 10) & (KBINS - 1)], 1u);
        __syncthreads();
        find_digits(L, side == 0 ? q_hi : q_lo, 0u);
        const uint32_t b2 = L.state[0];
        if (side == 0)
            HI = ((uint64_t)b1 << 21) + ((uint64_t)(b2 + 1) << 10);
        else
            LO = (b1 << 21) | (b2 << 10);
    }
    const uint32_t HIm1 = (uint32_t)(HI - 1);

    // ---- one pass over the row ----
    uint32_t woff = 0;  // kept keys of this wave so far (wave-uniform)
    uint32_t c_hi = 0;  // keys >= HI of this thread
    uint32_t* mkey = L.mid + w * KWCAP;
    uint32_t* midx = L.mid + KCAP + w * KWCAP;
    auto take4 = [&](int base, const uint32_t (&u)[4]) {
        uint32_t nib = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const bool valid = base + x < n_cand;
            const bool gh = valid && u[x] > HIm1;
            const bool md = valid && u[x] >= LO && u[x] <= HIm1;
            nib |= (gh ? 1u : 0u) << x;
            const uint64_t bm = __ballot(md);
            if (bm) {
                const uint32_t pos = woff + __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
                if (md && pos < (uint32_t)KWCAP) {
                    mkey[pos] = u[x];
                    midx[pos] = (uint32_t)(base + x);
                }
                woff += (uint32_t)__popcll(bm);
            }
        }
        if (nib) {
            atomicOr(&L.sel[base >> 5], nib << (base & 31));
            c_hi += (uint32_t)__popc(nib);
        }
    };
#pragma unroll
    for (int j = 0; j < KBATCH; ++j) take4(pos_of(KBATCH * j), skey[j]);
#pragma unroll 1
    for (int b0 = 1; b0 < KBATCH; ++b0) {
#pragma unroll
        for (int j = 0; j < KBATCH; ++j) cur[j] = nxt[j];
        if (b0 + 1 < KBATCH) {
#pragma unroll
            for (int j = 0; j < KBATCH; ++j) nxt[j] = load1(KBATCH * j + b0 + 1);
        }
#pragma unroll
        for (int j = 0; j < KBATCH; ++j) {
            const uint32_t u[4] = {order_key(cur[j].x), order_key(cur[j].y), order_key(cur[j].z),
                                   order_key(cur[j].w)};
            take4(pos_of(KBATCH * j + b0), u);
        }
    }
    if (lane == 0) L.wcnt[w] = woff;
    uint32_t n_hi;
    (void)block_excl_scan(c_hi, L.wsum, &n_hi);  // barriers publish wcnt too
    uint32_t n_mid = 0;
    bool ovf = false;
#pragma unroll
    for (int i = 0; i < KWAVES; ++i) {
        n_mid += L.wcnt[i];
        ovf |= L.wcnt[i] > (uint32_t)KWCAP;
    }

    uint32_t* tie = L.hist;
    uint32_t T, need_eq;
    if (!ovf && n_hi < (uint32_t)k && n_hi + n_mid >= (uint32_t)k) {
        // ---- exact selection among the kept keys ----
        const uint64_t span = HI - LO;  // >= 1
        const uint32_t width = span <= 1 ? 0u : 64u - (uint32_t)__clzll(span - 1);
        auto kept = [&](auto&& f) {
#pragma unroll
            for (int i = 0; i < KWAVES; ++i) {
                const uint32_t n = L.wcnt[i];
                for (uint32_t j = tid; j < n; j += KTH) f(L.mid[i * KWCAP + j] - LO);
            }
        };
        uint32_t rel;
        radix_select(L, kept, width, (uint32_t)k - n_hi, rel, need_eq);
        T = LO + rel;
        zero_words(tie, KWORDS);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KWAVES; ++i) {
            const uint32_t n = L.wcnt[i];
            for (uint32_t j = tid; j < n; j += KTH) {
                const uint32_t u = L.mid[i * KWCAP + j], p = L.mid[KCAP + i * KWCAP + j];
                if (u > T) atomicOr(&L.sel[p >> 5], 1u << (p & 31));
                else if (u == T) atomicOr(&tie[p >> 5], 1u << (p & 31));
            }
        }
    } else {
        // ---- exact selection over the whole row ----
        auto all = [&](auto&& f) {
            for (int p = tid; p < n_cand; p += KTH) f(order_key(row[p]));
        };
        radix_select(L, all, 32u, (uint32_t)k, T, need_eq);
        // every bitmap word is written once: 64 positions per wave step
        for (int p0 = 0; p0 < KMAXN; p0 += KTH) {
            const int p = p0 + tid;
            uint32_t u = 0;
            const bool valid = p < n_cand;
            if (valid) u = order_key(row[p]);
            const uint64_t g = __ballot(valid && u > T);
            const uint64_t e = __ballot(valid && u == T);
            if (lane == 0) {
                const int wd = (p0 + 64 * w) >> 5;
                L.sel[wd] = (uint32_t)g;
                L.sel[wd + 1] = (uint32_t)(g >> 32);
                tie[wd] = (uint32_t)e;
                tie[wd + 1] = (uint32_t)(e >> 32);
            }
        }
    }
    __syncthreads();

    emit_ascending(L, L.sel, tie, need_eq, k, L.mid, out);
}

// ---------------------------------------------------------------------------
// Streaming indexer + top-k: the selection without the score matrix.
//
// 1. stream_sample_kernel scores one 64-key tile in every SPERIOD keys (a
//    1/32 sample spread over the row) on the float32 chain and stores their
//    order keys (0 where a key is not a candidate).
// 2. stream_bracket_kernel picks, per query row, the order key LO of the
//    sample rank rho + 6 sqrt(rho) + 8, rho = k * sample size / candidates:
//    LO sits well below the k-th largest candidate, so about 1.9 k
//    candidates have keys >= LO.  LO = 0 marks a row that goes the direct
//    way (too few candidates for a sample).  The same launch stores the
//    largest key norm of every 64-key tile (stream_norm_tiles).
// 3. stream_filter_kernel scores every candidate approximately on bf16
//    matrix instructions (the products of two bf16 values are exact; only
//    the order and rounding of the float32 sums differ from the chain) and
//    keeps the position of every candidate whose approximate score is not
//    below LO minus a bound on that difference, in a region of SCAP slots
//    per (row, 512-key chunk) that the two half-waves holding the row fill
//    from either end, counting on once their counts add up to more than
//    SCAP.  Every candidate whose chain score reaches LO is kept.
// 4. stream_select_kernel, one workgroup per row: every kept candidate's
//    chain score lies within a known bound of its stored approximate score,
//    so the k-th largest approximate score brackets the k-th chain score;
//    candidates clear of that bracket are in or out for certain, and only
//    the few inside it are scored on the exact chain and ranked (ties in
//    position order).  The selected positions leave ascending.
// 5. A row step 4 cannot settle (an adversarial order that fooled the
//    sample, a region that overflowed, a non-finite score) is selected by
//    the same workgroup directly (select_direct): its scores are recomputed
//    with the same float32 chain at each pass of an exact selection over the
//    whole row.
constexpr int SPERIOD = kStreamPeriod;  // keys per sample tile
constexpr int SCAP = kStreamCap;        // kept slots per (row, chunk)
static_assert(kStreamChunk == XKC, "filter regions are the indexer's key chunks");
static_assert(SCAP % 8 == 0, "regions are loaded in 16-byte pieces");
static_assert(64 * (KMAXN / SPERIOD) <= KTH * 8, "sample row fits the bracket kernel's registers");

__global__ void __launch_bounds__(64 * XW, 2)
stream_sample_kernel(const uint16_t* __restrict__ qi, const uint16_t* __restrict__ ki, int32_t n_q, int32_t n_kv,
                     int32_t d, int32_t q_offset, uint32_t* __restrict__ samp, int32_t s_max)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int hh = lane >> 5, col = lane & 31;
    const int r0 = (blockIdx.y * XW + w) * XQ;
    if (r0 >= n_q) return;
    const int s_begin = blockIdx.x * SPERIOD;
    const int r = r0 + col;
    const bool r_ok = r < n_q;
    const int t = q_offset + r;
    uint32_t* srow = samp + (int64_t)(r_ok ? r : 0) * s_max + blockIdx.x * XT;
    auto store = [&](int s0, const f32x32* acc) {
        if (!r_ok) return;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int j = 32 * b + 8 * m + 4 * hh;
                uint32_t u[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int sk = s0 + j + i;
                    u[i] = (acc && sk <= t && sk < n_kv) ? order_key((*acc)[16 * b + 4 * m + i]) : 0u;
                }
                *reinterpret_cast<uint4*>(srow + j) = make_uint4(u[0], u[1], u[2], u[3]);
            }
    };
    if (s_begin > q_offset + min(r0 + XQ, n_q) - 1) {  // no candidate of the wave in this tile
        store(s_begin, nullptr);
        return;
    }
    indexer_walk(qi, ki, n_q, n_kv, d, r0, s_begin, s_begin + XT,
                 [&](int s0, const f32x32& acc) { store(s0, &acc); });
}

__device__ void stream_norm_tiles(const uint16_t* __restrict__ ki, int32_t n_kv, int32_t d, int32_t ntile,
                                  float* __restrict__ tnorm, int blk);

struct __attribute__((aligned(16))) BracketLds {
    uint32_t hist[KBINS];
    uint32_t wsum[KWAVES];
    uint32_t state[4];
};

// The first nnorm blocks store the key tiles' norms (stream_norm_tiles), the
// rest pick LO, one block per query row.
__global__ void __launch_bounds__(KTH)
stream_bracket_kernel(const uint32_t* __restrict__ samp, int32_t s_max, int32_t n_kv, int32_t q_offset, int32_t k,
                      uint32_t* __restrict__ lo, const uint16_t* __restrict__ ki, int32_t d, int32_t ntile,
                      int32_t nnorm, float* __restrict__ tnorm)
{
    if ((int)blockIdx.x < nnorm) {
        stream_norm_tiles(ki, n_kv, d, ntile, tnorm, (int)blockIdx.x);
        return;
    }
    __shared__ BracketLds L;
    const int r = (int)blockIdx.x - nnorm, tid = threadIdx.x;
    const int64_t t = (int64_t)q_offset + r;
    const int n_cand = (int)min((int64_t)n_kv, t + 1);
    // sample positions among the candidates: the first XT of every SPERIOD
    const int s_n = (n_cand / SPERIOD) * XT + min(n_cand % SPERIOD, XT);
    const float rho = (float)k * (float)s_n / (float)max(n_cand, 1);
    const float frank = ceilf(rho + 6.0f * sqrtf(rho) + 8.0f);
    if (n_cand <= k || frank > (float)s_n) {
        if (tid == 0) lo[r] = 0u;  // selected directly
        return;
    }
    constexpr int PER = 8;  // s_max <= 64 * 32 = KTH * PER
    uint32_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int j = tid + KTH * i;
        v[i] = j < s_max ? samp[(int64_t)r * s_max + j] : 0u;
    }
    auto each = [&](auto&& f) {
#pragma unroll
        for (int i = 0; i < PER; ++i) f(v[i]);
    };
    uint32_t value, rem;
    radix_select(L, each, 32u, (uint32_t)frank, value, rem);
    // >= 1, since 0 is no float's key; a NaN threshold (so many NaN scores) goes
    // the direct way
    if (tid == 0) lo[r] = value == 0xFFFFFFFFu ? 0u : value;
}

// The float whose order key is `key` (key < 0xFFFFFFFF, i.e. not a NaN):
// for every float v that is not a NaN, order_key(v) >= key exactly when
// v >= key_float(key), and a NaN v passes !(v < key_float(key)) as well.
__device__ __forceinline__ float key_float(uint32_t key)
{
    return __uint_as_float(key >= 0x80000000u ? key & 0x7FFFFFFFu : ~key);
}

// Largest norm of the key rows of every 64-key tile (one wave per tile, the
// float32 sum of squares in dimension order, rows past n_kv skipped); block
// `blk` of KTH threads covers tiles 4*blk .. 4*blk + 3.
__device__ void stream_norm_tiles(const uint16_t* __restrict__ ki, int32_t n_kv, int32_t d, int32_t ntile,
                                  float* __restrict__ tnorm, int blk)
{
    static_assert(KTH == 256, "four tiles per block");
    const int tile = blk * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (tile >= ntile) return;
    const int s = tile * 64 + lane;
    float ss = 0.f;
    if (s < n_kv) {
        const uint16_t* kr = ki + (int64_t)s * d;
        for (int i = 0; i < d; i += 8) {
            const u32x4 kw = *reinterpret_cast<const u32x4*>(kr + i);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float lo = __uint_as_float(kw[x] << 16), hi = __uint_as_float(kw[x] & 0xFFFF0000u);
                ss = __builtin_fmaf(lo, lo, ss);
                ss = __builtin_fmaf(hi, hi, ss);
            }
        }
    }
    float m = sqrtf(ss);
    // a non-finite norm stays the maximum (NaN compares false: keep it)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(m, off);
        m = (o > m || o != o) ? o : m;
    }
    if (lane == 0) tnorm[tile] = m;
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// The approximate scores: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = the
// lane's key row, B = the lane's query), two 32-key blocks per 64-key tile;
// element i of block b of a lane is key s0 + 32b + 8(i/4) + 4hh + i%4 of query
// col.  The sum of d exact products differs from the dimension-order chain
// only in the order and rounding of its float32 additions: each of the two is
// within (d - 1) u sum|q_i k_i| of the exact dot product (u = 2^-24; twice u
// for an adder that truncates), and sum|q_i k_i| <= |q| |k|, so the two scores
// differ by less than 4 d u |q| |k| (+1 % for the rounding of the norms, plus
// d * 2^-125 for flushed denormal partial sums).  A candidate is kept when its
// approximate score is not below LO's float minus that bound, with |k| the
// tile's largest key norm: every candidate whose chain score reaches LO passes.
template <int NC>
__global__ void __launch_bounds__(64 * XW, 2)
stream_filter_kernel(const uint16_t* __restrict__ qi, const uint16_t* __restrict__ ki, int32_t n_q, int32_t n_kv,
                     int32_t d, int32_t q_offset, const uint32_t* __restrict__ lo, const float* __restrict__ tnorm,
                     int32_t nchunk, uint32_t* __restrict__ ccnt, uint32_t* __restrict__ ckept)
{
    // the workgroup's four waves share each 64-key tile, staged in LDS through
    // registers (double-buffered, the next tile's loads in flight during this
    // tile's products); rows padded to KRS elements so that the A-operand
    // reads of 16 lanes hit distinct banks
    constexpr int KRS = NC * 16 + 8;
    constexpr int CPR = NC * 2;                                // 16-byte chunks per row
    constexpr int SPT = (XT * CPR + 64 * XW - 1) / (64 * XW);  // chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t kt[2][XT * KRS];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hh = lane >> 5, col = lane & 31;
    const int rg0 = blockIdx.y * XW * XQ;  // the workgroup's first query row
    if (rg0 >= n_q) return;
    const int s_begin = blockIdx.x * XKC;
    const int s_end_g = min(min(s_begin + XKC, n_kv), q_offset + min(rg0 + XW * XQ, n_q));
    if (s_begin >= s_end_g) return;  // no row of the workgroup reads this chunk's counts
    const int r0 = rg0 + w * XQ;
    const bool wave_on = r0 < n_q;
    // this wave's candidates end before s_end (none: the wave only stages)
    const int s_end = wave_on ? min(min(s_begin + XKC, n_kv), q_offset + min(r0 + XQ, n_q)) : s_begin;
    const int t_min = q_offset + r0;  // first query position of the wave

    const int r = r0 + col;
    const bool r_ok = r < n_q;
    const int t = q_offset + r;
    const uint32_t lo_r = r_ok ? lo[r] : 0u;
    const float lo_f = key_float(lo_r);
    // B operand: the lane's query, dims 16c + 8hh .. + 7 (zero past d), and |q|
    bf16x8 qop[NC];
    float qq = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (r_ok && 16 * c + 8 * hh < d) x = *reinterpret_cast<const u32x4*>(qi + (int64_t)r * d + 16 * c + 8 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = __uint_as_float(x[e] << 16), b = __uint_as_float(x[e] & 0xFFFF0000u);
            qq = __builtin_fmaf(a, a, qq);
            qq = __builtin_fmaf(b, b, qq);
        }
        qop[c] = __builtin_bit_cast(bf16x8, x);
    }
    qq += __shfl_xor(qq, 32);
    const float cq = 4.04f * (float)d * 0x1p-24f * sqrtf(qq);
    const float cabs = (float)d * 0x1p-125f;

    const int64_t region = (int64_t)(r_ok ? r : 0) * nchunk + blockIdx.x;
    uint32_t* kdst = ckept + region * SCAP;
    uint32_t cnt = 0;
    // staging: thread chunk it = tid + 256 i is row it / CPR, 16-byte chunk it % CPR
    u32x4 stg[SPT];
    auto fetch = [&](int s0) {
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int it = tid + 64 * XW * i;
            const int row = it / CPR, ch = it % CPR;
            stg[i] = u32x4{0u, 0u, 0u, 0u};
            if (it < XT * CPR && 8 * ch < d) {
                const int64_t key = min(s0 + row, n_kv - 1);
                stg[i] = *reinterpret_cast<const u32x4*>(ki + key * d + 8 * ch);
            }
        }
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int it = tid + 64 * XW * i;
            if (it < XT * CPR) *reinterpret_cast<u32x4*>(&kt[buf][(it / CPR) * KRS + 8 * (it % CPR)]) = stg[i];
        }
    };
    fetch(s_begin);
    put(0);
    __syncthreads();
    int buf = 0;
    for (int s0 = s_begin; s0 < s_end_g; s0 += XT, buf ^= 1) {
        const bool more = s0 + XT < s_end_g;
        if (more) fetch(s0 + XT);
        if (s0 < s_end) {
            f32x16 acc[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
                const uint16_t* kr = &kt[buf][(32 * b + col) * KRS + 8 * hh];
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * c)), qop[c], acc[b], 0,
                        0, 0);
            }
            // lo_f minus the bound, widened by |lo_f| 2^-22 so that the rounding
            // of the subtraction cannot raise the threshold; NaN (non-finite
            // norms) keeps everything
            const float thr = lo_f - (cq * tnorm[s0 / XT] + cabs + fabsf(lo_f) * 0x1p-22f);
            // bit e = 16b + i: the key s0 + 32b + 8(i/4) + 4hh + i%4 is kept
            uint32_t keep = 0;
#pragma unroll
            for (int e = 0; e < 32; ++e) keep |= (!(acc[e >> 4][e & 15] < thr) ? 1u : 0u) << e;
            if (s0 + XT - 1 > min(t_min, n_kv - 1)) {  // a tile past some row's last candidate
                uint32_t ok = 0;
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const int sk = s0 + 32 * (e >> 4) + 8 * ((e >> 2) & 3) + 4 * hh + (e & 3);
                    ok |= (sk <= t && sk < n_kv ? 1u : 0u) << e;
                }
                keep &= ok;
            }
            if (lo_r == 0u) keep = 0;  // row selected directly (or not a row)
            // kept scores by group of four (static register indices; one select
            // among four per kept score), in position order
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                uint32_t m = (keep >> (4 * g)) & 0xFu;
                const float x0 = acc[g >> 2][4 * (g & 3)], x1 = acc[g >> 2][4 * (g & 3) + 1];
                const float x2 = acc[g >> 2][4 * (g & 3) + 2], x3 = acc[g >> 2][4 * (g & 3) + 3];
                while (m) {
                    const int i = __builtin_ctz(m);
                    m &= m - 1u;
                    if (cnt < (uint32_t)SCAP) {
                        const int slot = hh ? SCAP - 1 - (int)cnt : (int)cnt;
                        const float x = i == 0 ? x0 : (i == 1 ? x1 : (i == 2 ? x2 : x3));
                        const uint32_t p = (uint32_t)(s0 - s_begin + 32 * (g >> 2) + 8 * (g & 3) + 4 * hh + i);
                        kdst[slot] = (__float_as_uint(x) & 0xFFFFFE00u) | p;  // p < 512
                    }
                    ++cnt;
                }
            }
        }
        if (more) put(buf ^ 1);
        __syncthreads();
    }
    if (r_ok && s_begin < s_end) ccnt[region * 2 + hh] = cnt;
}

// The indexer's float32 chain for one (query, key): fused multiply-adds in
// dimension order from zero (the same bits as the matrix-core chain).
__device__ __forceinline__ float chain_score(const float* __restrict__ qf, const uint16_t* __restrict__ kr, int d)
{
    float acc = 0.f;
    for (int i = 0; i < d; i += 8) {
        const u32x4 kw = *reinterpret_cast<const u32x4*>(kr + i);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            acc = __builtin_fmaf(qf[i + 2 * x], __uint_as_float(kw[x] << 16), acc);
            acc = __builtin_fmaf(qf[i + 2 * x + 1], __uint_as_float(kw[x] & 0xFFFF0000u), acc);
        }
    }
    return acc;
}

// The caps keep the select's LDS within a quarter of a CU's 160 KB, so that
// four rows run per CU.  A row past either cap takes the direct path.
constexpr int SKC = 5120;   // kept candidates a row may carry into the select
constexpr int SAMB = 256;   // candidates a row may leave ambiguous
constexpr int SREG = KMAXN / XKC;  // regions of a row at most
static_assert(SKC >= 4096, "the kept words stage the output of up to 4096 indices");
static_assert(2 * SREG == KTH, "two threads per region in the classification");
constexpr int SMALL = 256;  // keys in the rank's histogram bin that are ranked directly

struct __attribute__((aligned(16))) SelectLds {
    uint32_t sel[KWORDS];     // bit p: candidate p is selected
    uint32_t hist[KBINS];     // digit histogram; the keys of the rank's bin; tie bitmap
    uint32_t kw[SKC];         // kept words, region after region; output staging
    uint32_t amb[SAMB];       // chain keys of the ambiguous candidates
    uint16_t apos[SAMB];      // their positions
    uint32_t rfirst[SREG];    // where each region's kept words start in kw
    uint32_t rcount[SREG];    // and how many there are
    uint32_t rc0[SREG];       // how many of them fill the region from its start
    uint32_t wsum[KWAVES];
    uint32_t wmax[KWAVES];
    uint32_t state[4];
};

// The T-th largest of the keys that each(f) hands to f and how many keys
// equal to it rank within the first T (`width` significant bits): one
// histogram pass, then the rank's bin ranked directly when it is small, else
// the radix passes.
template <class Each>
__device__ void select_rank(SelectLds& L, Each&& each, uint32_t width, uint32_t rank, uint32_t& T, uint32_t& rem_out)
{
    const int tid = threadIdx.x;
    const uint32_t nb = min(11u, width), shift = width - nb;
    zero_words(L.hist, KBINS);
    __syncthreads();
    each([&](uint32_t v) { atomicAdd(&L.hist[v >> shift], 1u); });
    __syncthreads();
    find_digits(L, rank, 0u);
    const uint32_t bin = L.state[0], rem = L.state[1];
    const uint32_t m = L.hist[bin];
    __syncthreads();
    if (m <= (uint32_t)SMALL && shift > 0u) {
        uint32_t* bk = L.hist;
        if (tid == 0) L.state[2] = 0u;
        __syncthreads();
        each([&](uint32_t v) {
            if ((v >> shift) == bin) bk[atomicAdd(&L.state[2], 1u)] = v;
        });
        __syncthreads();
        if ((uint32_t)tid < m) {
            const uint32_t x = bk[tid];
            uint32_t gt = 0, ge = 0;
            for (uint32_t j = 0; j < m; ++j) {
                const uint32_t y = bk[j];
                gt += y > x ? 1u : 0u;
                ge += y >= x ? 1u : 0u;
            }
            if (gt < rem && rem <= ge) {  // x is the key (every thread holding it writes the same)
                L.state[0] = x;
                L.state[1] = rem - gt;
            }
        }
        __syncthreads();
        T = L.state[0];
        rem_out = L.state[1];
        __syncthreads();
    } else {
        radix_select(L, each, width, rank, T, rem_out);
    }
}

// Exact top-k of row r straight from the scores, for the rows the bracket
// cannot settle: the scores are recomputed with the indexer's float32 chain
// (vector FMA in dimension order, the same bits) at each pass of an exact
// selection over the whole row.  Called by every thread of the workgroup;
// qf holds d floats and stage k words of LDS, both apart from L's fields.
template <class Lds>
__device__ void select_direct(Lds& L, float* qf, uint32_t* stage, const uint16_t* __restrict__ qi,
                              const uint16_t* __restrict__ ki, int r, int n_cand, int d, int k,
                              int32_t* __restrict__ out)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    __syncthreads();  // the caller's last reads of L are done
    for (int i = tid; i < d; i += KTH) qf[i] = __uint_as_float((uint32_t)qi[(int64_t)r * d + i] << 16);
    __syncthreads();
    auto score_key = [&](int p) { return order_key(chain_score(qf, ki + (int64_t)p * d, d)); };
    auto all = [&](auto&& f) {
        for (int p = tid; p < n_cand; p += KTH) f(score_key(p));
    };
    uint32_t T, need_eq;
    radix_select(L, all, 32u, (uint32_t)k, T, need_eq);
    uint32_t* tie = L.hist;
    // every bitmap word is written once: 64 positions per wave step
    for (int p0 = 0; p0 < KMAXN; p0 += KTH) {
        const int p = p0 + tid;
        const bool valid = p < n_cand;
        const uint32_t u = valid ? score_key(p) : 0u;
        const uint64_t g = __ballot(valid && u > T);
        const uint64_t e = __ballot(valid && u == T);
        if (lane == 0) {
            const int wd = (p0 + 64 * w) >> 5;
            L.sel[wd] = (uint32_t)g;
            L.sel[wd + 1] = (uint32_t)(g >> 32);
            tie[wd] = (uint32_t)e;
            tie[wd + 1] = (uint32_t)(e >> 32);
        }
    }
    __syncthreads();
    emit_ascending(L, L.sel, tie, need_eq, k, stage, out);
}

// Exact top-k of row r from its kept candidates.  Each chain score c lies
// within a bound b of its approximate score a (the filter's bound, widened
// for the rounding of a +- b), and every b of the row is at most bmax, so the
// k-th largest chain score lies within bmax of A_k, the k-th largest
// approximate score.  A candidate with a - b above that interval is in the
// top-k, one with a + b below it is not, and only the rest -- the few near
// the k-th score -- are scored on the chain and ranked exactly (ties by
// position).  If the interval lies at or above LO, at least k candidates
// reach LO, so every candidate the filter dropped ranks below the top-k.  A
// row that cannot be settled this way (threshold 0, a region overflowed,
// more than SKC kept or SAMB ambiguous, fewer than k kept, the interval
// below LO, a non-finite score or bound) is selected by select_direct.
__global__ void __launch_bounds__(KTH)
stream_select_kernel(const uint16_t* __restrict__ qi, const uint16_t* __restrict__ ki, int32_t n_kv, int32_t d,
                     int32_t q_offset, int32_t k, uint32_t* __restrict__ lo, int32_t nchunk,
                     const uint32_t* __restrict__ ccnt, const float* __restrict__ tnorm,
                     const uint32_t* __restrict__ ckept, int32_t* __restrict__ idx_out)
{
    __shared__ SelectLds L;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int64_t t = (int64_t)q_offset + r;
    const int n_cand = (int)min((int64_t)n_kv, t + 1);
    int32_t* out = idx_out + (int64_t)r * k;
    if (n_cand <= k) {
        for (int e = tid; e < k; e += KTH) out[e] = e < n_cand ? e : -1;
        return;
    }
    const uint32_t lo_r = lo[r];
    // thread tid owns region tid, the row's 512-key chunk tid
    const int n_reg = (n_cand + XKC - 1) / XKC;  // <= KTH
    const bool mine = lo_r != 0u && tid < n_reg;
    const int64_t reg = (int64_t)r * nchunk + tid;
    uint32_t c0 = 0, c1 = 0;
    if (mine) {
        c0 = ccnt[2 * reg];
        c1 = ccnt[2 * reg + 1];
    }
    const bool ovf = __syncthreads_or(c0 + c1 > (uint32_t)SCAP) != 0;
    uint32_t total;
    const uint32_t before = block_excl_scan(ovf ? 0u : c0 + c1, L.wsum, &total);
    // the direct way: q staged past the k output words the staging needs
    auto direct = [&]() {
        select_direct(L, reinterpret_cast<float*>(L.kw + 4096), L.kw, qi, ki, r, n_cand, d, k, out);
    };
    static_assert(SKC >= 4096 + 256, "q (d <= 256) staged past the output staging");
    if (lo_r == 0u || ovf || total < (uint32_t)k) return direct();
    // ---- kept (score, position) to LDS: the first c0 and the last c1 slots of
    // each region; the region's tile norms; and, folded into one block
    // reduction, the largest tile norm, the largest |score|, the smallest and
    // largest score keys, |q|^2 and whether any score is not finite ----
    uint32_t tmax = 0, amax = 0, kmin_n = 0, kmax = 0;  // kmin_n = ~(smallest key)
    uint32_t bad = 0;
    float qq = 0.f;
    // The row's regions lie one after another in memory, in 16-byte pieces.
    constexpr int PPR = SCAP / 4;                        // pieces per region
    constexpr int PPT = (SREG * PPR + KTH - 1) / KTH;    // pieces per thread at most
    const int npieces = n_reg * PPR;
    const u32x4* rowk = reinterpret_cast<const u32x4*>(ckept + (int64_t)r * nchunk * SCAP);
    auto take = [&](uint32_t v) {  // a word into the reductions
        const float a = __uint_as_float(v & 0xFFFFFE00u);
        bad |= !(fabsf(a) <= 1.0e38f) ? 1u : 0u;
        amax = max(amax, __float_as_uint(fabsf(a)));
        const uint32_t key = order_key(a);
        kmin_n = max(kmin_n, ~key);
        kmax = max(kmax, key);
    };
    const bool trim = total > (uint32_t)SKC;
    u32x4 kw[PPT];
    if (!trim) {
        // every thread takes pieces (coalesced), loaded before the region
        // table is known
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int pc = tid + KTH * i;
            kw[i] = pc < npieces ? rowk[pc] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (mine) {
        // the region's eight tile norms (tiles past n_kv read as tile 0's)
        constexpr int TPR = XKC / XT;
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
            const int tl = tid * TPR + i;
            tmax = max(tmax, __float_as_uint(tnorm[tl * XT < n_kv ? tl : 0]));  // >= 0 (NaN: the largest bits)
        }
        L.rfirst[tid] = before;
        L.rc0[tid] = c0;
        L.rcount[tid] = c0 + c1;
    }
    __syncthreads();
    // kept words of a region: slots [0, c0) and [SCAP - c1, SCAP)
    auto kept_slot = [&](int g, uint32_t j, uint32_t& rank) {
        const uint32_t c0g = L.rc0[g];
        const uint32_t tail0 = (uint32_t)SCAP - (L.rcount[g] - c0g);  // first of the last c1 slots
        rank = j < c0g ? j : c0g + (j - tail0);
        return j < c0g || j >= tail0;
    };
    uint32_t xkey = 0u;  // a trimmed row keeps the words whose key is at least xkey
    if (!trim) {
        // slot j goes to first + its rank among the region's kept words
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int pc = tid + KTH * i;
            if (pc < npieces) {
                const int g = pc / PPR, j0 = 4 * (pc % PPR);
                const uint32_t first = L.rfirst[g];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    uint32_t rank;
                    if (kept_slot(g, (uint32_t)(j0 + x), rank)) {
                        L.kw[first + rank] = kw[i][x];
                        take(kw[i][x]);
                    }
                }
            }
        }
    } else {
        // More kept words than LDS holds (rare: about one row in several
        // thousand at the DSA prefill shape): keep those whose key is at least
        // the (SKC - 256)-th largest, read from memory at every pass.  The
        // words left out are shown to rank below the top-k once the bracket
        // of the k-th score is known, else the row takes the direct way.
        auto each_kept = [&](auto&& f) {
            for (int pc = tid; pc < npieces; pc += KTH) {
                const int g = pc / PPR, j0 = 4 * (pc % PPR);
                const u32x4 v4 = rowk[pc];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    uint32_t rank;
                    if (kept_slot(g, (uint32_t)(j0 + x), rank)) f(order_key(__uint_as_float(v4[x] & 0xFFFFFE00u)));
                }
            }
        };
        uint32_t gmin_n = 0, gmax = 0;
        each_kept([&](uint32_t key) {
            gmin_n = max(gmin_n, ~key);
            gmax = max(gmax, key);
        });
        gmin_n = block_max(gmin_n, L.wmax);
        gmax = block_max(gmax, L.wmax);
        const uint32_t gmin = ~gmin_n, gspan = gmax - gmin;
        const uint32_t gwidth = gspan == 0u ? 0u : 32u - (uint32_t)__clz(gspan);
        uint32_t xrel, xrem;
        select_rank(L, [&](auto&& f) { each_kept([&](uint32_t key) { f(key - gmin); }); }, gwidth,
                    (uint32_t)(SKC - 256), xrel, xrem);
        xkey = xrel + gmin;
        // the region owners count and place their words at or above xkey,
        // reading the region twice in 16-byte pieces
        auto region_pass = [&](auto&& f) {
#pragma unroll 1
            for (int i = 0; i < PPR; ++i) {
                const u32x4 v4 = rowk[tid * PPR + i];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    uint32_t rank;
                    const uint32_t v = v4[x];
                    if (kept_slot(tid, (uint32_t)(4 * i + x), rank) &&
                        order_key(__uint_as_float(v & 0xFFFFFE00u)) >= xkey)
                        f(v);
                }
            }
        };
        uint32_t nk = 0;
        if (mine) region_pass([&](uint32_t) { ++nk; });
        uint32_t total2;
        const uint32_t first = block_excl_scan(nk, L.wsum, &total2);
        if (total2 > (uint32_t)SKC) return direct();  // ties at xkey
        if (mine) {
            uint32_t n = first;
            region_pass([&](uint32_t v) {
                L.kw[n++] = v;
                take(v);
            });
        }
        __syncthreads();  // every thread has read rc0 / rcount of the untrimmed regions
        if (mine) {
            L.rfirst[tid] = first;
            L.rcount[tid] = nk;
        }
        total = total2;
    }
    for (int i = tid; i < d; i += KTH) {
        const float x = __uint_as_float((uint32_t)qi[(int64_t)r * d + i] << 16);
        qq = __builtin_fmaf(x, x, qq);
    }
    {
        const int lane = tid & 63, w = tid >> 6;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            tmax = max(tmax, (uint32_t)__shfl_xor(tmax, off));
            amax = max(amax, (uint32_t)__shfl_xor(amax, off));
            kmin_n = max(kmin_n, (uint32_t)__shfl_xor(kmin_n, off));
            kmax = max(kmax, (uint32_t)__shfl_xor(kmax, off));
            bad |= (uint32_t)__shfl_xor(bad, off);
            qq += __shfl_xor(qq, off);
        }
        uint32_t* red = L.hist;  // [6][KWAVES]
        if (lane == 0) {
            red[0 * KWAVES + w] = tmax;
            red[1 * KWAVES + w] = amax;
            red[2 * KWAVES + w] = kmin_n;
            red[3 * KWAVES + w] = kmax;
            red[4 * KWAVES + w] = bad;
            red[5 * KWAVES + w] = __float_as_uint(qq);
        }
        __syncthreads();  // also publishes L.kw, L.rfirst, L.rcount
        tmax = amax = kmin_n = kmax = bad = 0;
        qq = 0.f;
#pragma unroll
        for (int i = 0; i < KWAVES; ++i) {
            tmax = max(tmax, red[i]);
            amax = max(amax, red[KWAVES + i]);
            kmin_n = max(kmin_n, red[2 * KWAVES + i]);
            kmax = max(kmax, red[3 * KWAVES + i]);
            bad |= red[4 * KWAVES + i];
            qq += __uint_as_float(red[5 * KWAVES + i]);
        }
        __syncthreads();
    }
    if (bad) return direct();
    const float cq = 4.04f * (float)d * 0x1p-24f * sqrtf(qq);
    const float cabs = (float)d * 0x1p-125f;
    // chain score c_j within b_j of the stored a_j: the filter's bound, plus
    // the 9 mantissa bits the filter dropped (less than 2^-14 |a_j| for a
    // normal value, 2^-140 below; 2^-12 |a_j| + 2^-126 covers it), widened for
    // the rounding of a_j +- b_j; bmax bounds every b_j of the row
    auto bound = [&](float a_signed, float tn) {
        const float a = fabsf(a_signed);
        const float b = cq * tn + cabs + a * 0x1p-12f + 0x1p-126f;
        return b + (a + b) * 0x1p-21f;
    };
    float bmax = cq * __uint_as_float(tmax) + cabs + __uint_as_float(amax) * 0x1p-12f + 0x1p-126f;
    bmax += (__uint_as_float(amax) + bmax) * 0x1p-21f;
    if (!(bmax <= 1.0e30f)) return direct();  // non-finite norms: the direct way
    // ---- A_k, the k-th largest approximate score (keys relative to the row's
    // smallest kept key, only the bits their range needs) ----
    const uint32_t kmin = ~kmin_n;
    const uint32_t span = kmax - kmin;
    const uint32_t width = span == 0u ? 0u : 32u - (uint32_t)__clz(span);
    auto each_a = [&](auto&& f) {
        for (uint32_t j = tid; j < total; j += KTH) f(order_key(__uint_as_float(L.kw[j] & 0xFFFFFE00u)) - kmin);
    };
    uint32_t akr, rem;
    select_rank(L, each_a, width, (uint32_t)k, akr, rem);
    const float ak = key_float(akr + kmin);
    // the k-th largest chain score lies within bmax of A_k: [lo_e, hi_e]
    const float marg = bmax + (fabsf(ak) + bmax) * 0x1p-21f;
    const float hi_e = ak + marg, lo_e = ak - marg;
    if (!(lo_e >= key_float(lo_r))) return direct();  // fewer than k provably reach LO
    if (xkey != 0u) {
        // a word left out has a stored score below xf, so a chain score below
        // xf + bmax: that must lie at or below the bracket of the k-th
        const float xf = key_float(xkey);
        const float xe = xf + bmax + (fabsf(xf) + bmax) * 0x1p-21f;
        if (!(xe <= lo_e)) return direct();
    }
    // ---- sure-in to the bitmap; the ambiguous ones scored on the chain ----
    __syncthreads();  // every thread has read the rank out of L.state / L.hist
    zero_words(L.sel, KWORDS);
    if (tid == 0) L.state[2] = 0u;
    for (int i = tid; i < d; i += KTH) reinterpret_cast<float*>(L.hist)[i] = __uint_as_float((uint32_t)qi[(int64_t)r * d + i] << 16);
    __syncthreads();
    // two threads per region, alternate words; the region's tile norms in
    // registers
    uint32_t n_in = 0;
    bool full = false;
    const int g = tid % SREG, half = tid / SREG;
    if (g < n_reg) {
        constexpr int TPR = XKC / XT;
        float tnr[TPR];
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
            const int tl = g * TPR + i;
            tnr[i] = tnorm[tl * XT < n_kv ? tl : 0];
        }
        const uint32_t first = L.rfirst[g], cnt = L.rcount[g];
        const uint32_t pbase = (uint32_t)g * XKC;
    for (uint32_t i = half; i < cnt; i += 2) {
        const uint32_t v = L.kw[first + i];
        const float a = __uint_as_float(v & 0xFFFFFE00u);
        const uint32_t pl = v & 0x1FFu;
        float tn = tnr[0];
#pragma unroll
        for (int x = 1; x < TPR; ++x) tn = (pl >> 6) == (uint32_t)x ? tnr[x] : tn;
        const float b = bound(a, tn);
        const uint32_t p = pbase + pl;
        if (a - b > hi_e) {
            atomicOr(&L.sel[p >> 5], 1u << (p & 31));
            ++n_in;
        } else if (!(a + b < lo_e)) {
            const uint32_t slot = atomicAdd(&L.state[2], 1u);
            if (slot < (uint32_t)SAMB) L.apos[slot] = (uint16_t)p;
            else full = true;
        }
    }
    }
    uint32_t n_in_all;
    block_excl_scan(n_in, L.wsum, &n_in_all);
    if (__syncthreads_or(full)) return direct();
    const uint32_t n_amb = L.state[2];
    // the ambiguous ones on the chain, all at once (one key row per thread):
    // scored inside the loop above, a wave would wait for a row's load at
    // every trip that meets one
    static_assert(SAMB <= KTH, "one ambiguous candidate per thread");
    if ((uint32_t)tid < n_amb)
        L.amb[tid] = order_key(chain_score(reinterpret_cast<const float*>(L.hist), ki + (int64_t)L.apos[tid] * d, d));
    __syncthreads();
    const uint32_t k2 = (uint32_t)k - n_in_all;  // >= 1: sure-in scores exceed the k-th
    // ---- the k2-th largest chain key among the ambiguous ones ----
    auto each_amb = [&](auto&& f) {
        for (uint32_t j = tid; j < n_amb; j += KTH) f(L.amb[j]);
    };
    uint32_t T, need_eq;
    select_rank(L, each_amb, 32u, k2, T, need_eq);
    uint32_t* tie = L.hist;
    zero_words(tie, KWORDS);
    __syncthreads();
    for (uint32_t j = tid; j < n_amb; j += KTH) {
        const uint32_t u = L.amb[j], p = L.apos[j];
        if (u > T) atomicOr(&L.sel[p >> 5], 1u << (p & 31));
        else if (u == T) atomicOr(&tie[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    emit_ascending(L, L.sel, tie, need_eq, k, L.kw, out);
}

}  // namespace

hipError_t launch_indexer_scores(const uint16_t* q_idx, const uint16_t* k_idx, int32_t n_q,
                                 int32_t n_kv, int32_t d_idx, int32_t q_offset, float* scores,
                                 hipStream_t stream)
{
    dim3 grid((n_kv + XKC - 1) / XKC, (n_q + XQ * XW - 1) / (XQ * XW));
    hipLaunchKernelGGL(indexer_kernel, grid, dim3(64 * XW), 0, stream, q_idx, k_idx, n_q, n_kv, d_idx,
                       q_offset, scores);
    return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int32_t n_q, int32_t n_kv, int32_t q_offset,
                       int32_t topk, int32_t* idx_out, hipStream_t stream)
{
    if ((n_kv & 3) == 0)
        hipLaunchKernelGGL(topk_kernel<true>, dim3(n_q), dim3(KTH), 0, stream, scores, n_q, n_kv, q_offset,
                           topk, idx_out);
    else
        hipLaunchKernelGGL(topk_kernel<false>, dim3(n_q), dim3(KTH), 0, stream, scores, n_q, n_kv, q_offset,
                           topk, idx_out);
    return hipGetLastError();
}

}  // namespace sa

namespace sa {

hipError_t launch_indexer_topk_stream(const uint16_t* q_idx, const uint16_t* k_idx, int32_t n_q, int32_t n_kv,
                                      int32_t d_idx, int32_t q_offset, int32_t topk, int32_t* idx_out,
                                      uint8_t* ws, const StreamTopkLayout& L, hipStream_t stream)
{
    uint32_t* samp = reinterpret_cast<uint32_t*>(ws + L.samp);
    uint32_t* lo = reinterpret_cast<uint32_t*>(ws + L.lo);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
    float* tnorm = reinterpret_cast<float*>(ws + L.tnorm);
    uint32_t* kept = reinterpret_cast<uint32_t*>(ws + L.kept);
    const unsigned qgroups = (unsigned)((n_q + XQ * XW - 1) / (XQ * XW));
    hipLaunchKernelGGL(stream_sample_kernel, dim3((unsigned)(L.s_max / XT), qgroups), dim3(64 * XW), 0, stream, q_idx,
                       k_idx, n_q, n_kv, d_idx, q_offset, samp, L.s_max);
    const int nnorm = (L.ntile + 3) / 4;
    hipLaunchKernelGGL(stream_bracket_kernel, dim3((unsigned)(nnorm + n_q)), dim3(KTH), 0, stream, samp, L.s_max, n_kv,
                       q_offset, topk, lo, k_idx, d_idx, L.ntile, nnorm, tnorm);
    const dim3 fgrid((unsigned)L.nchunk, qgroups);
    if (d_idx <= 64)
        hipLaunchKernelGGL(stream_filter_kernel<4>, fgrid, dim3(64 * XW), 0, stream, q_idx, k_idx, n_q, n_kv, d_idx,
                           q_offset, lo, tnorm, L.nchunk, cnt, kept);
    else if (d_idx <= 128)
        hipLaunchKernelGGL(stream_filter_kernel<8>, fgrid, dim3(64 * XW), 0, stream, q_idx, k_idx, n_q, n_kv, d_idx,
                           q_offset, lo, tnorm, L.nchunk, cnt, kept);
    else
        hipLaunchKernelGGL(stream_filter_kernel<16>, fgrid, dim3(64 * XW), 0, stream, q_idx, k_idx, n_q, n_kv, d_idx,
                           q_offset, lo, tnorm, L.nchunk, cnt, kept);
    hipLaunchKernelGGL(stream_select_kernel, dim3((unsigned)n_q), dim3(KTH), 0, stream, q_idx, k_idx, n_kv, d_idx,
                       q_offset, topk, lo, L.nchunk, cnt, tnorm, kept, idx_out);
    return hipGetLastError();
}

}  // namespace sa

namespace sa {
namespace {

// Scratch of sa_indexer_topk_noalloc, for callers that cannot allocate: one
// copy of this array per device, held until the process ends.  In host code
// the name is a stand-in, not a device address: launches take the address
// that noalloc_scratch looks up per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t noalloc_scratch(uint8_t** ptr)
{
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = static_cast<uint8_t*>(addr[dev]);
    return hipSuccess;
}

}  // namespace sa
