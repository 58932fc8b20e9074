// indexer_topk.hip -- indexer scores and per-query top-k selection.
//
// "Sparse Attention" glossary, section on common sparsity patterns: DeepSeek
// Sparse Attention runs a small indexer that scores every earlier token for
// each query, then attends only to the 2,048 best-scored tokens.  The pages
// give no indexer formula; the score used here is the plain dot product of
// the indexer query and key, accumulated in float32 as one fused
// multiply-add chain in dimension order (a fixed order makes the selection
// reproducible bit for bit).  Ties in the selection go to the lower index.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------------------
// Indexer: tile of 64 queries x 128 keys per workgroup, 256 threads, each
// thread a 4 x 8 register tile.  Operands are staged in LDS as float32,
// dimension-major, 64 dimensions at a time; every accumulator runs its own
// sequential fma chain over the dimensions, so the result does not depend on
// the tiling.
constexpr int IQ = 64, IS = 128, ID = 64, ITH = 256;

__global__ void __launch_bounds__(ITH)
indexer_kernel(const uint16_t* __restrict__ qi, const uint16_t* __restrict__ ki, int32_t n_q,
               int32_t n_kv, int32_t d, int32_t q_offset, float* __restrict__ scores)
{
    __shared__ __attribute__((aligned(16))) float qs[ID][IQ];
    __shared__ __attribute__((aligned(16))) float ks[ID][IS];
    const int s0 = blockIdx.x * IS;
    const int r0 = blockIdx.y * IQ;
    const int t_hi = q_offset + min(r0 + IQ, n_q) - 1;  // last query position of the tile
    if (s0 > t_hi) return;                                // no candidate in this tile
    const int tid = threadIdx.x;
    const int tq = tid >> 4, ts = tid & 15;              // 16 x 16 thread grid

    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    for (int c0 = 0; c0 < d; c0 += ID) {
        const int dc = min(ID, d - c0);
        __syncthreads();
        // stage q: 64 rows x dc dims; 8 dims per 16-byte load
        for (int u = tid; u < IQ * (ID / 8); u += ITH) {
            const int r = u / (ID / 8), c8 = (u % (ID / 8)) * 8;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (r0 + r < n_q && c8 < dc)
                w = *reinterpret_cast<const u32x4*>(qi + (int64_t)(r0 + r) * d + c0 + c8);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                qs[c8 + 2 * x][r] = __uint_as_float(w[x] << 16);
                qs[c8 + 2 * x + 1][r] = __uint_as_float(w[x] & 0xFFFF0000u);
            }
        }
        for (int u = tid; u < IS * (ID / 8); u += ITH) {
            const int r = u / (ID / 8), c8 = (u % (ID / 8)) * 8;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (s0 + r < n_kv && c8 < dc)
                w = *reinterpret_cast<const u32x4*>(ki + (int64_t)(s0 + r) * d + c0 + c8);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                ks[c8 + 2 * x][r] = __uint_as_float(w[x] << 16);
                ks[c8 + 2 * x + 1][r] = __uint_as_float(w[x] & 0xFFFF0000u);
            }
        }
        __syncthreads();
        for (int c = 0; c < dc; ++c) {
            const float4 qa = *reinterpret_cast<const float4*>(&qs[c][tq * 4]);
            const float4 k0 = *reinterpret_cast<const float4*>(&ks[c][ts * 8]);
            const float4 k1 = *reinterpret_cast<const float4*>(&ks[c][ts * 8 + 4]);
            const float qv[4] = {qa.x, qa.y, qa.z, qa.w};
            const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(qv[i], kv[j], acc[i][j]);
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = r0 + tq * 4 + i;
        if (r >= n_q) continue;
        const int t = q_offset + r;
        const int s = s0 + ts * 8;
        float* dst = scores + (int64_t)r * n_kv + s;
        if (s + 7 <= t && s + 7 < n_kv && (n_kv & 3) == 0) {
            *reinterpret_cast<float4*>(dst) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s + j <= t && s + j < n_kv) dst[j] = acc[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Top-k: one workgroup of 1024 threads per query row; the row's candidates
// (at most 65,536) stay in registers, 64 per thread, as order-preserving
// 32-bit keys.  Four most-significant-digit-first radix passes with 256-bin
// LDS histograms find the key T of the k-th largest candidate and how many
// candidates equal to T must be taken; a flag per candidate then lets each
// thread emit a contiguous index range in ascending order after one scan.
constexpr int KTH = 1024;
constexpr int KPER = 64;           // candidates per thread
constexpr int KMAXN = KTH * KPER;  // 65,536

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;  // -0 ranks equal to +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of v over the workgroup (KTH threads); returns the inclusive
// prefix and writes the total to *total.
__device__ int block_scan_incl(int v, int* wsum, int* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        int s = lane < KTH / 64 ? wsum[lane] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(s, off, 64);
            if (lane >= off) s += y;
        }
        if (lane < KTH / 64) wsum[lane] = s;
    }
    __syncthreads();
    const int before = w > 0 ? wsum[w - 1] : 0;
    *total = wsum[KTH / 64 - 1];
    __syncthreads();
    return x + before;
}

__global__ void __launch_bounds__(KTH)
topk_kernel(const float* __restrict__ scores, int32_t n_q, int32_t n_kv, int32_t q_offset,
            int32_t k, int32_t* __restrict__ idx_out)
{
    __shared__ uint32_t hist[256];
    __shared__ int wsum[KTH / 64];
    __shared__ uint32_t sel_state[2];  // prefix, remaining k
    __shared__ __attribute__((aligned(16))) uint8_t flag[KMAXN];

    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t t = (int64_t)q_offset + r;
    const int n_cand = (int)min((int64_t)n_kv, t + 1);
    const float* row = scores + (int64_t)r * n_kv;
    int32_t* out = idx_out + (int64_t)r * k;

    if (n_cand <= k) {
        for (int e = tid; e < k; e += KTH) out[e] = e < n_cand ? e : -1;
        return;
    }

    // candidates: thread tid holds indices 4*tid + 4096*it + x (x < 4)
    uint32_t key[KPER];
#pragma unroll
    for (int it = 0; it < KPER / 4; ++it) {
        const int base = 4 * tid + 4096 * it;
        if (base + 3 < n_cand && (n_kv & 3) == 0) {
            const float4 f = *reinterpret_cast<const float4*>(row + base);
            key[4 * it + 0] = order_key(f.x);
            key[4 * it + 1] = order_key(f.y);
            key[4 * it + 2] = order_key(f.z);
            key[4 * it + 3] = order_key(f.w);
        } else {
#pragma unroll
            for (int x = 0; x < 4; ++x)
                key[4 * it + x] = base + x < n_cand ? order_key(row[base + x]) : 0u;
        }
    }

    if (tid == 0) {
        sel_state[0] = 0u;
        sel_state[1] = (uint32_t)k;
    }
    uint32_t prefix = 0;
    uint32_t remain = (uint32_t)k;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += KTH) hist[i] = 0;
        __syncthreads();
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
        for (int it = 0; it < KPER / 4; ++it)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int idx = 4 * tid + 4096 * it + x;
                const uint32_t kk = key[4 * it + x];
                if (idx < n_cand && (kk & hi_mask) == prefix)
                    atomicAdd(&hist[(kk >> shift) & 255u], 1u);
            }
        __syncthreads();
        // wave 0 finds the digit: bins scanned from the top
        if (tid < 64) {
            // lane owns bins 255-4*lane .. 252-4*lane (descending)
            uint32_t c4[4];
            uint32_t sum = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                c4[x] = hist[255 - 4 * lane - x];
                sum += c4[x];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            const uint32_t excl = incl - sum;
            if (excl < remain && remain <= incl) {
                uint32_t run = excl;
                for (int x = 0; x < 4; ++x) {
                    if (run + c4[x] >= remain) {
                        const uint32_t digit = 255u - 4u * lane - x;
                        sel_state[0] = prefix | (digit << shift);
                        sel_state[1] = remain - run;
                        break;
                    }
                    run += c4[x];
                }
            }
        }
        __syncthreads();
        prefix = sel_state[0];
        remain = sel_state[1];
        __syncthreads();
    }
    const uint32_t T = prefix;  // key of the k-th largest; take `remain` of the ties

    // flags: 1 = above T, 2 = equal to T, 0 = below / not a candidate
#pragma unroll
    for (int it = 0; it < KPER / 4; ++it) {
        const int base = 4 * tid + 4096 * it;
        if (base < KMAXN) {
            uint32_t w = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t kk = key[4 * it + x];
                const uint32_t f = (base + x < n_cand) ? (kk > T ? 1u : (kk == T ? 2u : 0u)) : 0u;
                w |= f << (8 * x);
            }
            *reinterpret_cast<uint32_t*>(flag + base) = w;
        }
    }
    __syncthreads();

    // each thread scans its contiguous 64 flags
    const int c0 = tid * KPER;
    int n_gt = 0, n_eq = 0;
    for (int e = 0; e < KPER; e += 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(flag + c0 + e);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t f = (w >> (8 * x)) & 255u;
            n_gt += f == 1u;
            n_eq += f == 2u;
        }
    }
    int tot;
    const int eq_incl = block_scan_incl(n_eq, wsum, &tot);
    int eq_rank = eq_incl - n_eq;
    // selected count of this thread
    int take_eq = (int)remain - eq_rank;
    take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
    const int mine = n_gt + take_eq;
    const int pos_incl = block_scan_incl(mine, wsum, &tot);
    int pos = pos_incl - mine;
    for (int e = 0; e < KPER; e += 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(flag + c0 + e);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const uint32_t f = (w >> (8 * x)) & 255u;
            bool take = f == 1u;
            if (f == 2u) {
                take = eq_rank < (int)remain;
                ++eq_rank;
            }
            if (take) {
                if (pos < k) out[pos] = c0 + e + x;
                ++pos;
            }
        }
    }
    (void)lane;
}

}  // namespace

hipError_t launch_indexer_scores(const uint16_t* q_idx, const uint16_t* k_idx, int32_t n_q,
                                 int32_t n_kv, int32_t d_idx, int32_t q_offset, float* scores,
                                 hipStream_t stream)
{
    dim3 grid((n_kv + IS - 1) / IS, (n_q + IQ - 1) / IQ);
    hipLaunchKernelGGL(indexer_kernel, grid, dim3(ITH), 0, stream, q_idx, k_idx, n_q, n_kv, d_idx,
                       q_offset, scores);
    return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int32_t n_q, int32_t n_kv, int32_t q_offset,
                       int32_t topk, int32_t* idx_out, hipStream_t stream)
{
    hipLaunchKernelGGL(topk_kernel, dim3(n_q), dim3(KTH), 0, stream, scores, n_q, n_kv, q_offset,
                       topk, idx_out);
    return hipGetLastError();
}

}  // namespace sa
