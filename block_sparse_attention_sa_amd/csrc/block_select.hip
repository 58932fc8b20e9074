// block_select.hip -- content-selected key blocks per (batch, head, query block).
//
// "Sparse Attention" glossary, section on common sparsity patterns: Native
// Sparse Attention selects the most relevant blocks of keys for each query
// block, and different heads may attend to different blocks (the
// sparse-transformer blog, section on combining templates, notes that
// different heads carry different patterns).  The pages give no scoring
// formula; the one used here:
//   * the mean query of the block and the mean key of each key block, fp64
//     sums in row order divided by the block size (rows past the end count
//     as zero; the block size is a power of two, so the division is exact);
//   * score = their dot product as an fp64 fused multiply-add chain;
//   * the block's own (diagonal) key blocks are always kept, plus the
//     n_select causally reachable key blocks of highest score (ties to the
//     lower block).
// Every operation has one fixed order, so the selection is reproducible bit
// for bit.  The lists then drive the unchanged block kernel with a causal
// element mask on the tiles that are not entirely causal.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int SEL_TH = 256;

// mean over the rows [blk*bs, blk*bs + bs) of one (b, h): one thread per
// column; stored [bh][blk][d], or [bh][d][blk] when TRANSPOSED (the key means,
// read one dimension at a time by lanes that hold consecutive blocks)
template <bool TRANSPOSED>
__global__ void pool_kernel(const uint16_t* __restrict__ x, int64_t sb, int64_t sh, int64_t sn, int32_t heads,
                            int32_t n, int32_t d, int32_t bs, int32_t nblk, double* __restrict__ mean)
{
    const int blk = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
    if (c >= d) return;
    const int b = bh / heads, h = bh % heads;
    const uint16_t* base = x + b * sb + h * sh + c;
    const int r0 = blk * bs, r1 = min(r0 + bs, n);
    // the sum runs in row order; the loads of 16 rows are issued ahead of it
    double acc = 0.0;
    int r = r0;
    for (; r + 16 <= r1; r += 16) {
        uint16_t x16[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x16[u] = base[(int64_t)(r + u) * sn];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += (double)__uint_as_float((uint32_t)x16[u] << 16);
    }
    for (; r < r1; ++r) acc += (double)__uint_as_float((uint32_t)base[(int64_t)r * sn] << 16);
    mean[TRANSPOSED ? ((int64_t)bh * d + c) * nblk + blk : ((int64_t)bh * nblk + blk) * d + c] = acc / bs;
}

__device__ __forceinline__ int64_t causal_pairs(int64_t p0, int64_t p1, int64_t s0, int64_t s1)
{
    // sum over query positions qp in [p0, p1] of the keys s in [s0, s1) with
    // s <= qp: the sum of clamp(x, 0, L) over x = qp + 1 - s0 in [a, b]
    const int64_t L = s1 - s0, a = p0 + 1 - s0, b = p1 + 1 - s0;
    const int64_t lo = max(a, (int64_t)0), hi = min(b, L);
    const int64_t ramp = lo <= hi ? (lo + hi) * (hi - lo + 1) / 2 : 0;
    const int64_t flat = max((int64_t)0, b - max(a, L + 1) + 1) * L;
    return ramp + flat;
}

__global__ void __launch_bounds__(SEL_TH)
select_kernel(const double* __restrict__ qm, const double* __restrict__ km, int32_t n_q, int32_t n_kv, int32_t d,
              int32_t q_offset, int32_t bq, int32_t bk, int32_t nqb, int32_t nkb, int32_t n_sel,
              int32_t* __restrict__ kv_count, int32_t* __restrict__ kv_index, uint8_t* __restrict__ kv_partial,
              unsigned long long* __restrict__ live_pairs)
{
    __shared__ double q_s[256];
    __shared__ double score[kSelectMaxBlocks];
    __shared__ uint8_t flag[kSelectMaxBlocks];  // 1 own, 2 reachable (a candidate), 0 neither
    __shared__ uint8_t keep_s[kSelectMaxBlocks];
    __shared__ int32_t wsum[SEL_TH / 64];
    __shared__ unsigned long long wpairs[SEL_TH / 64];
    const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int64_t item = (int64_t)bh * nqb + i;
    const int r0 = i * bq, r1 = min(r0 + bq, n_q);
    const int64_t p0 = (int64_t)q_offset + r0, p1 = (int64_t)q_offset + r1 - 1;
    for (int c = tid; c < d; c += SEL_TH) q_s[c] = qm[item * d + c];
    __syncthreads();
    for (int j = tid; j < nkb; j += SEL_TH) {
        const int64_t s0 = (int64_t)j * bk, s1 = min((int64_t)(j + 1) * bk, (int64_t)n_kv);
        const double* kj = km + (int64_t)bh * d * nkb + j;  // dimension c at kj[c * nkb]
        // the chain runs in dimension order; 16 loads are issued ahead of it
        double dot = 0.0;
        for (int c = 0; c < d; c += 16) {  // d is a multiple of 16
            double k16[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) k16[u] = kj[(int64_t)(c + u) * nkb];
#pragma unroll
            for (int u = 0; u < 16; ++u) dot = fma(q_s[c + u], k16[u], dot);
        }
        score[j] = dot;
        const bool own = s0 <= p1 && s1 - 1 >= p0;
        flag[j] = own ? 1 : (s0 <= p1 ? 2 : 0);
    }
    __syncthreads();
    // kept: own, or a candidate of rank below n_sel in the order (score
    // descending, block ascending); block j is ranked by thread j % SEL_TH
    for (int j = tid; j < nkb; j += SEL_TH) {
        uint8_t kp = flag[j] == 1 ? 1 : 0;
        if (flag[j] == 2) {
            const double sj = score[j];
            int rank = 0;
#pragma unroll 8
            for (int jj = 0; jj < nkb; ++jj)
                rank += (flag[jj] == 2 && (score[jj] > sj || (score[jj] == sj && jj < j))) ? 1 : 0;
            kp = rank < n_sel ? 1 : 0;
        }
        keep_s[j] = kp;
    }
    __syncthreads();
    // thread t owns blocks [4t, 4t + 4) for the list, which rises with j
    constexpr int PER = kSelectMaxBlocks / SEL_TH;
    bool keep[PER];
    int n_keep = 0;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int j = PER * tid + x;
        keep[x] = j < nkb && keep_s[j] != 0;
        n_keep += keep[x] ? 1 : 0;
    }
    // ascending positions in the list: a block scan of the counts
    int incl = n_keep;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int before = incl - n_keep, total = 0;
#pragma unroll
    for (int x = 0; x < SEL_TH / 64; ++x) {
        before += x < w ? wsum[x] : 0;
        total += wsum[x];
    }
    unsigned long long pairs = 0;
    int e = before;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int j = PER * tid + x;
        if (!keep[x]) continue;
        const int64_t s0 = (int64_t)j * bk, s1 = min((int64_t)(j + 1) * bk, (int64_t)n_kv);
        const int64_t cnt = causal_pairs(p0, p1, s0, s1);
        pairs += (unsigned long long)cnt;
        kv_index[item * nkb + e] = j;
        kv_partial[item * nkb + e] = cnt != (p1 - p0 + 1) * (s1 - s0) ? 1 : 0;
        ++e;
    }
    for (int x = total + tid; x < nkb; x += SEL_TH) {
        kv_index[item * nkb + x] = -1;
        kv_partial[item * nkb + x] = 0;
    }
    if (tid == 0) kv_count[item] = total;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pairs += __shfl_xor(pairs, off, 64);
    if (lane == 0) wpairs[w] = pairs;
    __syncthreads();
    if (tid == 0) {
        unsigned long long s = 0;
#pragma unroll
        for (int x = 0; x < SEL_TH / 64; ++x) s += wpairs[x];
        atomicAdd(live_pairs, s);
    }
}

}  // namespace

hipError_t launch_select_blocks(const SelectParams& p, hipStream_t stream)
{
    hipError_t e = launch_zero_i64(p.live_pairs, stream);
    if (e != hipSuccess) return e;
    const int bh = p.batch * p.heads;
    hipLaunchKernelGGL(pool_kernel<false>, dim3(p.nqb, bh), dim3(p.d), 0, stream, p.q, p.q_sb, p.q_sh, p.q_sn,
                       p.heads, p.n_q, p.d, p.bq, p.nqb, p.qm);
    hipLaunchKernelGGL(pool_kernel<true>, dim3(p.nkb, bh), dim3(p.d), 0, stream, p.k, p.k_sb, p.k_sh, p.k_sn,
                       p.heads, p.n_kv, p.d, p.bk, p.nkb, p.km);
    hipLaunchKernelGGL(select_kernel, dim3(p.nqb, bh), dim3(SEL_TH), 0, stream, p.qm, p.km, p.n_q, p.n_kv, p.d,
                       p.q_offset, p.bq, p.bk, p.nqb, p.nkb, p.n_sel, p.kv_count, p.kv_index, p.kv_partial,
                       (unsigned long long*)p.live_pairs);
    return hipGetLastError();
}

}  // namespace sa
