// block_mask.hip -- pattern -> per-query-block lists of live key blocks.
//
// "Sparse Attention" glossary, section on turning a pattern into savings:
// the mask is split into fixed blocks and blocks without any allowed pair
// are skipped; a block is live when it holds at least one allowed pair.
//
// Two kernels.
//   count:   one workgroup per (query block, group of key blocks).  A group
//            that no pattern term can reach (tested on the block's row and
//            key ranges) writes zero counts and exits.  Otherwise every
//            (row, 32-key chunk) pair of the group is evaluated as a 32-bit
//            allowed mask (each pattern term is an interval of keys for a
//            fixed query, or a short progression for the strided term), and
//            popcounts are summed per key block.  Counts go straight into
//            kv_index, which serves as the count array between the kernels;
//            each cell is owned by one workgroup, so no atomics or zeroing.
//   compact: one workgroup per query block turns the counts into the
//            ascending live list, the partial flags and the live count, and
//            adds the block's pairs to live_pairs (zeroed by the count kernel).
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupChunks = 16;  // 32-key chunks per count workgroup (at least one key block)

__device__ __host__ __forceinline__ int32_t group_chunks(int32_t bk)
{
    return bk / 32 > kGroupChunks ? bk / 32 : kGroupChunks;
}

__global__ void zero_i64(int64_t* p) { *p = 0; }

// Can any term allow a pair with q in [qa, qb] (absolute) and kv in [ka, kb]?
// Conservative: true may still mean no pair; false is exact.
__device__ bool group_reachable(const DevPattern& p, int64_t qa, int64_t qb, int64_t ka, int64_t kb)
{
    if (p.causal && ka > qb) return false;
    const int64_t kc = p.causal ? (kb < qb ? kb : qb) : kb;  // causal upper key bound
    if (kc < ka) return false;
    bool any = false;
    if (p.window_left >= 0) any |= (qa - p.window_left <= kc) && (qb + (int64_t)p.window_right >= ka);
    any |= ka < p.sinks;
    any |= qa < p.global_tokens || ka < p.global_tokens;
    if (p.stride > 0) any |= ka <= qb - p.stride_phase;
    if (p.unit > 0) {
        if (p.unit_window >= 0) {
            const int64_t ua = qa / p.unit - p.unit_window, ub = qb / p.unit + p.unit_window;
            any |= ua <= kc / p.unit && ub >= ka / p.unit;
        }
        if (p.n_rand > 0) any = true;  // table lookups are left to the exact count
    }
    return any;
}

// Thread layout: t = row_phase * G + chunk; each thread sums the popcounts of
// its chunk over the rows row_phase, row_phase + 256/G, ... of the block.
__global__ void __launch_bounds__(kThreads)
count_kernel(DevPattern p, int32_t n_q, int32_t n_kv, int32_t bq, int32_t bk, int32_t nkb,
             int32_t ngroups, int32_t* counts /* = kv_index */, int64_t* live_pairs)
{
    __shared__ int32_t cell[kGroupChunks];  // key blocks per group <= kGroupChunks
    const int i = blockIdx.x / ngroups;
    const int grp = blockIdx.x % ngroups;
    const int t = threadIdx.x;
    if (blockIdx.x == 0 && t == 0) *live_pairs = 0;

    const int32_t G = group_chunks(bk);
    const int32_t cpb = bk / 32;                 // chunks per key block
    const int32_t bpg = G / cpb;                 // key blocks per group
    const int32_t nchunks = (n_kv + 31) / 32;
    const int32_t j0 = grp * bpg, j1 = min(j0 + bpg, nkb);
    const int32_t c0 = j0 * cpb, c1 = min(j1 * cpb, nchunks);
    const int32_t q0 = i * bq, q1 = min(q0 + bq, n_q);
    int32_t* out = counts + (int64_t)i * nkb;

    if (t < j1 - j0) cell[t] = 0;
    const bool reach = group_reachable(p, (int64_t)q0 + p.q_offset, (int64_t)q1 - 1 + p.q_offset,
                                       (int64_t)c0 * 32, min((int64_t)c1 * 32, (int64_t)n_kv) - 1);
    __syncthreads();
    if (reach) {
        const int32_t ck = c0 + t % G;
        const int32_t rstep = kThreads / G;
        int32_t acc = 0;
        if (ck < c1) {
            const int32_t k0 = ck * 32;
            for (int32_t row = q0 + t / G; row < q1; row += rstep) {
                RowCtx rc;
                row_ctx(p, row + p.q_offset, rc);
                acc += __popc(allowed_bits32(p, rc, k0));
            }
            if (acc) atomicAdd(&cell[ck / cpb - j0], acc);
        }
        __syncthreads();
    }
    if (t < j1 - j0) out[j0 + t] = cell[t];
}

__global__ void __launch_bounds__(kThreads)
compact_kernel(int32_t n_q, int32_t n_kv, int32_t bq, int32_t bk, int32_t nkb, int32_t* kv_count,
               int32_t* kv_index /* counts on entry */, uint8_t* kv_partial,
               unsigned long long* live_pairs)
{
    extern __shared__ int32_t cnt[];  // nkb counts, then kThreads scan slots
    int32_t* scan = cnt + nkb;
    const int i = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t rowbase = (int64_t)i * nkb;
    for (int j = t; j < nkb; j += kThreads) cnt[j] = kv_index[rowbase + j];
    __syncthreads();

    // thread t owns cells [t*per, (t+1)*per)
    const int per = (nkb + kThreads - 1) / kThreads;
    const int j0 = t * per, j1 = min(j0 + per, nkb);
    int live = 0;
    long long pairs = 0;
    for (int j = j0; j < j1; ++j) {
        live += cnt[j] > 0;
        pairs += cnt[j];
    }
    // exclusive scan of `live` over the workgroup: within waves, then over
    // the wave totals
    const int lane = t & 63, w = t >> 6;
    int x = live;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) scan[w] = x;
    __syncthreads();
    int before = 0, total_live = 0;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) {
        const int v = scan[k];
        before += k < w ? v : 0;
        total_live += v;
    }
    int pos = before + x - live;
    const int32_t q0 = i * bq;
    const int64_t rows_in = min(q0 + bq, n_q) - q0;
    for (int j = j0; j < j1; ++j) {
        const int32_t c = cnt[j];
        if (c > 0) {
            const int64_t k0 = (int64_t)j * bk;
            const int64_t k1 = min((int64_t)n_kv, k0 + bk);
            kv_index[rowbase + pos] = j;
            kv_partial[rowbase + pos] = (uint8_t)((int64_t)c != rows_in * (k1 - k0));
            ++pos;
        }
    }
    __syncthreads();  // every count read before the padding overwrites them
    for (int e = total_live + t; e < nkb; e += kThreads) {
        kv_index[rowbase + e] = -1;
        kv_partial[rowbase + e] = 0;
    }
    if (t == 0) kv_count[i] = total_live;
    // wave sums, then one atomic per workgroup (integers: exact in any order);
    // every wave's atomic on the one counter would be serialised
    __shared__ long long wpairs[kThreads / 64];
    for (int off = 32; off > 0; off >>= 1) pairs += __shfl_down(pairs, off, 64);
    if (lane == 0) wpairs[w] = pairs;
    __syncthreads();
    if (t == 0) {
        long long sum = 0;
#pragma unroll
        for (int k = 0; k < kThreads / 64; ++k) sum += wpairs[k];
        if (sum) atomicAdd(live_pairs, (unsigned long long)sum);
    }
}

}  // namespace

hipError_t launch_zero_i64(int64_t* p, hipStream_t stream)
{
    hipLaunchKernelGGL(zero_i64, dim3(1), dim3(1), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_block_mask(const DevPattern& p, int32_t n_q, int32_t n_kv, int32_t block_q,
                             int32_t block_kv, int32_t* kv_count, int32_t* kv_index,
                             uint8_t* kv_partial, int64_t* live_pairs, hipStream_t stream)
{
    const int32_t nqb = (n_q + block_q - 1) / block_q;
    const int32_t nkb = (n_kv + block_kv - 1) / block_kv;
    if (nkb == 0) {
        // no keys: every list is empty
        hipLaunchKernelGGL(compact_kernel, dim3(nqb), dim3(kThreads), sizeof(int32_t) * kThreads, stream,
                           n_q, n_kv, block_q, block_kv, 0, kv_count, kv_index, kv_partial,
                           reinterpret_cast<unsigned long long*>(live_pairs));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_zero_i64(live_pairs, stream);
    }
    const int32_t bpg = group_chunks(block_kv) / (block_kv / 32);
    const int32_t ngroups = (nkb + bpg - 1) / bpg;
    hipLaunchKernelGGL(count_kernel, dim3((unsigned)((int64_t)nqb * ngroups)), dim3(kThreads), 0, stream, p,
                       n_q, n_kv, block_q, block_kv, nkb, ngroups, kv_index, live_pairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = sizeof(int32_t) * ((size_t)nkb + kThreads);
    hipLaunchKernelGGL(compact_kernel, dim3(nqb), dim3(kThreads), lds, stream, n_q, n_kv, block_q, block_kv,
                       nkb, kv_count, kv_index, kv_partial, reinterpret_cast<unsigned long long*>(live_pairs));
    return hipGetLastError();
}

}  // namespace sa
