// block_mask.hip -- pattern -> per-query-block lists of live key blocks.
//
// "Sparse Attention" glossary, section on turning a pattern into savings:
// the mask is split into fixed blocks and blocks without any allowed pair
// are skipped; a block is live when it holds at least one allowed pair.
//
// One workgroup per query block.  Instead of testing pairs one at a time,
// every pattern term is an interval (or a short arithmetic progression) of
// key positions for a fixed query, so the allowed keys of one query inside a
// 32-key chunk form a 32-bit mask built from a few shifts; a popcount gives
// the pair count.  Counts accumulate per key block in LDS, then the live
// blocks are compacted in ascending order with a workgroup scan.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

// Bits [lo, hi) of the chunk [k0, k0 + 32), positions clamped to the chunk.
__device__ __forceinline__ uint32_t range_bits(int64_t lo, int64_t hi, int64_t k0)
{
    int64_t a = lo > k0 ? lo : k0;
    int64_t b = hi < k0 + 32 ? hi : k0 + 32;
    if (b <= a) return 0u;
    uint32_t ua = (uint32_t)(a - k0), ub = (uint32_t)(b - k0);
    uint32_t hi_mask = ub >= 32 ? 0xFFFFFFFFu : ((1u << ub) - 1u);
    uint32_t lo_mask = (1u << ua) - 1u;
    return hi_mask & ~lo_mask;
}

// Allowed keys of absolute query position q among keys [k0, k0 + 32) with
// k0 + 32 possibly beyond n_kv (the caller clips).
__device__ uint32_t chunk_mask(const DevPattern& p, int64_t q, int64_t k0, int32_t qu,
                               const int32_t* rnd)
{
    uint32_t m = 0;
    if (p.window_left >= 0)
        m |= range_bits(q - p.window_left, q + (int64_t)p.window_right + 1, k0);
    m |= range_bits(0, p.sinks, k0);
    if (q < p.global_tokens)
        m = 0xFFFFFFFFu;
    else
        m |= range_bits(0, p.global_tokens, k0);
    if (p.stride > 0) {
        // keys kv <= q - phase with (q - phase - kv) % stride == 0
        int64_t top = q - p.stride_phase;
        if (top > k0 + 31) top = k0 + 31;
        if (top >= k0) {
            int64_t a = q - p.stride_phase - top;  // >= 0
            int64_t r = a % p.stride;
            int64_t kv = top - (r == 0 ? 0 : p.stride - r);
            for (; kv >= k0; kv -= p.stride) m |= 1u << (uint32_t)(kv - k0);
        }
    }
    if (p.unit > 0) {
        if (p.unit_window >= 0)
            m |= range_bits((int64_t)(qu - p.unit_window) * p.unit,
                            (int64_t)(qu + p.unit_window + 1) * p.unit, k0);
        for (int i = 0; i < p.n_rand && i < kMaxRand; ++i)
            if (rnd[i] >= 0)
                m |= range_bits((int64_t)rnd[i] * p.unit, (int64_t)(rnd[i] + 1) * p.unit, k0);
    }
    if (p.causal)
        m &= range_bits(0, q + 1, k0);
    return m;
}

__global__ void zero_i64(int64_t* p) { *p = 0; }

__global__ void __launch_bounds__(kThreads)
build_block_mask_kernel(DevPattern p, int32_t n_q, int32_t n_kv, int32_t bq, int32_t bk,
                        int32_t nkb, int32_t* kv_count, int32_t* kv_index, uint8_t* kv_partial,
                        unsigned long long* live_pairs)
{
    extern __shared__ int32_t cell[];  // nkb counters, then kThreads scan slots
    int32_t* scan = cell + nkb;
    const int i = blockIdx.x;
    const int t = threadIdx.x;
    const int32_t q0 = i * bq;
    const int32_t q1 = min(q0 + bq, n_q);
    const int32_t nchunks = (n_kv + 31) / 32;

    for (int j = t; j < nkb; j += kThreads) cell[j] = 0;
    __syncthreads();

    // Each thread owns chunks c = t, t + T, ... and walks every row of the block.
    for (int32_t c = t; c < nchunks; c += kThreads) {
        const int64_t k0 = (int64_t)c * 32;
        const uint32_t clip = range_bits(0, n_kv, k0);
        int32_t cnt = 0;
        for (int32_t qr = q0; qr < q1; ++qr) {
            const int64_t q = (int64_t)qr + p.q_offset;
            int32_t qu = 0;
            int32_t rnd[kMaxRand];
            if (p.unit > 0) {
                qu = (int32_t)(q / p.unit);
                for (int r = 0; r < kMaxRand; ++r)
                    rnd[r] = (r < p.n_rand && qu < p.rand_rows)
                                 ? p.rand_units[(int64_t)qu * p.n_rand + r]
                                 : -1;
            }
            cnt += __popc(chunk_mask(p, q, k0, qu, rnd) & clip);
        }
        if (cnt) atomicAdd(&cell[(int32_t)(k0 / bk)], cnt);
    }
    __syncthreads();

    // Ordered compaction: thread t owns cells [t*per, (t+1)*per).
    const int per = (nkb + kThreads - 1) / kThreads;
    const int j0 = t * per, j1 = min(j0 + per, nkb);
    int live = 0;
    long long pairs = 0;
    for (int j = j0; j < j1; ++j) {
        live += cell[j] > 0;
        pairs += cell[j];
    }
    scan[t] = live;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        int v = t >= off ? scan[t - off] : 0;
        __syncthreads();
        scan[t] += v;
        __syncthreads();
    }
    int pos = scan[t] - live;  // exclusive prefix
    const int64_t rowbase = (int64_t)i * nkb;
    const int64_t rows_in = q1 - q0;
    for (int j = j0; j < j1; ++j) {
        int32_t cnt = cell[j];
        if (cnt > 0) {
            const int64_t k0 = (int64_t)j * bk;
            const int64_t k1 = min((int64_t)n_kv, k0 + bk);
            kv_index[rowbase + pos] = j;
            kv_partial[rowbase + pos] = (uint8_t)((int64_t)cnt != rows_in * (k1 - k0));
            ++pos;
        }
    }
    const int total_live = scan[kThreads - 1];
    for (int e = total_live + t; e < nkb; e += kThreads) {
        kv_index[rowbase + e] = -1;
        kv_partial[rowbase + e] = 0;
    }
    if (t == 0) kv_count[i] = total_live;

    // live pairs: wave reduction, then one atomic per wave (integer, so exact
    // whatever the order)
    for (int off = 32; off > 0; off >>= 1) pairs += __shfl_down(pairs, off, 64);
    if ((t & 63) == 0 && pairs) atomicAdd(live_pairs, (unsigned long long)pairs);
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
    hipLaunchKernelGGL(zero_i64, dim3(1), dim3(1), 0, stream, live_pairs);
    const size_t lds = sizeof(int32_t) * ((size_t)nkb + kThreads);
    hipLaunchKernelGGL(build_block_mask_kernel, dim3(nqb), dim3(kThreads), lds, stream, p, n_q,
                       n_kv, block_q, block_kv, nkb, kv_count, kv_index, kv_partial,
                       reinterpret_cast<unsigned long long*>(live_pairs));
    return hipGetLastError();
}

}  // namespace sa
