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
// accumulation.
//   * bwd_dq_kernel: a wave owns 32 queries and walks their live key tiles in
//     32-key steps (K, K^T and V staged in LDS by the workgroup); S^T and
//     dP^T come out with one query per lane, so the row's LSE and D are one
//     register each; dS goes through a per-wave LDS tile into dQ += dS K.
//   * bwd_dkdv_kernel: a wave owns 32 keys and walks the query tiles whose
//     lists hold its key block (lists transposed by bwd_transpose_kernel);
//     S and dP come out with one key per lane; P^T and dS^T go through
//     per-wave LDS tiles into dV += P^T dO and dK += dS^T Q.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint16_t bf16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// The pair predicate of the pattern for one (query position, key) pair: the
// same terms as allowed_bits32, one pair at a time.
__device__ bool allowed_pair(const DevPattern& p, int32_t q, int32_t kv)
{
    if (kv >= p.n_kv || (p.causal && kv > q)) return false;
    if (p.window_left >= 0 && q - kv <= p.window_left && kv - q <= p.window_right) return true;
    if (kv < p.sinks) return true;
    if (p.stride > 0 && q >= kv && fmod_(q - kv, p.stride_div) == p.stride_phase) return true;
    if (q < p.global_tokens || kv < p.global_tokens) return true;
    if (p.unit > 0) {
        const int32_t qu = fdiv(q, p.unit_div), ku = fdiv(kv, p.unit_div);
        if (p.unit_window >= 0 && abs(qu - ku) <= p.unit_window) return true;
        if (qu < p.rand_rows)
            for (int i = 0; i < p.n_rand; ++i)
                if (p.rand_units[(int64_t)qu * p.n_rand + i] == ku) return true;
    }
    return false;
}

// D[row] = sum_c dO[row][c] * O[row][c]; 16 lanes per row
__global__ void __launch_bounds__(256) bwd_dsum_kernel(const uint16_t* __restrict__ dout, const float* __restrict__ o,
                                                       int64_t rows, int32_t d, float* __restrict__ dsum)
{
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    float acc = 0.f;
    if (row < rows)
        for (int c = l; c < d; c += 16)
            acc += __uint_as_float((uint32_t)dout[row * d + c] << 16) * o[row * d + c];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (row < rows && l == 0) dsum[row] = acc;
}

// For every list row L and key block j: the query blocks whose list holds j,
// ascending, with the list's partial flag.
__global__ void bwd_transpose_kernel(const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_index,
                                     const uint8_t* __restrict__ kv_partial, int32_t n_lists, int32_t nqb,
                                     int32_t nkb, int32_t* __restrict__ q_count, int32_t* __restrict__ q_index,
                                     uint8_t* __restrict__ q_partial)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)n_lists * nkb) return;
    const int64_t L = t / nkb;
    const int j = (int)(t % nkb);
    int n = 0;
    for (int i = 0; i < nqb; ++i) {
        const int64_t row = L * nqb + i;
        const int cnt = min(kv_count[row], nkb);
        for (int e = 0; e < cnt; ++e)
            if (kv_index[row * nkb + e] == j) {
                q_index[t * nqb + n] = i;
                q_partial[t * nqb + n] = kv_partial[row * nkb + e];
                ++n;
                break;
            }
    }
    q_count[t] = n;
}

// Rows [r0, r0 + 32) of a [.., n, D] bf16 tensor into LDS: row-major `rm`
// ([32][D]) and, when T, transposed `tr` ([D][32]); rows at or past n are zero.
template <int D, bool T>
__device__ __forceinline__ void stage32(const uint16_t* __restrict__ src, int r0, int n, uint16_t* rm, uint16_t* tr,
                                        int tid, int nthreads)
{
    constexpr int CH = D / 8;  // 16-byte chunks per row
    for (int idx = tid; idx < 32 * CH; idx += nthreads) {
        const int r = idx / CH, ch = idx % CH;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (r0 + r < n) w = *reinterpret_cast<const u32x4*>(src + (int64_t)(r0 + r) * D + 8 * ch);
        *reinterpret_cast<u32x4*>(rm + r * D + 8 * ch) = w;
        if (T) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                tr[(8 * ch + 2 * x) * 32 + r] = (uint16_t)(w[x] & 0xFFFFu);
                tr[(8 * ch + 2 * x + 1) * 32 + r] = (uint16_t)(w[x] >> 16);
            }
        }
    }
}

template <int D, int BQ, int BK>
__global__ void __launch_bounds__(BQ * 2)
bwd_dq_kernel(BwdParams a)
{
    constexpr int NW = BQ / 32, NT = BQ * 2, NDC = D / 16, NDB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t kt[32 * D];
    __shared__ __attribute__((aligned(16))) uint16_t ktt[D * 32];
    __shared__ __attribute__((aligned(16))) uint16_t vt[32 * D];
    __shared__ __attribute__((aligned(16))) uint16_t dst[NW][32 * 32];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
    const int qb = blockIdx.x % a.nqb, bh = blockIdx.x / a.nqb;
    const int q = qb * BQ + 32 * w + l32;  // this lane's query row
    const bool q_ok = q < a.n_q;
    const uint16_t* qg = a.q + (int64_t)bh * a.n_q * D;
    const uint16_t* gg = a.dout + (int64_t)bh * a.n_q * D;
    const uint16_t* kg = a.k + (int64_t)bh * a.n_kv * D;
    const uint16_t* vg = a.v + (int64_t)bh * a.n_kv * D;
    // B operands Q^T and dO^T: lane holds row q, dims 16s + 8hh .. + 7
    bf16x8 qop[NDC], gop[NDC];
#pragma unroll
    for (int s = 0; s < NDC; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (q_ok) {
            x = *reinterpret_cast<const u32x4*>(qg + (int64_t)q * D + 16 * s + 8 * hh);
            y = *reinterpret_cast<const u32x4*>(gg + (int64_t)q * D + 16 * s + 8 * hh);
        }
        qop[s] = __builtin_bit_cast(bf16x8, x);
        gop[s] = __builtin_bit_cast(bf16x8, y);
    }
    const float lse = q_ok ? a.lse[(int64_t)bh * a.n_q + q] : INFINITY;
    const float dsum = q_ok ? a.dsum[(int64_t)bh * a.n_q + q] : 0.f;
    const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;  // a row without keys has no pair
    RowCtx rc;
    row_ctx(a.pat, q + a.pat.q_offset, rc);
    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

    const int64_t lrow = (a.per_head_lists ? (int64_t)bh * a.nqb : 0) + qb;
    const int cnt = min(a.kv_count[lrow], a.nkb);
    for (int e = 0; e < cnt; ++e) {
        const int j = a.kv_index[lrow * a.nkb + e];
        if ((unsigned)j >= (unsigned)a.nkb) continue;
        const bool part = a.kv_partial[lrow * a.nkb + e] != 0;
        for (int t = 0; t < BK / 32; ++t) {
            const int k0 = j * BK + 32 * t;
            if (k0 >= a.n_kv) break;
            const bool need_mask = part || k0 + 32 > a.n_kv;
            __syncthreads();
            stage32<D, true>(kg, k0, a.n_kv, kt, ktt, tid, NT);
            stage32<D, false>(vg, k0, a.n_kv, vt, nullptr, tid, NT);
            __syncthreads();
            // S^T = K Q^T and dP^T = V dO^T: lane = query, element i = key 8(i/4) + 4hh + i%4
            f32x16 s, dp;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(kt + l32 * D + 16 * c + 8 * hh), qop[c], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(vt + l32 * D + 16 * c + 8 * hh), gop[c], dp, 0, 0, 0);
            }
            uint32_t mbits = 0xFFFFFFFFu;
            if (need_mask) mbits = allowed_bits32(a.pat, rc, k0) >> (4 * hh);
            uint16_t* myds = dst[w];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const bool ok = (mbits >> (8 * (i >> 2) + (i & 3))) & 1u;
                const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -lse2)) : 0.f;
                const float ds = p * (dp[i] - dsum);
                myds[l32 * 32 + 8 * (i >> 2) + 4 * hh + (i & 3)] = bf16_bits(ds);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // dQ (queries x d) += dS (queries x keys) K (keys x d)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 aop = lds8(myds + l32 * 32 + 16 * ks + 8 * hh);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        aop, lds8(ktt + (32 * db + l32) * 32 + 16 * ks + 8 * hh), dq[db], 0, 0, 0);
            }
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
__global__ void __launch_bounds__(BK * 2)
bwd_dkdv_kernel(BwdParams a)
{
    constexpr int NW = BK / 32, NT = BK * 2, NDC = D / 16, NDB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t qt[32 * D];
    __shared__ __attribute__((aligned(16))) uint16_t qtt[D * 32];
    __shared__ __attribute__((aligned(16))) uint16_t gt[32 * D];
    __shared__ __attribute__((aligned(16))) uint16_t gtt[D * 32];
    __shared__ __attribute__((aligned(16))) uint16_t ptt[NW][32 * 32];
    __shared__ __attribute__((aligned(16))) uint16_t dstt[NW][32 * 32];
    __shared__ float lse_s[32], dsum_s[32];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
    const int kb = blockIdx.x % a.nkb, bh = blockIdx.x / a.nkb;
    const int kv = kb * BK + 32 * w + l32;  // this lane's key row
    const bool k_ok = kv < a.n_kv;
    const uint16_t* qg = a.q + (int64_t)bh * a.n_q * D;
    const uint16_t* gg = a.dout + (int64_t)bh * a.n_q * D;
    const uint16_t* kg = a.k + (int64_t)bh * a.n_kv * D;
    const uint16_t* vg = a.v + (int64_t)bh * a.n_kv * D;
    // B operands K^T and V^T: lane holds key row kv, dims 16s + 8hh .. + 7
    bf16x8 kop[NDC], vop[NDC];
#pragma unroll
    for (int s = 0; s < NDC; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (k_ok) {
            x = *reinterpret_cast<const u32x4*>(kg + (int64_t)kv * D + 16 * s + 8 * hh);
            y = *reinterpret_cast<const u32x4*>(vg + (int64_t)kv * D + 16 * s + 8 * hh);
        }
        kop[s] = __builtin_bit_cast(bf16x8, x);
        vop[s] = __builtin_bit_cast(bf16x8, y);
    }
    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

    const int64_t lrow = (a.per_head_lists ? (int64_t)bh * a.nkb : 0) + kb;
    const int cnt = min(a.q_count[lrow], a.nqb);
    for (int e = 0; e < cnt; ++e) {
        const int i_blk = a.q_index[lrow * a.nqb + e];
        const bool part = a.q_partial[lrow * a.nqb + e] != 0;
        for (int t = 0; t < BQ / 32; ++t) {
            const int q0 = i_blk * BQ + 32 * t;
            if (q0 >= a.n_q) break;
            const bool need_mask = part || q0 + 32 > a.n_q || kb * BK + BK > a.n_kv;
            __syncthreads();
            stage32<D, true>(qg, q0, a.n_q, qt, qtt, tid, NT);
            stage32<D, true>(gg, q0, a.n_q, gt, gtt, tid, NT);
            if (tid < 32) {
                const int qr = q0 + tid;
                const float l = qr < a.n_q ? a.lse[(int64_t)bh * a.n_q + qr] : INFINITY;
                lse_s[tid] = l == -INFINITY ? INFINITY : l * kLog2e;
                dsum_s[tid] = qr < a.n_q ? a.dsum[(int64_t)bh * a.n_q + qr] : 0.f;
            }
            __syncthreads();
            // S = Q K^T and dP = dO V^T: lane = key, element i = query 8(i/4) + 4hh + i%4
            f32x16 s, dp;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(qt + l32 * D + 16 * c + 8 * hh), kop[c], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds8(gt + l32 * D + 16 * c + 8 * hh), vop[c], dp, 0, 0, 0);
            }
            uint16_t* myp = ptt[w];
            uint16_t* myds = dstt[w];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int qi = 8 * (i >> 2) + 4 * hh + (i & 3);
                const int qr = q0 + qi;
                bool ok = true;
                if (need_mask) ok = qr < a.n_q && allowed_pair(a.pat, qr + a.pat.q_offset, kv);
                const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -lse_s[qi])) : 0.f;
                const float ds = p * (dp[i] - dsum_s[qi]);
                myp[l32 * 32 + qi] = bf16_bits(p);
                myds[l32 * 32 + qi] = bf16_bits(ds);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // dV (keys x d) += P^T (keys x queries) dO; dK += dS^T Q
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 pop = lds8(myp + l32 * 32 + 16 * ks + 8 * hh);
                const bf16x8 sop = lds8(myds + l32 * 32 + 16 * ks + 8 * hh);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        pop, lds8(gtt + (32 * db + l32) * 32 + 16 * ks + 8 * hh), dv[db], 0, 0, 0);
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        sop, lds8(qtt + (32 * db + l32) * 32 + 16 * ks + 8 * hh), dk[db], 0, 0, 0);
                }
            }
        }
    }
    // element (db, i): key row 8(i/4) + 4hh + i%4 of the wave, dim 32 db + l32
    float* dkg = a.dk + (int64_t)bh * a.n_kv * D;
    float* dvg = a.dv + (int64_t)bh * a.n_kv * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kr = kb * BK + 32 * w + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (kr < a.n_kv) {
                dkg[(int64_t)kr * D + 32 * db + l32] = dk[db][i] * a.scale;
                dvg[(int64_t)kr * D + 32 * db + l32] = dv[db][i];
            }
        }
}

template <int D, int BQ, int BK>
hipError_t launch_bwd_t(const BwdParams& a, hipStream_t stream)
{
    const int64_t bh = (int64_t)a.batch * a.heads;
    hipLaunchKernelGGL((bwd_dq_kernel<D, BQ, BK>), dim3((unsigned)(bh * a.nqb)), dim3(BQ * 2), 0, stream, a);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BQ, BK>), dim3((unsigned)(bh * a.nkb)), dim3(BK * 2), 0, stream, a);
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
    const int64_t rows = (int64_t)a.batch * a.heads * a.n_q;
    hipLaunchKernelGGL(bwd_dsum_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, a.dout, a.o, rows,
                       head_dim, a.dsum);
    const int64_t nt = (int64_t)a.n_lists * a.nkb;
    hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, stream, a.kv_count,
                       a.kv_index, a.kv_partial, a.n_lists, a.nqb, a.nkb, a.q_count, a.q_index, a.q_partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (head_dim == 128) return launch_bwd_d<128>(a, block_q, block_kv, stream);
    if (head_dim == 64) return launch_bwd_d<64>(a, block_q, block_kv, stream);
    return hipErrorInvalidValue;
}

}  // namespace sa
