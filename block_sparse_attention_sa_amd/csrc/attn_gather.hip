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
// the gather bandwidth.  One wave per (batch, head, query):
//   pass 1: D/8 lanes share one key row (16 contiguous bytes each, so a key
//           row is one coalesced 256-byte (D=128) read); partial dots are
//           reduced across those lanes; scores go to LDS;
//   pass 2: row max and sum of exp2 over the LDS scores;
//   pass 3: the same lane grouping reads V rows and accumulates p * v in
//           float32; the key groups are reduced at the end.
// Work items are ordered head-major so that concurrently running waves share
// one head's K/V in the caches.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWaves = 4;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int D, bool OF32>
__global__ void __launch_bounds__(kWaves * 64)
attn_gather_kernel(AttnParams a)
{
    constexpr int LPK = D / 8;        // lanes per key row (8 bf16 each)
    constexpr int KPS = 64 / LPK;     // keys per wave step
    extern __shared__ float sc_all[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float* sc = sc_all + wave * a.topk;

    const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
    const int64_t n_items = (int64_t)a.batch * a.heads * a.n_q;
    if (item >= n_items) return;
    // head-major order: item = (bh) * n_q + t
    const int t = (int)(item % a.n_q);
    const int bh = (int)(item / a.n_q);
    const int b = bh / a.heads, h = bh % a.heads;

    const uint16_t* kg = a.k + b * a.k_sb + h * a.k_sh;
    const uint16_t* vg = a.v + b * a.v_sb + h * a.v_sh;
    const int32_t* list = a.gidx + bh * a.g_bh_stride + (int64_t)t * a.topk;

    const int sub = lane % LPK;      // which 8-element slice of the row
    const int kgrp = lane / LPK;     // which key of the step

    // query slice, float32
    float qv[8];
    {
        const u32x4 w = *reinterpret_cast<const u32x4*>(a.q + b * a.q_sb + h * a.q_sh +
                                                        (int64_t)t * a.q_sn + sub * 8);
        for (int i = 0; i < 4; ++i) {
            qv[2 * i] = bf_lo(w[i]);
            qv[2 * i + 1] = bf_hi(w[i]);
        }
    }

    // pass 1: scores (log2 domain, scale folded in)
    const float c = a.scale_log2;
    for (int e0 = 0; e0 < a.topk; e0 += KPS * 4) {
        float part[4];
        int keyid[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * KPS + kgrp;
            int s = e < a.topk ? list[e] : -1;
            s = (s >= 0 && s < a.n_kv) ? s : -1;
            keyid[u] = s;
            float acc = 0.f;
            if (s >= 0) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(kg + (int64_t)s * a.k_sn + sub * 8);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc = __builtin_fmaf(qv[2 * i], bf_lo(w[i]), acc);
                    acc = __builtin_fmaf(qv[2 * i + 1], bf_hi(w[i]), acc);
                }
            }
            part[u] = acc;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int off = 1; off < LPK; off <<= 1) part[u] += __shfl_xor(part[u], off, 64);
            const int e = e0 + u * KPS + kgrp;
            if (sub == 0 && e < a.topk) sc[e] = keyid[u] >= 0 ? part[u] * c : -INFINITY;
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

    // pass 2: max and sum
    float mx = -INFINITY;
    for (int e = lane; e < a.topk; e += 64) mx = fmaxf(mx, sc[e]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float msafe = mx == -INFINITY ? 0.f : mx;
    float sum = 0.f;
    for (int e = lane; e < a.topk; e += 64) {
        const float p = __builtin_amdgcn_exp2f(sc[e] - msafe);
        sc[e] = p;
        sum += p;
    }
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

    // pass 3: O = sum p v
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int e0 = 0; e0 < a.topk; e0 += KPS * 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * KPS + kgrp;
            if (e < a.topk) {
                int s = list[e];
                const float p = sc[e];
                if (s >= 0 && s < a.n_kv && p != 0.f) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(vg + (int64_t)s * a.v_sn + sub * 8);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] = __builtin_fmaf(p, bf_lo(w[i]), acc[2 * i]);
                        acc[2 * i + 1] = __builtin_fmaf(p, bf_hi(w[i]), acc[2 * i + 1]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int off = LPK; off < 64; off <<= 1) acc[i] += __shfl_xor(acc[i], off, 64);

    if (kgrp == 0) {
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
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
            a.lse[(int64_t)bh * a.n_q + t] =
                sum > 0.f ? (msafe + __log2f(sum)) * 0.69314718055994531f : -INFINITY;
    }
}

template <int D, bool OF32>
hipError_t launch_one(const AttnParams& a, hipStream_t stream)
{
    const int64_t items = (int64_t)a.batch * a.heads * a.n_q;
    const int64_t wgs = (items + kWaves - 1) / kWaves;
    const size_t lds = sizeof(float) * (size_t)kWaves * a.topk;
    hipLaunchKernelGGL((attn_gather_kernel<D, OF32>), dim3((unsigned)wgs), dim3(kWaves * 64), lds,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_gather(const AttnParams& a, int head_dim, int o_f32, hipStream_t stream)
{
    if (head_dim == 128) return o_f32 ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
    if (head_dim == 64) return o_f32 ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace sa
