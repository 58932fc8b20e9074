// attn_block.hip -- fused block-sparse attention forward over live key tiles.
//
// What is computed: for every query row, softmax(q.k^T * scale) over the
// allowed keys, times V, and the logsumexp (blog "Sparse transformers: how to
// cut the O(n^2) of attention", section on how it looks in code; masking with
// -inf before the softmax equals a softmax over the allowed keys only).
// How: only the key tiles listed as live for the query block are visited
// ("Sparse Attention" glossary, section on turning a pattern into savings:
// the kernel skips empty tiles); the pair predicate is applied only on tiles
// marked partial (or clipped by the sequence end); the softmax is carried
// online across tiles (running max, running sum, rescaled accumulator).
//
// gfx950 mapping.  A workgroup owns one (batch, head, query block) and has
// BQ/32 waves of 32 query rows each.  Per live tile:
//   * K and V tiles [BK x D] bf16 are copied HBM -> LDS with 16-byte loads
//     (XOR-swizzled 16-byte chunks so MFMA operand reads avoid bank
//     conflicts);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//     wave's Q^T held in registers).  In the accumulator layout one lane
//     holds one query column, so row max / row sum are in-lane reductions
//     plus one v_permlane32_swap between the two half-waves;
//   * P^T (bf16) stays in the accumulator registers and is directly the B
//     operand of O^T += V^T P^T; the V^T operand is read from LDS with
//     ds_read_b64_tr_b16 (transposing 16-bit reads), so no transpose pass;
//   * exp2 with the scale folded into one FMA; the running max is raised
//     only when some row's tile max exceeds it by more than 8 (log2 units),
//     which keeps every exponent <= 2^8 and skips most accumulator rescales.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLazyLog2 = 8.0f;  // rescale threshold in log2 units

template <int D>
__device__ __forceinline__ int kswz(int r)
{
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int r)
{
    return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

// workgroup id -> logical work item, so that consecutive work items (the
// query blocks of one head, which share key tiles) land on the same XCD
// when workgroups are dispatched round-robin over the 8 XCDs.  A bijection
// for any grid size, so correctness never depends on the dispatch order.
__device__ __forceinline__ int xcd_remap(int wg, int nwg)
{
    const int c = nwg / 8, r = nwg % 8;
    const int x = wg % 8, slot = wg / 8;
    const int base = x < r ? x * (c + 1) : r * (c + 1) + (x - r) * c;
    return base + slot;
}

__device__ __forceinline__ float wave_swap_other(float v)
{
    // value of lane l ^ 32
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

template <int D, int BQ, int BK, bool OF32>
__global__ void __launch_bounds__(BQ * 2)
attn_block_kernel(AttnParams a)
{
    constexpr int NW = BQ / 32;
    constexpr int T = NW * 64;
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int NSB = BK / 32;          // 32-key sub-blocks per tile
    constexpr int NDC = D / 16;           // k-steps of S^T
    constexpr int NDB = D / 32;           // 32-wide output column blocks
    constexpr int LOADS = BK * CH / T;    // 16-byte loads per thread per tensor
    static_assert(BK * CH % T == 0, "tile load split");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BK * D * 2];
    uint8_t* const kl = smem;
    uint8_t* const vl = smem + BK * D * 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hh = lane >> 5;     // half-wave
    const int l32 = lane & 31;

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = item % a.nqb;
    const int bh = item / a.nqb;
    const int b = bh / a.heads, h = bh % a.heads;

    const uint16_t* qg = a.q + b * a.q_sb + h * a.q_sh;
    const uint16_t* kg = a.k + b * a.k_sb + h * a.k_sh;
    const uint16_t* vg = a.v + b * a.v_sb + h * a.v_sh;

    const int qrow = qb * BQ + wave * 32 + l32;
    const bool qvalid = qrow < a.n_q;

    // Q^T operand: lane holds q[qrow][16*dc + 8*hh + 0..7]
    bf16x8 qf[NDC];
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qvalid) raw = *reinterpret_cast<const u32x4*>(qg + (int64_t)qrow * a.q_sn + 16 * dc + 8 * hh);
        qf[dc] = __builtin_bit_cast(bf16x8, raw);
    }

    RowCtx rc;
    row_ctx(a.pat, qrow + a.pat.q_offset, rc);

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c = a.scale_log2;
    const float thr = kLazyLog2 / c;

    const int n_tiles = a.kv_count[qb];
    const int32_t* idx_row = a.kv_index + (int64_t)qb * a.nkb;
    const uint8_t* part_row = a.kv_partial + (int64_t)qb * a.nkb;

    for (int e = 0; e < n_tiles; ++e) {
        const int j = idx_row[e];
        if ((unsigned)j >= (unsigned)a.nkb) continue;  // not a key block: skip (uniform)
        const int kv0 = j * BK;
        const bool need_mask = part_row[e] != 0 || kv0 + BK > a.n_kv;

        // ---- HBM -> registers
        u32x4 kr[LOADS], vr[LOADS];
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int u = tid + it * T;
            const int r = u / CH, cc = u % CH;
            const int kv = kv0 + r;
            u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
            if (kv < a.n_kv) {
                zk = *reinterpret_cast<const u32x4*>(kg + (int64_t)kv * a.k_sn + cc * 8);
                zv = *reinterpret_cast<const u32x4*>(vg + (int64_t)kv * a.v_sn + cc * 8);
            }
            kr[it] = zk;
            vr[it] = zv;
        }
        __syncthreads();  // previous tile fully consumed
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int u = tid + it * T;
            const int r = u / CH, cc = u % CH;
            *reinterpret_cast<u32x4*>(kl + r * D * 2 + ((cc ^ kswz<D>(r)) << 4)) = kr[it];
            *reinterpret_cast<u32x4*>(vl + r * D * 2 + ((cc ^ vswz<D>(r)) << 4)) = vr[it];
        }
        __syncthreads();

        // ---- S^T = K Q^T
        f32x16 s[NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
            for (int i = 0; i < 16; ++i) s[sb][i] = 0.f;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int r = sb * 32 + l32;
                const int cc = 2 * dc + hh;
                const bf16x8 ka = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(kl + r * D * 2 + ((cc ^ kswz<D>(r)) << 4)));
                s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[dc], s[sb], 0, 0, 0);
            }
        }

        // ---- element mask on partial / clipped tiles only
        if (need_mask) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kv = kv0 + sb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                    const bool ok = kv < a.n_kv && pair_allowed(a.pat, rc, kv);
                    s[sb][i] = ok ? s[sb][i] : -INFINITY;
                }
        }

        // ---- online softmax (row = lane's query)
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
        mx = fmaxf(mx, wave_swap_other(mx));
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run + thr)) {
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            m_run = m_new;
        }
        const float mc = m_run == -INFINITY ? 0.f : m_run * c;
        float lsum = 0.f;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], c, -mc));
                s[sb][i] = p;
                lsum += p;
            }
        l_run += lsum;

        // ---- O^T += V^T P^T
        const int g = lane >> 4, jj = lane & 15;
        const int vrow_off = 4 * (g >> 1) + (jj >> 2);
        const int vcol_off = 16 * (g & 1) + 4 * (jj & 3);
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                bf16x8 pb;
#pragma unroll
                for (int t = 0; t < 8; ++t) pb[t] = (__bf16)s[sb][8 * cb + t];
                const int r0 = sb * 32 + 16 * cb + vrow_off;
                const int r1 = r0 + 8;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int col = 32 * db + vcol_off;
                    const int ch = col >> 3, within = (col & 7) * 2;
                    const bf16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4*)(vl + r0 * D * 2 + ((ch ^ vswz<D>(r0)) << 4) + within));
                    const bf16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4*)(vl + r1 * D * 2 + ((ch ^ vswz<D>(r1)) << 4) + within));
                    const bf16x8 va = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue
    const float l_tot = l_run + wave_swap_other(l_run);
    if (qvalid) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int64_t obase = b * a.o_sb + h * a.o_sh + (int64_t)qrow * a.o_sn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dv = 32 * db + 8 * r4 + 4 * hh;
                const float x0 = o[db][4 * r4 + 0] * inv, x1 = o[db][4 * r4 + 1] * inv;
                const float x2 = o[db][4 * r4 + 2] * inv, x3 = o[db][4 * r4 + 3] * inv;
                if (OF32) {
                    float* op = reinterpret_cast<float*>(a.o) + obase + dv;
                    *reinterpret_cast<float4*>(op) = make_float4(x0, x1, x2, x3);
                } else {
                    uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + obase + dv;
                    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
                    const bf16x2 p01 = {(__bf16)x0, (__bf16)x1};
                    const bf16x2 p23 = {(__bf16)x2, (__bf16)x3};
                    const u32x2 w = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
                    *reinterpret_cast<u32x2*>(op) = w;
                }
            }
        if (a.lse && hh == 0)
            a.lse[((int64_t)b * a.heads + h) * a.n_q + qrow] =
                l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
    }
}

template <int D, int BQ, int BK, bool OF32>
hipError_t launch_one(const AttnParams& a, hipStream_t stream)
{
    const int64_t items = (int64_t)a.batch * a.heads * a.nqb;
    hipLaunchKernelGGL((attn_block_kernel<D, BQ, BK, OF32>), dim3((unsigned)items), dim3(BQ * 2), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int BQ, int BK>
hipError_t launch_o(const AttnParams& a, int o_f32, hipStream_t stream)
{
    return o_f32 ? launch_one<D, BQ, BK, true>(a, stream) : launch_one<D, BQ, BK, false>(a, stream);
}

template <int D>
hipError_t launch_d(const AttnParams& a, int bq, int bk, int o_f32, hipStream_t stream)
{
    if (bq == 128 && bk == 128) return launch_o<D, 128, 128>(a, o_f32, stream);
    if (bq == 128 && bk == 64) return launch_o<D, 128, 64>(a, o_f32, stream);
    if (bq == 64 && bk == 128) return launch_o<D, 64, 128>(a, o_f32, stream);
    if (bq == 64 && bk == 64) return launch_o<D, 64, 64>(a, o_f32, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_blocks(const AttnParams& a, int head_dim, int block_q, int block_kv,
                              int o_f32, hipStream_t stream)
{
    if (head_dim == 128) return launch_d<128>(a, block_q, block_kv, o_f32, stream);
    if (head_dim == 64) return launch_d<64>(a, block_q, block_kv, o_f32, stream);
    return hipErrorInvalidValue;
}

}  // namespace sa
