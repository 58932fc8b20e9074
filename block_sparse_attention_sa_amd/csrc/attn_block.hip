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
// gfx950 mapping.  A workgroup owns one (batch, head, query block of BQ rows).
// Each wave owns 32 query rows, two waves per SIMD.  (The kernel can also
// give a wave NB = 2 column blocks of 32 queries, so that every K and V
// operand read from LDS feeds two MFMAs; that measured slower at both head
// dims, and is not launched.)
//   * Live key tiles are walked in 64-key sub-tiles.  K and V sub-tiles go
//     HBM -> LDS by buffer loads with LDS destination (no staging registers),
//     double buffered; the loop body is unrolled over the two buffer pairs so
//     each copy names its LDS objects statically.  A sub-tile that reaches
//     past the last key is copied through resources that end at n_kv, so
//     rows past the sequence end read as zero.  16-byte chunks are XOR
//     swizzled per row so the operand reads hit distinct banks.
//   * The live list is held in lane registers and read with readlane.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//     in registers).  In the accumulator layout one lane holds one query, so
//     row max / row sum are in-lane reductions plus one v_permlane32_swap.
//   * P^T (bf16) stays in registers as the B operand of O^T += V^T P^T; V^T
//     is read with ds_read_b64_tr_b16 (transposing 16-bit reads).
//   * exp2 with the scale folded into one FMA, against a per-row reference
//     m that need not be the running max: any m gives the same softmax, as
//     long as no exponent overflows.  The first sub-tile a row sees sets m to
//     its max; later sub-tiles skip the row max unless some lane's sum of P
//     over the sub-tile exceeds 2^16, and then the exact max is taken, the
//     accumulator rescaled and P recomputed.  m is an actual score of the
//     row, so the largest term is at least 1 and nothing important underflows.
//   * Wave priorities (s_setprio): highest while a wave issues matrix
//     instructions, middle during its softmax, lowest otherwise, so that the
//     two waves sharing a SIMD tend to alternate matrix and vector phases.
//   * On a sub-tile that needs the mask, a wave whose rows may all see all of
//     its keys skips the element mask, and one whose rows may see none of
//     them skips the sub-tile.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kSumLimit = 65536.0f;  // largest per-lane sub-tile sum taken without a row max

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

__device__ __forceinline__ float other_half(float v)
{
    // value held by lane l ^ 32
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// Workgroup barrier that also orders LDS accesses: the fences keep the
// compiler from moving LDS reads or writes across it (s_barrier alone is not
// a memory operation to the compiler) and cost only an lgkmcnt(0) wait.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait until at most N buffer loads of this wave are outstanding and all LDS
// operations have completed (gfx9 s_waitcnt encoding), then barrier.  Later
// DMA (vmcnt) stays in flight.
template <int N>
__device__ __forceinline__ void wait_vm_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    lds_barrier();
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    const int32_t n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// TAIL: n_kv is not a multiple of the 64-key sub-tile, so one sub-tile per
// query block may reach past the last key (launched only then: the extra
// copy path costs registers).
// two waves per SIMD: with 64-row blocks at head_dim 64 four workgroups fit
// in LDS, otherwise two
template <int D, int BQ, int NB>
constexpr int attn_min_blocks()
{
    return NB != 1 ? 1 : ((BQ == 64 && D == 64) ? 4 : 2);
}

template <int D, int BQ, int BK, bool OF32, int NB, bool TAIL>
__global__ void __launch_bounds__(BQ * 2 / NB, (attn_min_blocks<D, BQ, NB>()))
attn_block_kernel(AttnParams a)
{
    constexpr int NW = BQ / (32 * NB);            // waves, 32*NB query rows each
    // NB: 32-query column blocks per wave
    constexpr int KS = 64;                        // keys per sub-tile (compute and DMA unit)
    constexpr int SUB = BK / KS;                  // sub-tiles per listed key block
    constexpr int CH = D / 8;                     // 16-byte chunks per row
    constexpr int NSB = KS / 32;                  // 32-key MFMA blocks per sub-tile
    constexpr int NDC = D / 16;                   // k-steps of S^T
    constexpr int NDB = D / 32;                   // 32-wide output column blocks
    constexpr int ROWS_PER_KB = 1024 / (D * 2);   // sub-tile rows per 1 KB DMA instruction
    constexpr int SUBTILE_BYTES = KS * D * 2;
    constexpr int DMA_W = SUBTILE_BYTES / 1024 / NW;  // DMA instructions per wave per tensor
    static_assert(SUBTILE_BYTES / 1024 % NW == 0, "DMA split");
    constexpr int KT = NW >= 4 ? 1 : (NW == 2 ? 2 : 4);  // period of the per-lane DMA offset terms

    // double-buffered K and V sub-tiles, as four separate LDS objects: the
    // compiler can then tell the buffer being filled by DMA from the one being
    // read, and does not hold the operand reads until the prefetch lands
    __shared__ __attribute__((aligned(1024))) uint8_t kl0[SUBTILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t kl1[SUBTILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t vl0[SUBTILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t vl1[SUBTILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hh = lane >> 5;  // half-wave
    const int l32 = lane & 31;

    // Longer lists first, so the short workgroups fill the gaps at the end of
    // the launch: under causality rows near the start see the fewest key
    // tiles (query blocks run from the last to the first); without it the
    // long rows are the global-token rows at the start (first to last).
    // With the long-row split, the first split_q query blocks of every head
    // are split_c work items each (list chunks), dispatched before the rest.
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int n_split = (a.batch * a.heads) * a.split_q * a.split_c;
    int qb, bh, chunk = -1;
    if (item < n_split) {
        chunk = item % a.split_c;
        const int t = item / a.split_c;
        qb = t % a.split_q;
        bh = t / a.split_q;
    } else {
        const int j = item - n_split, nrest = a.nqb - a.split_q;
        qb = a.split_q + (a.last_first ? nrest - 1 - j % nrest : j % nrest);
        bh = j / nrest;
    }
    const int b = bh / a.heads, h = bh % a.heads;
    const int nq_h = (a.n_q_rest > 0 && h > 0) ? a.n_q_rest : a.n_q;  // rows of this head

    const uint16_t* qg = a.q + b * a.q_sb + h * a.q_sh;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + b * a.k_sb + h * a.k_sh, (int64_t)a.n_kv * a.k_sn * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + b * a.v_sb + h * a.v_sh, (int64_t)a.n_kv * a.v_sn * 2);
    const uint32_t krow_b = (uint32_t)(a.k_sn * 2);
    const uint32_t vrow_b = (uint32_t)(a.v_sn * 2);

    const int64_t lrow = (a.per_head_lists ? (int64_t)bh * a.nqb : 0) + qb;  // list row of this work item
    // a split item walks list entries [chunk*split_e, chunk*split_e + split_e)
    const int e_first = chunk >= 0 ? chunk * a.split_e : 0;
    const int32_t* idx_row = a.kv_index + lrow * a.nkb + e_first;
    const uint8_t* part_row = a.kv_partial + lrow * a.nkb + e_first;
    int cnt = min(a.kv_count[lrow], a.nkb);
    if (chunk >= 0) cnt = max(0, min(cnt - e_first, a.split_e));
    const int n_sub = cnt * SUB;
    // The live list is held in registers, 64 entries at a time (lane j holds
    // entry base + j) and read with readlane, so the loop issues no memory
    // loads of its own besides the DMA.
    int l_idx = -1, l_part = 0;
    auto refill = [&](int base) {
        const int e = base + lane;
        l_idx = e < cnt ? idx_row[e] : -1;
        l_part = e < cnt ? (int)part_row[e] : 0;
    };
    auto list_at = [](int v, int e) { return __builtin_amdgcn_readlane(v, e & 63); };
    // first key of a sub-tile of list entry j; an entry that is not a key
    // block maps past the sequence end, where the copy reads zeros and the
    // mask drops every key
    auto sub_kv0 = [&](int j, int sub) {
        return ((unsigned)j < (unsigned)a.nkb ? j : a.nkb) * BK + sub * KS;
    };

    // DMA of a sub-tile into buffer slot.  Lane -> (row within its 1 KB
    // group, physical 16-byte chunk); the DMA of group g writes LDS bytes
    // [g*1024, g*1024 + 1024) and fetches rows g*ROWS_PER_KB + dma_r.  The
    // swizzles depend on the row only modulo 4, and a wave's groups advance by
    // NW, so the per-lane offset terms repeat with period KT and are computed
    // once; the uniform parts (sub-tile start, group) go in the scalar offset
    // operand, so the copies need no vector arithmetic or temporaries and
    // issue back to back.
    const int dma_r = lane / CH;
    const int dma_p = lane % CH;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t kterm[4];  // first KT entries used (a fixed bound keeps the host pass happy)
#pragma unroll
    for (int j = 0; j < KT; ++j) {
        const int r = (wave_u + j * NW) * ROWS_PER_KB + dma_r;
        kterm[j] = (uint32_t)dma_r * krow_b + (uint32_t)((dma_p ^ kswz<D>(r)) << 4);
    }
    const uint32_t vterm = (uint32_t)dma_r * vrow_b + (uint32_t)((dma_p ^ vswz<D>(dma_r)) << 4);
    const uint16_t* kbh = a.k + b * a.k_sb + h * a.k_sh;
    const uint16_t* vbh = a.v + b * a.v_sb + h * a.v_sh;
    // A sub-tile that reaches past the last key (a ragged end, or a list
    // entry that is not a key block): the buffer range check covers the
    // per-lane offset but not the scalar one, so these copies take a resource
    // whose base is the sub-tile's first row and whose size stops at n_kv,
    // with the whole row offset in the per-lane operand; rows past n_kv then
    // read as zero and nothing beyond the tensor is touched.
    auto dma_tail = [&](int kv0, uint8_t* kdst, uint8_t* vdst) {
        const int left = max(a.n_kv - kv0, 0);
        const __amdgpu_buffer_rsrc_t ks = make_rsrc(kbh + (int64_t)kv0 * a.k_sn, (int64_t)left * krow_b);
        const __amdgpu_buffer_rsrc_t vs = make_rsrc(vbh + (int64_t)kv0 * a.v_sn, (int64_t)left * vrow_b);
#pragma unroll
        for (int i = 0; i < DMA_W; ++i) {
            const int g = wave_u + i * NW;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ks, (lds_void*)(kdst + g * 1024), 16,
                                                     kterm[i % KT] + (uint32_t)(g * ROWS_PER_KB) * krow_b, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < DMA_W; ++i) {
            const int g = wave_u + i * NW;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vs, (lds_void*)(vdst + g * 1024), 16,
                                                     vterm + (uint32_t)(g * ROWS_PER_KB) * vrow_b, 0, 0, 0);
        }
    };
    auto dma = [&](int kv0, uint8_t* kdst, uint8_t* vdst) {
        // a sub-tile wholly past the last key (a list entry that is not a key
        // block) is not copied: the mask drops every key of it, so the wave
        // skips it without reading its buffer
        if (kv0 >= a.n_kv) return;
        if (TAIL && kv0 + KS > a.n_kv) {
            dma_tail(kv0, kdst, vdst);
            return;
        }
        // every row of the sub-tile exists: one resource per tensor, the
        // uniform row offset in the scalar operand
#pragma unroll
        for (int i = 0; i < DMA_W; ++i) {
            const int g = wave_u + i * NW;
            const uint32_t rows = (uint32_t)(kv0 + g * ROWS_PER_KB);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kdst + g * 1024), 16, kterm[i % KT],
                                                     (int)(rows * krow_b), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < DMA_W; ++i) {
            const int g = wave_u + i * NW;
            const uint32_t rows = (uint32_t)(kv0 + g * ROWS_PER_KB);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vdst + g * 1024), 16, vterm,
                                                     (int)(rows * vrow_b), 0, 0);
        }
    };
    refill(0);
    if (n_sub > 0) dma(sub_kv0(list_at(l_idx, 0), 0), kl0, vl0);

    // Q^T operands: column block nb, lane holds q[row][16*dc + 8*hh + 0..7]
    int qrow[NB];
    bf16x8 qf[NB][NDC];
    RowCtx rc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        qrow[nb] = qb * BQ + wave * 32 * NB + nb * 32 + l32;
        const bool ok = qrow[nb] < nq_h;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (ok) raw = *reinterpret_cast<const u32x4*>(qg + (int64_t)qrow[nb] * a.q_sn + 16 * dc + 8 * hh);
            qf[nb][dc] = __builtin_bit_cast(bf16x8, raw);
        }
        row_ctx(a.pat, qrow[nb] + a.pat.q_offset, rc[nb]);
    }

    f32x16 o[NB][NDB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[nb][db][i] = 0.f;
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = -INFINITY;
        l_run[nb] = 0.f;
    }
    const float c = a.scale_log2;
    bool have_ref = false;  // every row of the wave has a finite reference m

    // V^T transposed-read lane geometry
    const int tg = lane >> 4, tj = lane & 15;
    const int vrow_off = 4 * (tg >> 1) + (tj >> 2);
    const int vcol_off = 16 * (tg & 1) + 4 * (tj & 3);

    // two sub-tiles per trip, so that each copy of the body names its
    // buffers statically (even sub-tiles live in kl0/vl0, odd in kl1/vl1)
    for (int t0 = 0; t0 < n_sub; t0 += 2)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int t = t0 + par;
        if (t >= n_sub) break;
        const uint8_t* kb = par ? kl1 : kl0;
        const uint8_t* vb = par ? vl1 : vl0;
        const int e = t / SUB;
        const int ej = list_at(l_idx, e);
        const int kv0 = sub_kv0(ej, t % SUB);
        const bool need_mask = (unsigned)ej >= (unsigned)a.nkb || list_at(l_part, e) != 0 || kv0 + KS > a.n_kv;

        // sub-tile t has landed in every wave's share; every wave is done with t-1
        wait_vm_barrier<0>();
        if (t + 1 < n_sub) {
            const int e1 = (t + 1) / SUB;
            if (e1 != e && (e1 & 63) == 0) refill(e1);
            dma(sub_kv0(list_at(l_idx, e1), (t + 1) % SUB), par ? kl0 : kl1, par ? vl0 : vl1);
        }

        // K operands of the first two k-steps are requested before anything
        // else, so the LDS latency overlaps the mask-bit arithmetic
        bf16x8 ka[3][NSB];
        auto load_k = [&](bf16x8* dst, int dc) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int r = sb * 32 + l32;
                const int cc = 2 * dc + hh;
                dst[sb] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(kb + r * D * 2 + ((cc ^ kswz<D>(r)) << 4)));
            }
        };
        load_k(ka[0], 0);
        load_k(ka[1], 1);

        // allowed-key bits of partial / clipped sub-tiles, computed before the
        // score registers are live; all ones on full sub-tiles
        uint32_t mbits[NB][NSB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                uint32_t bits = 0xFFFFFFFFu;
                if (need_mask) {
                    const int32_t k0 = kv0 + sb * 32;
                    bits = allowed_bits32(a.pat, rc[nb], k0);
                }
                // accumulator element i holds key k0 + 8*(i/4) + 4*hh + i%4
                mbits[nb][sb] = bits >> (4 * hh);
            }
        bool apply_mask = need_mask;
        if (need_mask) {
            // no row of this wave may see a key of the sub-tile: every score
            // would be -inf and add nothing, so the wave skips the sub-tile;
            // every row may see every key: no element mask is needed
            uint32_t any = 0, all = 0x0F0F0F0Fu;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    any |= mbits[nb][sb];
                    all &= mbits[nb][sb];
                }
            if (__builtin_amdgcn_ballot_w64(any != 0) == 0) continue;
            apply_mask = __builtin_amdgcn_ballot_w64(all != 0x0F0F0F0Fu) != 0;
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- S^T = K Q^T  (K operands fetched two k-steps ahead)
        __builtin_amdgcn_s_setprio(2);
        f32x16 s[NB][NSB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[nb][sb][i] = 0.f;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
            if (dc + 2 < NDC) load_k(ka[(dc + 2) % 3], dc + 2);

#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    s[nb][sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc % 3][sb], qf[nb][dc], s[nb][sb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        __builtin_amdgcn_s_setprio(0);
        // V^T operands of the first two P.V steps are requested now; they
        // land while the softmax runs
        bf16x8 va[3][NDB];
        auto load_v = [&](bf16x8* dst, int step) {
            const int r0 = (step >> 1) * 32 + 16 * (step & 1) + vrow_off;
            const int r1 = r0 + 8;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int col = 32 * db + vcol_off;
                const int ch = col >> 3, within = (col & 7) * 2;
                const bf16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(vb + r0 * D * 2 + ((ch ^ vswz<D>(r0)) << 4) + within));
                const bf16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(vb + r1 * D * 2 + ((ch ^ vswz<D>(r1)) << 4) + within));
                dst[db] = bf16x8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
            }
        };
        load_v(va[0], 0);
        load_v(va[1], 1);
        __builtin_amdgcn_sched_barrier(0);

        __builtin_amdgcn_s_setprio(1);
        // ---- element mask on partial / clipped sub-tiles only
        if (apply_mask) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                    {
                        // keep = all ones where the key is allowed (one bit-field
                        // extract), then a bit-select against -inf
                        const int32_t keep = __builtin_amdgcn_sbfe((int32_t)mbits[nb][sb], 8 * (i >> 2) + (i & 3), 1);
                        s[nb][sb][i] = __int_as_float((__float_as_int(s[nb][sb][i]) & keep) |
                                                      (int32_t(0xFF800000u) & ~keep));
                    }
        }

        // ---- online softmax, one query per lane and column block; P packed to bf16.
        // p = exp2(s*c - m*c) against the row's reference m.  While every row of
        // the wave has a reference and no lane's sum over the sub-tile exceeds
        // kSumLimit, the sub-tile needs no row max; otherwise the exact max is
        // taken, the accumulator rescaled to it and P recomputed.
        bf16x8 pk[NB][NSB][2];
        float lt[NB];
        auto exps = [&](int nb) {
            const float mc = m_run[nb] == -INFINITY ? 0.f : m_run[nb] * c;
            float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four partial row sums
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][sb][8 * cb + u], c, -mc));
                        ls[u & 3] += p;
                        pk[nb][sb][cb][u] = (__bf16)p;
                    }
            lt[nb] = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        };
        bool exact = !have_ref;
        if (!exact) {
            bool over = false;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                exps(nb);
                over |= lt[nb] > kSumLimit;
            }
            exact = __builtin_amdgcn_ballot_w64(over) != 0;
        }
        if (exact) {
            bool unset = false;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                // row max as a tree (exact in any order): short dependency chains
                float mq[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) mq[x] = fmaxf(s[nb][0][4 * x], s[nb][0][4 * x + 1]);
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int i = (sb == 0 ? 2 : 0); i < 4; ++i)
#pragma unroll
                        for (int x = 0; x < 4; ++x) mq[x] = fmaxf(mq[x], s[nb][sb][4 * x + i]);
                float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
                mx = fmaxf(mx, other_half(mx));
                const float m_new = fmaxf(m_run[nb], mx);
                if (__any(m_new > m_run[nb])) {
                    const float alpha =
                        m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run[nb] - m_new) * c);
                    l_run[nb] *= alpha;
                    // one 16-register accumulator block at a time keeps the
                    // temporaries of this rarely taken path small
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) o[nb][db][i] *= alpha;
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    m_run[nb] = m_new;
                }
                exps(nb);
                unset |= m_run[nb] == -INFINITY;
            }
            have_ref = __builtin_amdgcn_ballot_w64(unset) == 0;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) l_run[nb] += lt[nb];

        // ---- O^T += V^T P^T  (V^T operands fetched two steps ahead)
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int step = 0; step < 2 * NSB; ++step) {
            if (step + 2 < 2 * NSB) load_v(va[(step + 2) % 3], step + 2);
            const int sb = step >> 1, cb = step & 1;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    o[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[step % 3][db], pk[nb][sb][cb], o[nb][db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // ---- epilogue
    if (chunk >= 0) {
        // a list chunk of a split row: normalised partial O and its LSE
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float l_tot = l_run[nb] + other_half(l_run[nb]);
            const int r = qrow[nb] - qb * BQ;  // row within the block
            const int64_t slot = (((int64_t)bh * a.split_q + qb) * a.split_c + chunk) * BQ + r;
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            float* op = a.part_o + slot * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int dv = 32 * db + 8 * r4 + 4 * hh;
                    *reinterpret_cast<float4*>(op + dv) =
                        make_float4(o[nb][db][4 * r4 + 0] * inv, o[nb][db][4 * r4 + 1] * inv,
                                    o[nb][db][4 * r4 + 2] * inv, o[nb][db][4 * r4 + 3] * inv);
                }
            if (hh == 0) a.part_lse[slot] = l_tot > 0.f ? m_run[nb] * a.scale + logf(l_tot) : -INFINITY;
        }
        return;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l_tot = l_run[nb] + other_half(l_run[nb]);
        if (qrow[nb] < nq_h) {
            float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            const float lse = l_tot > 0.f ? m_run[nb] * a.scale + logf(l_tot) : -INFINITY;
            const int64_t obase = b * a.o_sb + h * a.o_sh + (int64_t)qrow[nb] * a.o_sn;
            float* lp = a.lse ? a.lse + b * a.lse_sb + h * a.lse_sh + (int64_t)qrow[nb] * a.lse_sn : nullptr;
            // Merge mode: O and LSE already hold this row's attention over a
            // disjoint key set; fold this part in with log-sum-exp weights,
            // O = (e^l1 O1 + e^l2 O2) / (e^l1 + e^l2), LSE = log(e^l1 + e^l2).
            // A part without keys leaves the row as it is.
            float w1 = 0.f, lse_out = lse;
            bool write = true;
            if (OF32 && a.merge) {
                const float l1 = *lp;
                write = lse != -INFINITY;
                if (write && l1 != -INFINITY) {
                    const float m = fmaxf(l1, lse);
                    const float e1 = __expf(l1 - m), e2 = __expf(lse - m);
                    const float rs = 1.f / (e1 + e2);
                    lse_out = m + logf(e1 + e2);
                    w1 = e1 * rs;
                    inv *= e2 * rs;
                }
            }
            if (write) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int dv = 32 * db + 8 * r4 + 4 * hh;
                        float x0 = o[nb][db][4 * r4 + 0] * inv, x1 = o[nb][db][4 * r4 + 1] * inv;
                        float x2 = o[nb][db][4 * r4 + 2] * inv, x3 = o[nb][db][4 * r4 + 3] * inv;
                        if (OF32) {
                            float* op = reinterpret_cast<float*>(a.o) + obase + dv;
                            if (w1 != 0.f) {
                                const float4 o1 = *reinterpret_cast<const float4*>(op);
                                x0 += w1 * o1.x;
                                x1 += w1 * o1.y;
                                x2 += w1 * o1.z;
                                x3 += w1 * o1.w;
                            }
                            *reinterpret_cast<float4*>(op) = make_float4(x0, x1, x2, x3);
                        } else {
                            uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + obase + dv;
                            const bf16x2 p01 = {(__bf16)x0, (__bf16)x1};
                            const bf16x2 p23 = {(__bf16)x2, (__bf16)x3};
                            const u32x2 w = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
                            *reinterpret_cast<u32x2*>(op) = w;
                        }
                    }
                if (lp && hh == 0) *lp = lse_out;
            }
        }
    }
}

template <int D, int BQ, int BK, bool OF32>
hipError_t launch_one(const AttnParams& a, hipStream_t stream)
{
    // one 32-query column block per wave at both head dims (two per wave ran
    // 15-36 % slower at head_dim 64)
    constexpr int NB = 1;
    const int64_t items = (int64_t)a.batch * a.heads * (a.nqb - a.split_q + (int64_t)a.split_q * a.split_c);
    if (a.n_kv % 64)
        hipLaunchKernelGGL((attn_block_kernel<D, BQ, BK, OF32, NB, true>), dim3((unsigned)items), dim3(BQ * 2 / NB), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((attn_block_kernel<D, BQ, BK, OF32, NB, false>), dim3((unsigned)items), dim3(BQ * 2 / NB),
                           0, stream, a);
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

// Long-row split, second pass: one wave per split row folds its chunks'
// partial (O, LSE) into the row's O and LSE with log-sum-exp weights,
// O = sum_c e^(l_c - L) O_c, L = log sum_c e^(l_c); chunks without keys
// (l_c = -inf) weigh nothing, a row without any key gets O = 0, L = -inf.
template <int D, bool OF32>
__global__ void __launch_bounds__(256) split_merge_kernel(AttnParams a, int32_t bq)
{
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t rows = (int64_t)a.batch * a.heads * a.split_q * bq;
    if (w >= rows) return;
    const int r = (int)(w % bq);
    const int64_t t = w / bq;
    const int qb = (int)(t % a.split_q), bh = (int)(t / a.split_q);
    const int q = qb * bq + r;
    if (q >= a.n_q) return;
    const int b = bh / a.heads, h = bh % a.heads;
    const int64_t slot0 = ((int64_t)bh * a.split_q + qb) * a.split_c * bq + r;  // chunk c at slot0 + c*bq
    // chunk weights, 64 chunks at a time: lane c holds chunk c0 + c
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    const int64_t obase = b * a.o_sb + h * a.o_sh + (int64_t)q * a.o_sn;
    if (a.split_c <= 64) {
        // Up to 64 chunks: one LSE per lane, and the partial O of the first
        // PF chunks requested together with it, so the row costs one memory
        // round trip before its arithmetic instead of three.  32 covers the
        // chunks of 8 list entries of a 256-block row in that one trip (16:
        // W4 134.3 -> 130.6 us with 32, same sums in the same order).
        constexpr int PF = 32;
        const int nc = a.split_c;
        const float* po = a.part_o + slot0 * D + lane;
        const float lv = lane < nc ? a.part_lse[slot0 + (int64_t)lane * bq] : -INFINITY;
        float ob[PF][PER];
#pragma unroll
        for (int c = 0; c < PF; ++c)
#pragma unroll
            for (int i = 0; i < PER; ++i) ob[c][i] = c < nc ? po[(int64_t)c * bq * D + 64 * i] : 0.f;
        float m = lv;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        const float wl = m != -INFINITY ? __expf(lv - m) : 0.f;  // 0 for a chunk without keys
        float s = wl;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
#pragma unroll
        for (int c = 0; c < PF; ++c) {
            const float wc = __shfl(wl, c);
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] += wc * ob[c][i];
        }
        for (int c0 = PF; c0 < nc; c0 += PF) {
#pragma unroll
            for (int c = 0; c < PF; ++c)
#pragma unroll
                for (int i = 0; i < PER; ++i) ob[c][i] = c0 + c < nc ? po[(int64_t)(c0 + c) * bq * D + 64 * i] : 0.f;
#pragma unroll
            for (int c = 0; c < PF; ++c) {
                const float wc = __shfl(wl, c0 + c);
#pragma unroll
                for (int i = 0; i < PER; ++i) acc[i] += wc * ob[c][i];
            }
        }
        const float inv = s > 0.f ? 1.f / s : 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const float x = acc[i] * inv;
            if (OF32) reinterpret_cast<float*>(a.o)[obase + lane + 64 * i] = x;
            else reinterpret_cast<uint16_t*>(a.o)[obase + lane + 64 * i] = __builtin_bit_cast(uint16_t, (__bf16)x);
        }
        if (a.lse && lane == 0)
            a.lse[b * a.lse_sb + h * a.lse_sh + (int64_t)q * a.lse_sn] = s > 0.f ? m + logf(s) : -INFINITY;
        return;
    }
    float m = -INFINITY;
    for (int c0 = 0; c0 < a.split_c; c0 += 64)
        if (c0 + lane < a.split_c) m = fmaxf(m, a.part_lse[slot0 + (int64_t)(c0 + lane) * bq]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float s = 0.f;
    if (m != -INFINITY) {
        for (int c0 = 0; c0 < a.split_c; c0 += 64) {
            const int nc = min(64, a.split_c - c0);
            const float wl = lane < nc ? __expf(a.part_lse[slot0 + (int64_t)(c0 + lane) * bq] - m) : 0.f;
            float ws = wl;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off);
            s += ws;
            const float* po = a.part_o + (slot0 + (int64_t)c0 * bq) * D + lane;
#pragma unroll 8
            for (int c = 0; c < nc; ++c) {
                const float wc = __shfl(wl, c);  // 0 for a chunk without keys
#pragma unroll
                for (int i = 0; i < PER; ++i) acc[i] += wc * po[(int64_t)c * bq * D + 64 * i];
            }
        }
    }
    const float inv = s > 0.f ? 1.f / s : 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float x = acc[i] * inv;
        if (OF32) reinterpret_cast<float*>(a.o)[obase + lane + 64 * i] = x;
        else reinterpret_cast<uint16_t*>(a.o)[obase + lane + 64 * i] = __builtin_bit_cast(uint16_t, (__bf16)x);
    }
    if (a.lse && lane == 0)
        a.lse[b * a.lse_sb + h * a.lse_sh + (int64_t)q * a.lse_sn] = s > 0.f ? m + logf(s) : -INFINITY;
}

}  // namespace

hipError_t launch_split_merge(const AttnParams& a, int head_dim, int block_q, int o_f32, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.heads * a.split_q * block_q;
    if (rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (head_dim == 128) {
        if (o_f32) hipLaunchKernelGGL((split_merge_kernel<128, true>), grid, dim3(256), 0, stream, a, block_q);
        else hipLaunchKernelGGL((split_merge_kernel<128, false>), grid, dim3(256), 0, stream, a, block_q);
    } else {
        if (o_f32) hipLaunchKernelGGL((split_merge_kernel<64, true>), grid, dim3(256), 0, stream, a, block_q);
        else hipLaunchKernelGGL((split_merge_kernel<64, false>), grid, dim3(256), 0, stream, a, block_q);
    }
    return hipGetLastError();
}

hipError_t launch_attn_blocks(const AttnParams& a, int head_dim, int block_q, int block_kv,
                              int o_f32, hipStream_t stream)
{
    if (head_dim == 128) return launch_d<128>(a, block_q, block_kv, o_f32, stream);
    if (head_dim == 64) return launch_d<64>(a, block_q, block_kv, o_f32, stream);
    return hipErrorInvalidValue;
}

}  // namespace sa
