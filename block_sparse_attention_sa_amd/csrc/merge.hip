// merge.hip -- fold a second partial attention result into a first one.
//
// When the allowed keys of every query row are split into two disjoint sets,
// softmax attention over their union is the two partial results weighted by
// exp(LSE): O = (e^l1 O1 + e^l2 O2) / (e^l1 + e^l2), LSE = log(e^l1 + e^l2)
// (plain log-sum-exp algebra on the masked softmax of the blog "Sparse
// transformers: how to cut the O(n^2) of attention", section on how it looks
// in code).  The strided template of that blog (section on the main sparsity
// templates: near neighbours plus positions at a fixed step) splits this way
// into its local band and its strided keys.
//
// One wave per row (b, h, q); lanes own columns lane + 64 j, so every load
// and store of a row is one coalesced 256-byte access per j.  The second
// partial's LSE may be stored in residue order (see MergeParams).
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 4;

template <int D>
__global__ void __launch_bounds__(kWaves * 64) merge_kernel(MergeParams p)
{
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (row >= p.rows) return;
    const int64_t q = row % p.n;
    const int64_t bh = row / p.n;
    if (q < p.q_first) return;  // no second partial: unchanged
    const int64_t r = (q - p.q_first) % p.group, i = (q - p.q_first) / p.group;
    if (i >= p.n2) return;
    const int64_t b = bh / p.heads, h = bh % p.heads;
    const float l2 = p.lse2[(bh * p.group + r) * p.n2 + i];
    const float l1 = p.lse[row];
    const float m = fmaxf(l1, l2);
    if (m == -INFINITY) return;  // neither part has a key: O stays 0, LSE -inf
    const float w1 = l1 == -INFINITY ? 0.f : expf(l1 - m);
    const float w2 = l2 == -INFINITY ? 0.f : expf(l2 - m);
    const float inv = 1.f / (w1 + w2);
    float* o = p.o + b * p.o_sb + h * p.o_sh + q * p.o_sn;
    const float* o2 = p.o2 + b * p.o2_sb + h * p.o2_sh + q * p.o2_sn;
    float x1[PER], x2[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        x1[j] = o[lane + 64 * j];
        x2[j] = o2[lane + 64 * j];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) o[lane + 64 * j] = (x1[j] * w1 + x2[j] * w2) * inv;
    if (lane == 0) p.lse[row] = m + logf(w1 + w2);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t stream)
{
    const unsigned grid = (unsigned)((p.rows + kWaves - 1) / kWaves);
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
    else if (head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sa
