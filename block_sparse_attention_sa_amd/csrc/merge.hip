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
// D/4 threads per row, four columns each (16-byte loads and stores), so a
// wave covers 64*4/D rows and every row costs one request per operand.
// The second partial's LSE may be stored in residue order (see MergeParams).
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ void __launch_bounds__(kThreads) merge_kernel(MergeParams p)
{
    constexpr int TPR = D / 4;                 // threads per row
    constexpr int RPB = kThreads / TPR;        // rows per workgroup
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = (threadIdx.x % TPR) * 4;
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
    float4* o = reinterpret_cast<float4*>(p.o + b * p.o_sb + h * p.o_sh + q * p.o_sn + c);
    const float4 x2 = *reinterpret_cast<const float4*>(p.o2 + b * p.o2_sb + h * p.o2_sh + q * p.o2_sn + c);
    const float4 x1 = *o;
    *o = make_float4((x1.x * w1 + x2.x * w2) * inv, (x1.y * w1 + x2.y * w2) * inv,
                     (x1.z * w1 + x2.z * w2) * inv, (x1.w * w1 + x2.w * w2) * inv);
    if (c == 0) p.lse[row] = m + logf(w1 + w2);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t stream)
{
    const int64_t rpb = kThreads / (head_dim / 4);
    const unsigned grid = (unsigned)((p.rows + rpb - 1) / rpb);
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, p);
    else if (head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sa
