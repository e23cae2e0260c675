// lse_merge.hip -- combine split partial results by logsumexp, gfx950.
//
// Each partial i of a row is (O_i normalised over its key subset, LSE_i);
// the subsets are disjoint, so the row's result is LSE = ln sum_i exp(LSE_i)
// and O = sum_i exp(LSE_i - LSE) O_i; an empty subset carries LSE_i = -inf and
// contributes nothing (split-KV of the flash-sparse-attn page; the Ascend SFA
// blog's decode-reduction core).  One wave per row.
#include "fsa_common.h"
#include "fsa_params.h"

namespace fsa {


template <int D>
__global__ void __launch_bounds__(256) lse_merge_kernel(const MergeParams p) {
    constexpr int DPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.nrows) return;
    if (p.ntok_live != nullptr && row / p.Hq >= (int64_t)*p.ntok_live) return;
    float m = -INFINITY;
    for (int i = lane; i < p.nparts; i += 64) m = fmaxf(m, p.part_lse[(int64_t)i * p.nrows + row]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float o_acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) o_acc[x] = 0.f;
    float L = -INFINITY;
    if (m != -INFINITY) {
        float s = 0.f;
        for (int i = lane; i < p.nparts; i += 64) s += __expf(p.part_lse[(int64_t)i * p.nrows + row] - m);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
        L = m + __logf(s);
        for (int i = 0; i < p.nparts; ++i) {
            const float li = p.part_lse[(int64_t)i * p.nrows + row];
            if (li == -INFINITY) continue;
            const float wgt = __expf(li - L);
            const float* po = p.part_o + ((int64_t)i * p.nrows + row) * D + lane * DPL;
#pragma unroll
            for (int x = 0; x < DPL; ++x) o_acc[x] = fmaf(wgt, po[x], o_acc[x]);
        }
    }
    uint16_t* o = p.out + row * D + lane * DPL;
    if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(o_acc[0], o_acc[1]);
    } else {
        const __bf16 h = (__bf16)o_acc[0];
        *o = __builtin_bit_cast(uint16_t, h);
    }
    if (p.lse != nullptr && lane == 0) {
        const int64_t li = p.lse_mode == 0 ? (row % p.Hq) * p.ntok + row / p.Hq : row;
        p.lse[li] = L;
    }
}

hipError_t launch_lse_merge(const MergeParams& p, int D, hipStream_t stream) {
    const dim3 grid((unsigned)((p.nrows + 3) / 4));
    if (D == 64)
        hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fsa
