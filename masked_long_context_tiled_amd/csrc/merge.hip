// Merge of two partial attention results over disjoint key sets (one step of a
// context-parallel ring): with weights w = exp(LSE - max(LSE_acc, LSE_part)),
//   O   = (w_acc O_acc + w_part O_part) / (w_acc + w_part)
//   LSE = max(LSE_acc, LSE_part) + ln(w_acc + w_part)
// which is the attention over the union of the two key sets. A side with LSE = -inf (no
// visible key) has weight 0; if both are -inf the row stays O = 0, LSE = -inf.
// O values are bf16 plus an optional bf16 residual (O + O_lo carries the fp32 result).
// HBM-bound: 16 lanes per (position, head) row, 8 elements per lane.
#include "common.h"

namespace mlct {

__global__ __launch_bounds__(256) void lse_merge_kernel(bf16* __restrict__ o, bf16* __restrict__ o_lo,
                                                        float* __restrict__ lse, const bf16* __restrict__ op,
                                                        const bf16* __restrict__ op_lo,
                                                        const float* __restrict__ lsep, int T, int Hq) {
    const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);   // row = pos * Hq + head
    const int part = threadIdx.x & 15;
    if (row >= (long)T * Hq) return;
    const int pos = (int)(row / Hq), head = (int)(row % Hq);
    const size_t li = (size_t)head * T + pos;
    const float la = lse[li], lp = lsep[li];
    const float m = fmaxf(la, lp);
    float wa = 0.f, wp = 0.f, lout = -INFINITY;
    if (m != -INFINITY) {
        wa = __expf(la - m);   // exp(-inf) = 0
        wp = __expf(lp - m);
        lout = m + __logf(wa + wp);
        const float inv = 1.f / (wa + wp);
        wa *= inv;
        wp *= inv;
    }
    const size_t off = (size_t)row * HEAD_DIM + part * 8;
    const u32x4 xa = *reinterpret_cast<const u32x4*>(o + off);
    const u32x4 xp = *reinterpret_cast<const u32x4*>(op + off);
    u32x4 ya = {0u, 0u, 0u, 0u}, yp = {0u, 0u, 0u, 0u};
    if (o_lo) ya = *reinterpret_cast<const u32x4*>(o_lo + off);
    if (op_lo) yp = *reinterpret_cast<const u32x4*>(op_lo + off);
    u32x4 hi, lo;
#pragma unroll
    for (int m2 = 0; m2 < 4; ++m2) {
        const float v0 = wa * (bf16_lo(xa[m2]) + bf16_lo(ya[m2])) + wp * (bf16_lo(xp[m2]) + bf16_lo(yp[m2]));
        const float v1 = wa * (bf16_hi(xa[m2]) + bf16_hi(ya[m2])) + wp * (bf16_hi(xp[m2]) + bf16_hi(yp[m2]));
        hi[m2] = pack_bf16(v0, v1);
        lo[m2] = pack_bf16(v0 - bf16_lo(hi[m2]), v1 - bf16_hi(hi[m2]));
    }
    *reinterpret_cast<u32x4*>(o + off) = hi;
    if (o_lo) *reinterpret_cast<u32x4*>(o_lo + off) = lo;
    // every lane of the row has read lse[li] before lane 0 writes it (the 16 lanes of a
    // row sit in one wave and execute in lock step)
    if (part == 0) lse[li] = lout;
}

int launch_lse_merge(const Problem& P, void* o, void* o_lo, float* lse, const void* o_part,
                     const void* o_part_lo, const float* lse_part, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long rows = (long)P.T * P.Hq;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s,
                       static_cast<bf16*>(o), static_cast<bf16*>(o_lo), lse, static_cast<const bf16*>(o_part),
                       static_cast<const bf16*>(o_part_lo), lse_part, P.T, P.Hq);
    return (int)hipGetLastError();
}

}  // namespace mlct
