// Dynamic block selection for block-sparse attention: TopK / TopP over mean-pooled block
// scores (the selection criterion that "LongCA-bench: 长上下文注意力基准测试" names for
// dynamic block-sparse attention; the page gives no formula, the definition used here is
// stated in attn.h at attn_block_select).
//
//   1. pool_kernel          block means of Q and K in fp32          HBM-bound (reads Q, K once)
//   2. block_score_kernel   s = scale * Qbar Kbar^T per KV group, fp32 FMA, 64 x 64 tiles
//   3. block_select_kernel  per (head, query block): sort the row by (score desc, index
//                           asc) with a bitonic sort in LDS, then keep the first k entries
//                           (TopK) or the shortest prefix whose softmax mass reaches p (TopP)
//
// Every score is a sequential fp32 FMA chain over the 128 dimensions, so the scores (and
// the selection, which only compares them) are deterministic.
#include <mutex>

#include "common.h"

namespace mlct {

// out[h][blk][d] = mean of x[pos][h][d] over the rows of block blk. 16 heads x 128 dims
// per workgroup pass, 8 dims per thread; rows are summed in ascending order.
__global__ __launch_bounds__(256) void pool_kernel(const bf16* __restrict__ x, int T, int H, int b, int nb,
                                                   float* __restrict__ out) {
    const int hl = threadIdx.x >> 4, part = threadIdx.x & 15;
    const int h = blockIdx.y * 16 + hl, blk = blockIdx.x;
    if (h >= H) return;
    const int r0 = blk * b, r1 = min(T, r0 + b);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const bf16* p = x + ((size_t)r0 * H + h) * HEAD_DIM + 8 * part;
    const size_t row = (size_t)H * HEAD_DIM;
    int pos = r0;
    for (; pos + 4 <= r1; pos += 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const u32x4*>(p + (size_t)(pos - r0 + u) * row);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                acc[2 * m] += bf16_lo(v[u][m]);
                acc[2 * m + 1] += bf16_hi(v[u][m]);
            }
    }
    for (; pos < r1; ++pos) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p + (size_t)(pos - r0) * row);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            acc[2 * m] += bf16_lo(v[m]);
            acc[2 * m + 1] += bf16_hi(v[m]);
        }
    }
    const float n = (float)(r1 - r0);
    float* o = out + ((size_t)h * nb + blk) * HEAD_DIM + 8 * part;
    f32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = acc[e] / n;
        hi[e] = acc[4 + e] / n;
    }
    *reinterpret_cast<f32x4*>(o) = lo;
    *reinterpret_cast<f32x4*>(o + 4) = hi;
}

// scores[g*G*nb + ra][kb] = scale * sum_d qbar[g*G*nb + ra][d] * kbar[g*nb + kb][d] for the
// 64 x 64 tile (ra0.., kb0..) of KV group g: the G heads' query blocks of the group are
// consecutive rows of qbar [Hq][nb][128], and consecutive rows of scores [Hq][nb][nb].
// Operands staged d-major in LDS; every thread computes a 4 x 4 patch.
constexpr int SC_LD = 64 + 4;
__global__ __launch_bounds__(256) void block_score_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar, float* __restrict__ scores,
                                                          int nb, int G, float scale) {
    __shared__ __attribute__((aligned(16))) float As[HEAD_DIM * SC_LD];
    __shared__ __attribute__((aligned(16))) float Bs[HEAD_DIM * SC_LD];
    const int t = threadIdx.x;
    const int g = blockIdx.z, kb0 = blockIdx.x * 64, ra0 = blockIdx.y * 64;
    const int rows = G * nb;
    const float* qg = qbar + (size_t)g * rows * HEAD_DIM;
    const float* kg = kbar + (size_t)g * nb * HEAD_DIM;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = t & 63, d0 = 4 * ((t >> 6) + 4 * i);
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, bv = {0.f, 0.f, 0.f, 0.f};
        if (ra0 + r < rows) a = *reinterpret_cast<const f32x4*>(qg + (size_t)(ra0 + r) * HEAD_DIM + d0);
        if (kb0 + r < nb) bv = *reinterpret_cast<const f32x4*>(kg + (size_t)(kb0 + r) * HEAD_DIM + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            As[(d0 + e) * SC_LD + r] = a[e];
            Bs[(d0 + e) * SC_LD + r] = bv[e];
        }
    }
    __syncthreads();
    const int ty = t >> 4, tx = t & 15;
    float c[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[i][j] = 0.f;
#pragma unroll 8
    for (int d = 0; d < HEAD_DIM; ++d) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&As[d * SC_LD + 4 * ty]);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&Bs[d * SC_LD + 4 * tx]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[i][j] = fmaf(a[i], bv[j], c[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = ra0 + 4 * ty + i;
        if (ra >= rows) continue;
        float* srow = scores + ((size_t)g * rows + ra) * nb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kb = kb0 + 4 * tx + j;
            if (kb < nb) srow[kb] = c[i][j] * scale;
        }
    }
}

// Order-preserving map of a float to an unsigned integer (a < b <=> key(a) < key(b)).
__device__ __forceinline__ uint32_t float_order(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One (head, query block) row per workgroup. Sort key = (~order(score)) << 32 | kb, so the
// ascending sort puts high scores first and equal scores by ascending kb; the forced
// diagonal gets key kb (high word 0), below every score's key; padding sorts last.
__global__ __launch_bounds__(256) void block_select_kernel(const float* __restrict__ scores, uint8_t* __restrict__ keep,
                                                           int nb, int P, int mode, int topk, float topp,
                                                           int keep_diag) {
    __shared__ unsigned long long keys[SEL_MAX_NB];
    __shared__ float part[256];
    __shared__ float red[4];
    const int t = threadIdx.x;
    const size_t row = blockIdx.x;
    const int qb = (int)(row % nb);
    const float* s = scores + row * nb;
    uint8_t* kp = keep + row * nb;

    float mx = -INFINITY;
    for (int i = t; i < P; i += 256) {
        unsigned long long key = ~0ull;
        if (i < nb) {
            const float v = s[i];
            mx = fmaxf(mx, v);
            key = (keep_diag && i == qb) ? (unsigned long long)i
                                         : ((unsigned long long)(~float_order(v)) << 32) | (unsigned)i;
        }
        keys[i] = key;
    }
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < P; i += 256) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const unsigned long long a = keys[i], b = keys[ixj];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        keys[i] = b;
                        keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }

    if (mode == ATTN_SELECT_TOPK) {
        for (int i = t; i < nb; i += 256) kp[(unsigned)keys[i]] = i < topk ? 1 : 0;
        return;
    }

    // TopP: softmax mass of the sorted entries, exclusive prefix sums in a fixed order
    // (each thread a run of P / 256 consecutive entries, then a scan of the run totals).
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int run = P / 256 > 0 ? P / 256 : 1;
    const int i0 = t * run;
    float local = 0.f;
    for (int i = i0; i < i0 + run && i < nb; ++i) local += expf(s[(unsigned)keys[i]] - mx);
    part[t] = local;
    __syncthreads();
    if (t == 0) {
        float acc = 0.f;
        for (int u = 0; u < 256; ++u) {
            const float x = part[u];
            part[u] = acc;
            acc += x;
        }
        red[0] = acc;
    }
    __syncthreads();
    const float target = topp * red[0];
    float before = part[t];
    for (int i = i0; i < i0 + run && i < nb; ++i) {
        const unsigned kb = (unsigned)keys[i];
        kp[kb] = before < target ? 1 : 0;
        before += expf(s[kb] - mx);
    }
}

int launch_block_select(const Problem& P, int mode, int topk, float topp, int keep_diag, const void* q,
                        const void* k, float* scores, uint8_t* keep, void* ws, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* qbar = static_cast<float*>(ws);
    float* kbar = reinterpret_cast<float*>(static_cast<char*>(ws) + select_qbar_bytes(P));
    const int b = P.sblock, nb = P.nb;
    hipLaunchKernelGGL(pool_kernel, dim3(nb, (P.Hq + 15) / 16), dim3(256), 0, s, static_cast<const bf16*>(q), P.T,
                       P.Hq, b, nb, qbar);
    hipLaunchKernelGGL(pool_kernel, dim3(nb, (P.Hk + 15) / 16), dim3(256), 0, s, static_cast<const bf16*>(k), P.T,
                       P.Hk, b, nb, kbar);
    hipLaunchKernelGGL(block_score_kernel, dim3((nb + 63) / 64, (P.G * nb + 63) / 64, P.Hk), dim3(256), 0, s, qbar,
                       kbar, scores, nb, P.G, P.scale);
    int Pp = 1;
    while (Pp < nb) Pp <<= 1;
    hipLaunchKernelGGL(block_select_kernel, dim3((unsigned)((size_t)P.Hq * nb)), dim3(256), 0, s, scores, keep, nb,
                       Pp, mode, topk, topp, keep_diag);
    return (int)hipGetLastError();
}

// Workspace of attn_block_select_noalloc: one static array on every GPU the library runs on.
// In host code the array's name stands for a host-side shadow, so its device address is
// looked up (hipGetSymbolAddress) once per device, with that device current, and only that
// address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[SEL_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex scratch_mu;
static void* scratch_dev[SCRATCH_MAX_DEVICES];

static hipError_t scratch_address(hipStream_t s, void** out) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (s != nullptr && (e = hipStreamGetDevice(s, &dev)) != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return hipSuccess;
}

int launch_block_select_scratch(const Problem& P, int mode, int topk, float topp, int keep_diag, const void* q,
                                const void* k, float* scores, uint8_t* keep, void* stream) {
    void* ws = nullptr;
    const hipError_t e = scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (e != hipSuccess) return (int)e;
    return launch_block_select(P, mode, topk, topp, keep_diag, q, k, scores, keep, ws, stream);
}

}  // namespace mlct
