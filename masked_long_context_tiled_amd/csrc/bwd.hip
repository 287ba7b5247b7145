// Masked attention backward for gfx950.
//
//   D_i  = sum_c dO[i, c] O[i, c]                              (bwd_pre_kernel, HBM-bound)
//   P    = exp(scale * Q K^T - LSE)  on the non-empty tiles    (recomputed)
//   dV  += P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//   dK  += scale * dS^T Q,  dQ += scale * dS K                 (bwd_kernel)
//
// Work item = one workgroup = 32 * NW keys of one KV head. Each wave keeps its 32 keys'
// K and V rows in registers (B operands of S and dP) and accumulates dK^T, dV^T for them
// over every non-empty query tile of the key tile's list and every query head of the
// group, so dK and dV are written once, without atomics. Query rows are processed 32 at a
// time, the next block's Q and dO prefetched into registers while the current one
// computes: they are staged in LDS in natural layout (A operands of S and dP) and
// transposed (A operands of dK^T and dV^T). S is computed untransposed, so P and dS come
// out of the accumulators already in the B-operand layout of the dK^T/dV^T products. dS
// goes through LDS once more for dQ = dS K (K^T staged once per work item); each row
// block's dQ partial is added to the fp32 output with hardware float atomics.
//
// Precision. S and dP use the bf16 inputs as they are. The three gradient products
// (P^T dO, dS^T Q, dS K) take fp16 operands: fp16 carries 11 significant bits against
// bf16's 8, which cuts the rounding of P and dS by 8x. To keep every fp16 operand inside
// fp16's range, dO, Q and K are multiplied by powers of two chosen from bounds measured in
// the preprocess (max |Q|, max |K|, max ||dO_i||, max ||V_j||; |dS_ij| <= 2 ||dO_i||
// max_j ||V_j|| bounds dS), and the scales are divided out of the fp32 results.
// D uses O plus its low half O_lo when the forward wrote one, i.e. the forward's fp32 O.
#include "common.h"

namespace mlct {

constexpr int QS_LD = HEAD_DIM + 8;   // bf16 per Q / dO row in LDS
constexpr int QT_LD = 32 + 8;         // fp16 per Q^T / dO^T row (32 query rows + pad)
enum { ST_DO_NORM2 = 0, ST_V_NORM2 = 1, ST_Q_ABS = 2, ST_K_ABS = 3 };

struct BwdArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const bf16* dout;
    const float* lse;
    const float* dbuf;    // D [Hq][T]
    const float* stats;   // BWD_STATS bounds
    float* dq;
    float* dk;
    float* dv;
    const int4* desc;
    const int* ptr;
    const int* ent;
    const int* order;
    int T, Hq, Hk, G, BMq, lgBMq, nb, sblock;
    float c;       // scale * log2(e)
    float scale;
};

// Largest power of two s with bound * s <= 2^15 (1 when the bound is 0 or not finite).
__device__ __forceinline__ float pow2_scale(float bound) {
    if (!(bound > 0.f) || isinf(bound)) return 1.f;
    const float e = fminf(fmaxf(floorf(__log2f(32768.f / bound)), -120.f), 120.f);
    return exp2f(e);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Non-negative floats order like their bit patterns. The plain read first skips the
// atomic when the slot already holds a larger value (the common case after a few blocks).
__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
    if (__float_as_uint(v) > __atomic_load_n(reinterpret_cast<unsigned int*>(p), __ATOMIC_RELAXED))
        atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

// Max over the workgroup (blockDim.x = 256), then one conditional atomic per workgroup.
__device__ __forceinline__ void block_max_to(float* p, float v) {
    __shared__ float part[4];
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) atomic_max_nonneg(p, fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3])));
}

// dq = 0 and the bound slots = 0.
__global__ void zero_kernel(float4* __restrict__ p, size_t n4, float* __restrict__ stats) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    if (i < BWD_STATS) stats[i] = 0.f;
    for (size_t j = i; j < n4; j += stride) p[j] = float4{0.f, 0.f, 0.f, 0.f};
}

// D[h][i] = sum_c dO[i][h][c] * (O + O_lo)[i][h][c], and max_i ||dO_i||^2.
// 16 lanes per (position, head) row.
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o, const bf16* __restrict__ o_lo,
                                                      const bf16* __restrict__ dout, float* __restrict__ dbuf,
                                                      float* __restrict__ stats, int T, int Hq) {
    const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int part = threadIdx.x & 15;
    float s = 0.f, n2 = 0.f;
    if (row < (long)T * Hq) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(o + row * HEAD_DIM + part * 8);
        const u32x4 y = *reinterpret_cast<const u32x4*>(dout + row * HEAD_DIM + part * 8);
        u32x4 z = {0u, 0u, 0u, 0u};
        if (o_lo) z = *reinterpret_cast<const u32x4*>(o_lo + row * HEAD_DIM + part * 8);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float d0 = bf16_lo(y[m]), d1 = bf16_hi(y[m]);
            s += d0 * (bf16_lo(x[m]) + bf16_lo(z[m])) + d1 * (bf16_hi(x[m]) + bf16_hi(z[m]));
            n2 += d0 * d0 + d1 * d1;
        }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
        s += __shfl_xor(s, off);
        n2 += __shfl_xor(n2, off);
    }
    if (part == 0 && row < (long)T * Hq) {
        const int pos = (int)(row / Hq), head = (int)(row % Hq);
        dbuf[(size_t)head * T + pos] = s;
    }
    block_max_to(stats + ST_DO_NORM2, n2);
}

// max |x| over n8 chunks of 8 bf16.
__global__ __launch_bounds__(256) void maxabs_kernel(const u32x4* __restrict__ p, size_t n8,
                                                     float* __restrict__ out) {
    float m = 0.f;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (size_t)gridDim.x * blockDim.x) {
        const u32x4 x = p[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(x[j])), fabsf(bf16_hi(x[j]))));
    }
    block_max_to(out, m);
}

// max over rows of the squared norm of 128-element bf16 rows; 16 lanes per row, the
// loop bound is uniform over the workgroup so every lane reaches the shuffles.
__global__ __launch_bounds__(256) void rownorm_kernel(const bf16* __restrict__ p, long nrows,
                                                      float* __restrict__ out) {
    float best = 0.f;
    const int part = threadIdx.x & 15;
    for (long base = (long)blockIdx.x * 16; base < nrows; base += (long)gridDim.x * 16) {
        const long row = base + (threadIdx.x >> 4);
        float n2 = 0.f;
        if (row < nrows) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(p + row * HEAD_DIM + part * 8);
#pragma unroll
            for (int m = 0; m < 4; ++m) n2 += bf16_lo(x[m]) * bf16_lo(x[m]) + bf16_hi(x[m]) * bf16_hi(x[m]);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) n2 += __shfl_xor(n2, off);
        best = fmaxf(best, n2);
    }
    block_max_to(out, best);
}

__global__ void cast_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n; j += stride) {
        const __bf16 b = (__bf16)in[j];
        out[j] = __builtin_bit_cast(uint16_t, b);
    }
}

// Rows of a list entry: row R = rb * 32 + q (rb = row block, q = 0..31) of entry e is
// query head hbase + (R >> lg) at position pbase + (R & mask).
struct RowMap {
    int hbase, pbase, lg, mask;
    __device__ __forceinline__ int head(int R) const { return hbase + (R >> lg); }
    __device__ __forceinline__ int pos(int R) const { return pbase + (R & mask); }
};

template <bool SPARSE>
__device__ __forceinline__ RowMap row_map(const BwdArgs& a, int g, int e) {
    RowMap m;
    if constexpr (SPARSE) {
        const int hi = e / a.nb, qb = e - hi * a.nb;   // once per entry
        m.hbase = g * a.G + hi;
        m.pbase = qb * a.sblock;
        m.lg = 30;
        m.mask = 0x3fffffff;
    } else {
        m.hbase = g * a.G;
        m.pbase = (e >> 1) * a.BMq;
        m.lg = a.lgBMq;
        m.mask = a.BMq - 1;
    }
    return m;
}

template <int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void bwd_kernel(BwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int KEYS = NW * 32;
    constexpr int KT_LD = KEYS + 8;
    constexpr int DS_LD = KEYS + 8;
    constexpr int UPT = 256 / NT;   // (row pair, 8 dims) staging units per thread per row block

    __shared__ __attribute__((aligned(16))) bf16 Qs[32 * QS_LD];
    __shared__ __attribute__((aligned(16))) bf16 dOs[32 * QS_LD];
    __shared__ __attribute__((aligned(16))) _Float16 Kt[HEAD_DIM * KT_LD];
    __shared__ __attribute__((aligned(16))) _Float16 Qt[HEAD_DIM * QT_LD];
    __shared__ __attribute__((aligned(16))) _Float16 dOt[HEAD_DIM * QT_LD];
    __shared__ __attribute__((aligned(16))) _Float16 dSs[32 * DS_LD];
    __shared__ float lse_s[32];
    __shared__ float dd_s[32];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int g = blockIdx.x % a.Hk, y = blockIdx.x / a.Hk;
    const int T = a.T;

    // fp16 operand scales (powers of two) from the preprocess bounds
    const float nrm_do = sqrtf(a.stats[ST_DO_NORM2]), nrm_v = sqrtf(a.stats[ST_V_NORM2]);
    const float sO = pow2_scale(fmaxf(2.f * nrm_do * nrm_v, nrm_do));
    const float sQ = pow2_scale(a.stats[ST_Q_ABS]);
    const float sK = pow2_scale(a.stats[ST_K_ABS]);

    int key_base, col;
    if constexpr (!SPARSE) {
        const int kt = a.order[y];
        key_base = kt * KEYS;
        col = kt;
    } else {
        key_base = y * a.sblock;
        col = g * a.nb + y;
    }
    const int lb = a.ptr[col], le = a.ptr[col + 1];
    const int my_key = key_base + w * 32 + l32;
    const bool key_ok = my_key < T;
    const size_t kv_row = (size_t)a.Hk * HEAD_DIM;

    // K and V rows of this lane's key as B operands (dims 16*ks + 8*hf .. +7).
    bf16x8 kf[8], vf[8];
    {
        const bf16* kp = a.k + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM + 8 * hf;
        const bf16* vp = a.v + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u}, z = {0u, 0u, 0u, 0u};
            if (key_ok) {
                x = *reinterpret_cast<const u32x4*>(kp + 16 * ks);
                z = *reinterpret_cast<const u32x4*>(vp + 16 * ks);
            }
            kf[ks] = as_bf16x8(x);
            vf[ks] = as_bf16x8(z);
        }
    }
    int4 kd = {0, 0, 0, 0};
    if (!SPARSE && key_ok) kd = a.desc[my_key];

    // K^T of the whole key tile into LDS as fp16 * sK (B operand of dQ = dS K).
    {
        const bf16* kb = a.k + (size_t)g * HEAD_DIM;
#pragma unroll
        for (int i = 0; i < (KEYS * 8) / NT; ++i) {
            const int u = tid + i * NT, p = u % (KEYS / 2), d0 = (u / (KEYS / 2)) * 8;
            const int key = key_base + 2 * p;
            u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
            if (key < T) x0 = *reinterpret_cast<const u32x4*>(kb + (size_t)key * kv_row + d0);
            if (key + 1 < T) x1 = *reinterpret_cast<const u32x4*>(kb + (size_t)(key + 1) * kv_row + d0);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                *reinterpret_cast<uint32_t*>(&Kt[(d0 + 2 * m) * KT_LD + 2 * p]) =
                    pack_f16(bf16_lo(x0[m]) * sK, bf16_lo(x1[m]) * sK);
                *reinterpret_cast<uint32_t*>(&Kt[(d0 + 2 * m + 1) * KT_LD + 2 * p]) =
                    pack_f16(bf16_hi(x0[m]) * sK, bf16_hi(x1[m]) * sK);
            }
        }
    }

    f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk_acc[db][r] = 0.f;
            dv_acc[db][r] = 0.f;
        }

    const int RB = SPARSE ? a.sblock / 32 : ROWS_PER_WG / 32;   // 32-row blocks per list entry
    const int nsteps = (le - lb) * RB;

    // prefetch registers: Q and dO rows (2 rows x 8 dims per unit), LSE and D
    u32x4 px0[UPT], px1[UPT], py0[UPT], py1[UPT];
    float pl = INFINITY, pd = 0.f;

#define BWD_LOAD_STEP(st)                                                                      \
    {                                                                                          \
        const int e_ = a.ent[lb + (st) / RB], rb_ = (st) % RB;                                 \
        const RowMap m_ = row_map<SPARSE>(a, g, e_);                                           \
        _Pragma("unroll") for (int i = 0; i < UPT; ++i) {                                      \
            const int u_ = tid + i * NT, q0_ = 2 * (u_ & 15), d0_ = (u_ >> 4) * 8;             \
            const int R0_ = rb_ * 32 + q0_;                                                    \
            const int p0_ = m_.pos(R0_), h0_ = m_.head(R0_);                                   \
            const int p1_ = m_.pos(R0_ + 1), h1_ = m_.head(R0_ + 1);                           \
            const size_t o0_ = ((size_t)p0_ * a.Hq + h0_) * HEAD_DIM + d0_;                    \
            const size_t o1_ = ((size_t)p1_ * a.Hq + h1_) * HEAD_DIM + d0_;                    \
            u32x4 z_ = {0u, 0u, 0u, 0u};                                                       \
            px0[i] = z_; py0[i] = z_; px1[i] = z_; py1[i] = z_;                                \
            if (p0_ < T) {                                                                     \
                px0[i] = *reinterpret_cast<const u32x4*>(a.q + o0_);                           \
                py0[i] = *reinterpret_cast<const u32x4*>(a.dout + o0_);                        \
            }                                                                                  \
            if (p1_ < T) {                                                                     \
                px1[i] = *reinterpret_cast<const u32x4*>(a.q + o1_);                           \
                py1[i] = *reinterpret_cast<const u32x4*>(a.dout + o1_);                        \
            }                                                                                  \
        }                                                                                      \
        if (tid < 32) {                                                                        \
            const int p_ = m_.pos(rb_ * 32 + tid), h_ = m_.head(rb_ * 32 + tid);               \
            pl = INFINITY; /* rows past the end and fully masked rows: P = 0 */                \
            pd = 0.f;                                                                          \
            if (p_ < T) {                                                                      \
                const float lse_ = a.lse[(size_t)h_ * T + p_];                                 \
                pl = lse_ == -INFINITY ? INFINITY : lse_ * LOG2E;                              \
                pd = a.dbuf[(size_t)h_ * T + p_];                                              \
            }                                                                                  \
        }                                                                                      \
    }

    if (nsteps > 0) BWD_LOAD_STEP(0);

    for (int step = 0; step < nsteps; ++step) {
        const int e = a.ent[lb + step / RB];
        const int rb = step % RB;
        const bool full = SPARSE ? true : ((e & 1) != 0);
        const RowMap rm = row_map<SPARSE>(a, g, e);

        lds_barrier();   // previous row block fully consumed
        // Stage: natural bf16 [q][d]; transposed fp16 [d][q] scaled by sQ / sO.
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT, q0 = 2 * (u & 15), d0 = (u >> 4) * 8;
            *reinterpret_cast<u32x4*>(&Qs[q0 * QS_LD + d0]) = px0[i];
            *reinterpret_cast<u32x4*>(&Qs[(q0 + 1) * QS_LD + d0]) = px1[i];
            *reinterpret_cast<u32x4*>(&dOs[q0 * QS_LD + d0]) = py0[i];
            *reinterpret_cast<u32x4*>(&dOs[(q0 + 1) * QS_LD + d0]) = py1[i];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                *reinterpret_cast<uint32_t*>(&Qt[(d0 + 2 * m) * QT_LD + q0]) =
                    pack_f16(bf16_lo(px0[i][m]) * sQ, bf16_lo(px1[i][m]) * sQ);
                *reinterpret_cast<uint32_t*>(&Qt[(d0 + 2 * m + 1) * QT_LD + q0]) =
                    pack_f16(bf16_hi(px0[i][m]) * sQ, bf16_hi(px1[i][m]) * sQ);
                *reinterpret_cast<uint32_t*>(&dOt[(d0 + 2 * m) * QT_LD + q0]) =
                    pack_f16(bf16_lo(py0[i][m]) * sO, bf16_lo(py1[i][m]) * sO);
                *reinterpret_cast<uint32_t*>(&dOt[(d0 + 2 * m + 1) * QT_LD + q0]) =
                    pack_f16(bf16_hi(py0[i][m]) * sO, bf16_hi(py1[i][m]) * sO);
            }
        }
        if (tid < 32) {
            lse_s[tid] = pl;
            dd_s[tid] = pd;
        }
        lds_barrier();

        if (step + 1 < nsteps) BWD_LOAD_STEP(step + 1);

        // S = Q K^T and dP = dO V^T: lane column = its key, rows q = acc_row(r, hf).
        f32x16 sacc, dpacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sacc[r] = 0.f;
            dpacc[r] = 0.f;
        }
        {
            const bf16* qr = Qs + l32 * QS_LD + 8 * hf;
            const bf16* dr = dOs + l32 * QS_LD + 8 * hf;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                sacc = mfma32(*reinterpret_cast<const bf16x8*>(qr + 16 * ks), kf[ks], sacc);
                dpacc = mfma32(*reinterpret_cast<const bf16x8*>(dr + 16 * ks), vf[ks], dpacc);
            }
        }

        // visibility of the 16 (row, key) cells of this lane: all of them on FULL tiles,
        // the interval test on PARTIAL ones (the branch is uniform over the workgroup)
        uint32_t vis = key_ok ? 0xffffu : 0u;
        if (!full && key_ok) {
            vis = 0u;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int p = rm.pos(rb * 32 + acc_row(r, hf));
                const bool v = (p >= kd.x && p < kd.y) || (p >= kd.z && p < kd.w);
                vis |= (uint32_t)v << r;
            }
        }

        // P (fp16, in [0, 1]) and dS * sO (fp16)
        float ds[16];
        f16x8 pb[2], sb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            u32x4 pk, sk;
#pragma unroll
            for (int e2 = 0; e2 < 8; e2 += 2) {
                float pv[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int r = kk * 8 + e2 + j;
                    const int q = acc_row(r, hf);
                    const float p = fast_exp2(fmaf(sacc[r], a.c, -lse_s[q]));
                    pv[j] = ((vis >> r) & 1u) ? p : 0.f;
                    ds[r] = pv[j] * (dpacc[r] - dd_s[q]) * sO;
                }
                pk[e2 >> 1] = pack_f16(pv[0], pv[1]);
                sk[e2 >> 1] = pack_f16(ds[kk * 8 + e2], ds[kk * 8 + e2 + 1]);
            }
            pb[kk] = as_f16x8(pk);
            sb[kk] = as_f16x8(sk);
        }

        // dV^T += dO^T P and dK^T += Q^T dS: query slot (hf, e) of step kk is row
        // 16*kk + 8*(e/4) + 4*hf + e%4.
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const _Float16* dtr = dOt + (db * 32 + l32) * QT_LD + 4 * hf;
            const _Float16* qtr = Qt + (db * 32 + l32) * QT_LD + 4 * hf;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x2 a0 = *reinterpret_cast<const u32x2*>(dtr + 16 * kk);
                const u32x2 a1 = *reinterpret_cast<const u32x2*>(dtr + 16 * kk + 8);
                dv_acc[db] = mfma32h(as_f16x8(u32x4{a0[0], a0[1], a1[0], a1[1]}), pb[kk], dv_acc[db]);
                const u32x2 b0 = *reinterpret_cast<const u32x2*>(qtr + 16 * kk);
                const u32x2 b1 = *reinterpret_cast<const u32x2*>(qtr + 16 * kk + 8);
                dk_acc[db] = mfma32h(as_f16x8(u32x4{b0[0], b0[1], b1[0], b1[1]}), sb[kk], dk_acc[db]);
            }
        }

        // dS * sO (fp16) to LDS as [q][key] for dQ.
#pragma unroll
        for (int r = 0; r < 16; ++r) dSs[acc_row(r, hf) * DS_LD + w * 32 + l32] = (_Float16)ds[r];
        lds_barrier();

        // dQ[q][d] += scale * sum_key dS[q][key] K[key][d]; wave w takes dim blocks w, w + NW, ...
        const float dq_unscale = a.scale / (sO * sK);
        for (int db = w; db < 4; db += NW) {
            f32x16 qacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) qacc[r] = 0.f;
            const _Float16* sr = dSs + l32 * DS_LD + 8 * hf;
            const _Float16* kr = Kt + (db * 32 + l32) * KT_LD + 8 * hf;
#pragma unroll
            for (int ks = 0; ks < KEYS / 16; ++ks)
                qacc = mfma32h(*reinterpret_cast<const f16x8*>(sr + 16 * ks),
                               *reinterpret_cast<const f16x8*>(kr + 16 * ks), qacc);
            // rows of a block are consecutive positions of one head unless G > 8
            const int R0 = rb * 32;
            const int p0 = rm.pos(R0);
            if (SPARSE || a.BMq >= 32) {
                float* dqp = a.dq + ((size_t)p0 * a.Hq + rm.head(R0)) * HEAD_DIM + db * 32 + l32;
                const size_t rs = (size_t)a.Hq * HEAD_DIM;
                if (p0 + 32 <= T) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        unsafeAtomicAdd(dqp + (size_t)acc_row(r, hf) * rs, qacc[r] * dq_unscale);
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (p0 + acc_row(r, hf) < T)
                            unsafeAtomicAdd(dqp + (size_t)acc_row(r, hf) * rs, qacc[r] * dq_unscale);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int R = R0 + acc_row(r, hf);
                    const int p = rm.pos(R);
                    if (p < T)
                        unsafeAtomicAdd(a.dq + ((size_t)p * a.Hq + rm.head(R)) * HEAD_DIM + db * 32 + l32,
                                        qacc[r] * dq_unscale);
                }
            }
        }
    }
#undef BWD_LOAD_STEP

    if (key_ok) {
        const float dk_unscale = a.scale / (sQ * sO), dv_unscale = 1.f / sO;
        float* dkp = a.dk + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM;
        float* dvp = a.dv + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = db * 32 + 8 * i4 + 4 * hf;
                *reinterpret_cast<float4*>(dkp + d0) =
                    float4{dk_acc[db][4 * i4] * dk_unscale, dk_acc[db][4 * i4 + 1] * dk_unscale,
                           dk_acc[db][4 * i4 + 2] * dk_unscale, dk_acc[db][4 * i4 + 3] * dk_unscale};
                *reinterpret_cast<float4*>(dvp + d0) =
                    float4{dv_acc[db][4 * i4] * dv_unscale, dv_acc[db][4 * i4 + 1] * dv_unscale,
                           dv_acc[db][4 * i4 + 2] * dv_unscale, dv_acc[db][4 * i4 + 3] * dv_unscale};
            }
    }
}

hipError_t launch_bwd_pre(const Problem& P, const void* q, const void* k, const void* v, const void* o,
                          const void* o_lo, const void* dout, float* dq, float* dbuf, hipStream_t s) {
    float* stats = reinterpret_cast<float*>(reinterpret_cast<char*>(dbuf) + bwd_stats_offset(P.Hq, P.T));
    const size_t n4 = (size_t)P.T * P.Hq * HEAD_DIM / 4;
    hipLaunchKernelGGL(zero_kernel, dim3(2048), dim3(256), 0, s, reinterpret_cast<float4*>(dq), n4, stats);
    const long rows = (long)P.T * P.Hq;
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s,
                       static_cast<const bf16*>(o), static_cast<const bf16*>(o_lo), static_cast<const bf16*>(dout),
                       dbuf, stats, P.T, P.Hq);
    const size_t nq8 = (size_t)P.T * P.Hq * HEAD_DIM / 8, nk8 = (size_t)P.T * P.Hk * HEAD_DIM / 8;
    hipLaunchKernelGGL(maxabs_kernel, dim3(1024), dim3(256), 0, s, static_cast<const u32x4*>(q), nq8,
                       stats + ST_Q_ABS);
    hipLaunchKernelGGL(maxabs_kernel, dim3(256), dim3(256), 0, s, static_cast<const u32x4*>(k), nk8,
                       stats + ST_K_ABS);
    hipLaunchKernelGGL(rownorm_kernel, dim3(256), dim3(256), 0, s, static_cast<const bf16*>(v),
                       (long)P.T * P.Hk, stats + ST_V_NORM2);
    return hipGetLastError();
}

hipError_t launch_bwd_main(const Problem& P, const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, const int4* desc,
                           const void* index, const float* dbuf, hipStream_t s) {
    const IndexLayout L = index_layout(P);
    const char* base = static_cast<const char*>(index);
    BwdArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.dout = static_cast<const bf16*>(dout);
    a.lse = lse;
    a.dbuf = dbuf;
    a.stats = reinterpret_cast<const float*>(reinterpret_cast<const char*>(dbuf) + bwd_stats_offset(P.Hq, P.T));
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.desc = desc;
    a.ptr = reinterpret_cast<const int*>(base + L.bwd_ptr);
    a.ent = reinterpret_cast<const int*>(base + L.bwd_ent);
    a.order = P.sparse ? nullptr : reinterpret_cast<const int*>(base + L.bwd_order);
    a.T = P.T;
    a.Hq = P.Hq;
    a.Hk = P.Hk;
    a.G = P.G;
    a.BMq = P.bBM;
    a.lgBMq = P.lgBM;
    a.nb = P.nb;
    a.sblock = P.sblock;
    a.c = P.scale * LOG2E;
    a.scale = P.scale;
    if (!P.sparse) {
        hipLaunchKernelGGL((bwd_kernel<4, false>), dim3(P.Hk * P.nkt_b), dim3(256), 0, s, a);
    } else if (P.sblock == 64) {
        hipLaunchKernelGGL((bwd_kernel<2, true>), dim3(P.Hk * P.nb), dim3(128), 0, s, a);
    } else {
        hipLaunchKernelGGL((bwd_kernel<4, true>), dim3(P.Hk * P.nb), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* in, void* out, size_t n, hipStream_t s) {
    hipLaunchKernelGGL(cast_kernel, dim3(2048), dim3(256), 0, s, in, static_cast<uint16_t*>(out), n);
    return hipGetLastError();
}

}  // namespace mlct
