// Masked attention backward for gfx950.
//
//   D_i  = sum_c dO[i, c] O[i, c]                              (bwd_pre_kernel, HBM-bound)
//   P    = exp(scale * Q K^T - LSE)  on the non-empty tiles    (recomputed)
//   dV  += P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//   dK  += scale * dS^T Q                                      (bwd_kernel, key-tile major)
//   dQ   = scale * dS K                                        (dq_kernel, query-tile major)
//
// bwd_kernel. Work item = 32 * NWK keys of one KV head, walking the non-empty query tiles
// of its key tile's list for every query head of the group, 32 query rows per step. It
// runs 2 * NWK waves (two per SIMD) in two roles on the same 32 keys: "A" waves compute
// S = Q K^T -> P and accumulate dV^T = dO^T P; "B" waves compute dP = dO V^T, receive P
// through LDS, form dS = P * (dP - D) and accumulate dK^T = Q^T dS. Each role keeps its
// keys' K or V rows in registers (B operands) and its 128 x 32 accumulator, so dK and dV
// are written once, without atomics. The B waves prefetch and stage the row blocks; S and
// dP are computed untransposed so P and dS leave the accumulators already in the B-operand
// layout of the dV^T / dK^T products, whose A operands (dO^T, Q^T) come from transposed
// LDS reads of the staged rows.
//
// dq_kernel. dQ in its own pass, query-tile major on the forward's tile lists (described
// at the kernel), so dQ needs no atomics and is deterministic.
//
// Precision. All products take fp16 operands: fp16 carries 11 significant bits against
// bf16's 8, which cuts the rounding of P and dS by 8x, and bf16 inputs convert exactly
// within range. To keep every operand inside fp16's range, Q, K, V and dO are multiplied
// by powers of two chosen from bounds measured in the preprocess (max |Q|, max |K|,
// max ||V_j||, max ||dO_i||; |dS_ij| <= 2 ||dO_i|| max_j ||V_j|| bounds dS), and the
// scales are divided out of the fp32 results. D uses O plus its low half O_lo when the
// forward wrote one, i.e. the forward's fp32 O.
#include "common.h"

namespace mlct {

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

// The bound slots = 0 (a kernel rather than a memset, so the sequence can be captured).
__global__ void zero_stats_kernel(float* __restrict__ stats) {
    if (threadIdx.x < BWD_STATS) stats[threadIdx.x] = 0.f;
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

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, source lane s
// supplies the address of 4 consecutive 16-bit elements and output lane i receives
// element i % 4 of source lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12. With source lane s
// pointing at M[r0 + s/4][c0 + 4*(s%4)], output lane i gets M[r0 .. r0+3][c0 + i].
__device__ __forceinline__ u32x2 ds_read_tr16(const _Float16* p) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Staged Q / dO rows: 128 fp16 (256 bytes) per row, the 16-byte chunk c of row q stored at
// chunk slot c ^ 4*(q % 4) ^ (q / 4 % 4). Sixteen consecutive rows of one chunk (row
// reads) and a 4-row x 4-chunk block (transposed reads) both land on distinct banks.
__device__ __forceinline__ int swz(int q, int c) { return c ^ (4 * (q & 3)) ^ ((q >> 2) & 3); }
__device__ __forceinline__ int swz_off(int q, int col) { return q * HEAD_DIM + swz(q, col >> 3) * 8 + (col & 7); }

// A operand (32 rows x 16 k) whose row m = lane % 32 is column c0 + m of a swizzled
// [rows][128] fp16 matrix M, k-slots e = 0..3 of the lane being rows r_lo + e and e = 4..7
// rows r_hi + e - 4.
__device__ __forceinline__ f16x8 tr_operand_swz(const _Float16* M, int r_lo, int r_hi, int c0, int lane) {
    const int s = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const u32x2 lo = ds_read_tr16(M + swz_off(r_lo + (s >> 2), col));
    const u32x2 hi = ds_read_tr16(M + swz_off(r_hi + (s >> 2), col));
    return as_f16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Same for a plain [rows][ld] fp16 matrix.
__device__ __forceinline__ f16x8 tr_operand(const _Float16* M, int ld, int r_lo, int r_hi, int c0, int lane) {
    const int s = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const u32x2 lo = ds_read_tr16(M + (r_lo + (s >> 2)) * ld + col);
    const u32x2 hi = ds_read_tr16(M + (r_hi + (s >> 2)) * ld + col);
    return as_f16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// 8 bf16 (one 16-byte chunk) -> 8 fp16 scaled by s.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_scaled(u32x4 x, float s) {
    u32x4 r;
#pragma unroll
    for (int m = 0; m < 4; ++m) r[m] = pack_f16(bf16_lo(x[m]) * s, bf16_hi(x[m]) * s);
    return r;
}

// Work item: NWK blocks of 32 keys of one KV head, 2 * NWK waves. Waves 0..NWK-1 ("A")
// compute S -> P and own dV^T and the dQ products; waves NWK..2*NWK-1 ("B") compute dP,
// receive P through LDS, form dS and own dK^T. Wave w and w + NWK handle the same 32
// keys and share a SIMD. All products run on fp16 operands: Q, K, V, dO are multiplied
// by the powers of two sQ, sK, sV, sO while being staged.
template <int NWK, bool SPARSE>
__global__ __launch_bounds__(NWK * 128) void bwd_kernel(BwdArgs a) {
    constexpr int NT = NWK * 128;
    constexpr int KEYS = NWK * 32;
    constexpr int CPT = 512 / (NT / 2);     // 16-byte chunks per B thread per tensor per row block

    __shared__ __attribute__((aligned(16))) _Float16 Qh[32 * HEAD_DIM];    // swizzled rows
    __shared__ __attribute__((aligned(16))) _Float16 dOh[32 * HEAD_DIM];   // swizzled rows
    __shared__ __attribute__((aligned(16))) _Float16 Ps[NWK * 2 * 64 * 8];  // [kb][kk][lane][8]
    __shared__ __attribute__((aligned(16))) float lse_s[32];
    __shared__ __attribute__((aligned(16))) float dd_s[32];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const bool is_a = w < NWK;
    const int kb = is_a ? w : w - NWK;
    const int g = blockIdx.x % a.Hk, y = blockIdx.x / a.Hk;
    const int T = a.T;

    // fp16 operand scales (powers of two) from the preprocess bounds
    const float nrm_do = sqrtf(a.stats[ST_DO_NORM2]), nrm_v = sqrtf(a.stats[ST_V_NORM2]);
    const float sO = pow2_scale(fmaxf(2.f * nrm_do * nrm_v, nrm_do));
    const float sQ = pow2_scale(a.stats[ST_Q_ABS]);
    const float sK = pow2_scale(a.stats[ST_K_ABS]);
    const float sV = pow2_scale(nrm_v);
    const float cS = a.c / (sQ * sK);       // exponent scale for the scaled scores
    const float inv_sV = 1.f / sV;

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
    const int my_key = key_base + kb * 32 + l32;
    const bool key_ok = my_key < T;
    const size_t kv_row = (size_t)a.Hk * HEAD_DIM;
    const bf16* kg = a.k + (size_t)g * HEAD_DIM;
    const bf16* vg = a.v + (size_t)g * HEAD_DIM;

    // A: K rows (B operand of S) and K^T fragments (B operand of dQ); B: V rows (B operand
    // of dP). All fp16, scaled.
    const int RB = SPARSE ? a.sblock / 32 : ROWS_PER_WG / 32;   // 32-row blocks per list entry
    const int nsteps = (le - lb) * RB;

    // Both roles run the same number of steps with three barriers each:
    //   b1: Q, dO, LSE, D of the row block staged (by B)
    //   b2: P in LDS (A), dP in registers (B)
    //   b3: every reader of the staged rows is done
    // A: [b1] S, P -> LDS [b2] dV [b3]        B: stage [b1] prefetch, dP [b2] dS, dK [b3]
    f32x16 acc[4];   // A: dV^T, B: dK^T (dims db*32 + acc_row(r, hf), key = lane column)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    if (is_a) {
        // K rows (B operand of S)
        f16x8 kf[8];
        {
            const bf16* rowp = kg + (size_t)my_key * kv_row + 8 * hf;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (key_ok) x = *reinterpret_cast<const u32x4*>(rowp + 16 * ks);
                kf[ks] = as_f16x8(bf16x8_to_f16x8_scaled(x, sK));
            }
        }
        int4 kd = {0, 0, 0, 0};
        if (!SPARSE && key_ok) kd = a.desc[my_key];

        for (int step = 0; step < nsteps; ++step) {
            const int e = a.ent[lb + step / RB];
            const int rb = step % RB;
            const bool full = SPARSE ? true : ((e & 1) != 0);
            const RowMap rm = row_map<SPARSE>(a, g, e);
            lds_barrier();   // b1

            // S = Q K^T (scaled by sQ * sK); rows q = acc_row(r, hf)
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                sacc = mfma32h(*reinterpret_cast<const f16x8*>(&Qh[swz_off(l32, 16 * ks + 8 * hf)]), kf[ks], sacc);
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
            // P (fp16); P and dS slots (hf, e) of step kk are rows 16*kk + 8*(e/4) + 4*hf + e%4
            f16x8 pb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float4 l0 = *reinterpret_cast<const float4*>(&lse_s[16 * kk + 4 * hf]);
                const float4 l1 = *reinterpret_cast<const float4*>(&lse_s[16 * kk + 8 + 4 * hf]);
                const float lr[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                u32x4 pk;
#pragma unroll
                for (int e2 = 0; e2 < 8; e2 += 2) {
                    const int r0 = kk * 8 + e2, r1 = r0 + 1;
                    const float p0 = fast_exp2(fmaf(sacc[r0], cS, -lr[e2]));
                    const float p1 = fast_exp2(fmaf(sacc[r1], cS, -lr[e2 + 1]));
                    pk[e2 >> 1] = pack_f16(((vis >> r0) & 1u) ? p0 : 0.f, ((vis >> r1) & 1u) ? p1 : 0.f);
                }
                pb[kk] = as_f16x8(pk);
                *reinterpret_cast<u32x4*>(&Ps[((kb * 2 + kk) * 64 + lane) * 8]) = pk;
            }
            lds_barrier();   // b2

            // dV^T += (dO * sO)^T P
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc[db] = mfma32h(tr_operand_swz(dOh, 16 * kk + 4 * hf, 16 * kk + 8 + 4 * hf, db * 32, lane),
                                      pb[kk], acc[db]);
            lds_barrier();   // b3
        }
    } else {
        // V rows (B operand of dP)
        f16x8 vf[8];
        {
            const bf16* rowp = vg + (size_t)my_key * kv_row + 8 * hf;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (key_ok) x = *reinterpret_cast<const u32x4*>(rowp + 16 * ks);
                vf[ks] = as_f16x8(bf16x8_to_f16x8_scaled(x, sV));
            }
        }
        const int btid = tid - NWK * 64;
        u32x4 pq[CPT], pdo[CPT];
        float pl = INFINITY, pd = 0.f;

#define BWD_LOAD_STEP(st)                                                                      \
    {                                                                                          \
        const int e_ = a.ent[lb + (st) / RB], rb_ = (st) % RB;                                 \
        const RowMap m_ = row_map<SPARSE>(a, g, e_);                                           \
        _Pragma("unroll") for (int i = 0; i < CPT; ++i) {                                      \
            const int c_ = btid + i * (NT / 2), R_ = rb_ * 32 + (c_ >> 4), d0_ = (c_ & 15) * 8; \
            const int p_ = m_.pos(R_);                                                         \
            const size_t o_ = ((size_t)p_ * a.Hq + m_.head(R_)) * HEAD_DIM + d0_;              \
            u32x4 z_ = {0u, 0u, 0u, 0u};                                                       \
            pq[i] = z_;                                                                        \
            pdo[i] = z_;                                                                       \
            if (p_ < T) {                                                                      \
                pq[i] = *reinterpret_cast<const u32x4*>(a.q + o_);                             \
                pdo[i] = *reinterpret_cast<const u32x4*>(a.dout + o_);                         \
            }                                                                                  \
        }                                                                                      \
        if (btid < 32) {                                                                       \
            const int p_ = m_.pos(rb_ * 32 + btid), h_ = m_.head(rb_ * 32 + btid);             \
            pl = INFINITY; /* rows past the end and fully masked rows: P = 0 */                \
            pd = 0.f;                                                                          \
            if (p_ < T) {                                                                      \
                const float lse_ = a.lse[(size_t)h_ * T + p_];                                 \
                pl = lse_ == -INFINITY ? INFINITY : lse_ * LOG2E;                              \
                pd = a.dbuf[(size_t)h_ * T + p_] * sO;                                         \
            }                                                                                  \
        }                                                                                      \
    }

        if (nsteps > 0) BWD_LOAD_STEP(0);
        for (int step = 0; step < nsteps; ++step) {
            // stage Q * sQ and dO * sO as swizzled fp16 rows, LSE (base 2) and D * sO
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = btid + i * (NT / 2), q = c >> 4, d0 = (c & 15) * 8;
                *reinterpret_cast<u32x4*>(&Qh[swz_off(q, d0)]) = bf16x8_to_f16x8_scaled(pq[i], sQ);
                *reinterpret_cast<u32x4*>(&dOh[swz_off(q, d0)]) = bf16x8_to_f16x8_scaled(pdo[i], sO);
            }
            if (btid < 32) {
                lse_s[btid] = pl;
                dd_s[btid] = pd;
            }
            lds_barrier();   // b1
            if (step + 1 < nsteps) BWD_LOAD_STEP(step + 1);

            // dP = dO V^T (scaled by sO * sV)
            f32x16 dpacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) dpacc[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                dpacc = mfma32h(*reinterpret_cast<const f16x8*>(&dOh[swz_off(l32, 16 * ks + 8 * hf)]), vf[ks], dpacc);
            lds_barrier();   // b2

            // dS * sO = P * (dP * sO - D * sO); dK^T += (Q * sQ)^T (dS * sO)
            f16x8 sb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const f16x8 ph = as_f16x8(*reinterpret_cast<const u32x4*>(&Ps[((kb * 2 + kk) * 64 + lane) * 8]));
                const float4 d0v = *reinterpret_cast<const float4*>(&dd_s[16 * kk + 4 * hf]);
                const float4 d1v = *reinterpret_cast<const float4*>(&dd_s[16 * kk + 8 + 4 * hf]);
                const float dr[8] = {d0v.x, d0v.y, d0v.z, d0v.w, d1v.x, d1v.y, d1v.z, d1v.w};
                u32x4 sk;
#pragma unroll
                for (int e2 = 0; e2 < 8; e2 += 2) {
                    const int r0 = kk * 8 + e2, r1 = r0 + 1;
                    const float x0 = (float)ph[e2] * fmaf(dpacc[r0], inv_sV, -dr[e2]);
                    const float x1 = (float)ph[e2 + 1] * fmaf(dpacc[r1], inv_sV, -dr[e2 + 1]);
                    sk[e2 >> 1] = pack_f16(x0, x1);
                }
                sb[kk] = as_f16x8(sk);
            }
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc[db] = mfma32h(tr_operand_swz(Qh, 16 * kk + 4 * hf, 16 * kk + 8 + 4 * hf, db * 32, lane),
                                      sb[kk], acc[db]);
            lds_barrier();   // b3
        }
#undef BWD_LOAD_STEP
    }

    if (key_ok) {
        const float unscale = is_a ? 1.f / sO : a.scale / (sQ * sO);
        float* outp = (is_a ? a.dv : a.dk) + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = db * 32 + 8 * i4 + 4 * hf;
                *reinterpret_cast<float4*>(outp + d0) =
                    float4{acc[db][4 * i4] * unscale, acc[db][4 * i4 + 1] * unscale,
                           acc[db][4 * i4 + 2] * unscale, acc[db][4 * i4 + 3] * unscale};
            }
    }
}

// dQ pass: dQ = scale * dS K, one query tile per work item, no atomics.
//
// Work item and tile lists are the forward's: 32 * NW (head, position) rows (the G heads
// of one KV head x 256/G positions, or one block-sparse (head, query block) row) walking
// 64-key tiles. Like the forward it works on transposed products so a lane owns one query
// row: S^T = K Q^T and dP^T = V dO^T (A = K / V rows from LDS, B = the wave's Q / dO rows
// in registers), then P^T, dS^T = P^T * (dP^T - D) with the row's LSE and D as per-lane
// scalars, and dQ^T += K^T dS^T with K^T read from the same LDS tile by transposed reads
// and dS^T straight from the accumulators as the B operand. Operands are fp16 scaled by
// the same powers of two as the main backward kernel.
template <int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void dq_kernel(BwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int CPT = 1024 / NT;               // 16-byte chunks per thread per tile per tensor
    constexpr int TPE = SPARSE ? NW / 2 : 1;     // 64-key tiles per list entry

    __shared__ __attribute__((aligned(16))) _Float16 Kh[FWD_BN * HEAD_DIM];   // swizzled rows
    __shared__ __attribute__((aligned(16))) _Float16 Vh[FWD_BN * HEAD_DIM];   // swizzled rows
    __shared__ int4 Ds[FWD_BN];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int g = blockIdx.x % a.Hk, y = blockIdx.x / a.Hk;
    const int T = a.T;

    const float nrm_do = sqrtf(a.stats[ST_DO_NORM2]), nrm_v = sqrtf(a.stats[ST_V_NORM2]);
    const float sO = pow2_scale(fmaxf(2.f * nrm_do * nrm_v, nrm_do));
    const float sQ = pow2_scale(a.stats[ST_Q_ABS]);
    const float sK = pow2_scale(a.stats[ST_K_ABS]);
    const float sV = pow2_scale(nrm_v);
    const float cS = a.c / (sQ * sK);
    const float inv_sV = 1.f / sV;

    int head, pos, lb, le;
    if constexpr (!SPARSE) {
        const int qt = a.order[y];
        const int R = w * 32 + l32;
        head = g * a.G + (R >> a.lgBMq);
        pos = qt * a.BMq + (R & (a.BMq - 1));
        lb = a.ptr[qt];
        le = a.ptr[qt + 1];
    } else {
        const int hi = y / a.nb, qb = y - hi * a.nb;
        head = g * a.G + hi;
        pos = qb * a.sblock + w * 32 + l32;
        const int r = head * a.nb + qb;
        lb = a.ptr[r];
        le = a.ptr[r + 1];
    }
    const bool row_ok = pos < T;
    const int ntiles = (le - lb) * TPE;

    // this lane's row: LSE (base 2), D * sO, Q * sQ and dO * sO as B operands
    float lse2 = INFINITY, dd = 0.f;
    f16x8 qf[8], df[8];
    {
        const size_t ro = ((size_t)pos * a.Hq + head) * HEAD_DIM + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u}, z = {0u, 0u, 0u, 0u};
            if (row_ok) {
                x = *reinterpret_cast<const u32x4*>(a.q + ro + 16 * ks);
                z = *reinterpret_cast<const u32x4*>(a.dout + ro + 16 * ks);
            }
            qf[ks] = as_f16x8(bf16x8_to_f16x8_scaled(x, sQ));
            df[ks] = as_f16x8(bf16x8_to_f16x8_scaled(z, sO));
        }
        if (row_ok) {
            const float l = a.lse[(size_t)head * T + pos];
            lse2 = l == -INFINITY ? INFINITY : l * LOG2E;
            dd = a.dbuf[(size_t)head * T + pos] * sO;
        }
    }

    f32x16 acc[4];   // dQ^T: dims db*32 + acc_row(r, hf), query = lane column
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    const bf16* kbase = a.k + (size_t)g * HEAD_DIM;
    const bf16* vbase = a.v + (size_t)g * HEAD_DIM;
    const size_t kv_row = (size_t)a.Hk * HEAD_DIM;
    u32x4 kreg[CPT], vreg[CPT];
    int4 dreg = {0, 0, 0, 0};
    int nkey0 = 0;
    bool nmask = false;

#define DQ_LOAD_TILE(t)                                                                        \
    {                                                                                          \
        const int e_ = a.ent[lb + (t) / TPE];                                                  \
        bool full_;                                                                            \
        if constexpr (SPARSE) {                                                                \
            nkey0 = e_ * a.sblock + ((t) % TPE) * FWD_BN;                                      \
            full_ = true;                                                                      \
        } else {                                                                               \
            nkey0 = (e_ >> 1) * FWD_BN;                                                        \
            full_ = (e_ & 1) != 0;                                                             \
        }                                                                                      \
        nmask = !full_ || nkey0 + FWD_BN > T;                                                  \
        _Pragma("unroll") for (int i = 0; i < CPT; ++i) {                                      \
            const int c_ = tid + i * NT, key_ = nkey0 + (c_ >> 4);                             \
            const size_t o_ = (size_t)key_ * kv_row + (c_ & 15) * 8;                           \
            u32x4 x_ = {0u, 0u, 0u, 0u}, z_ = {0u, 0u, 0u, 0u};                                \
            if (key_ < T) {                                                                    \
                x_ = *reinterpret_cast<const u32x4*>(kbase + o_);                              \
                z_ = *reinterpret_cast<const u32x4*>(vbase + o_);                              \
            }                                                                                  \
            kreg[i] = x_;                                                                      \
            vreg[i] = z_;                                                                      \
        }                                                                                      \
        if (!SPARSE && nmask && tid < FWD_BN) {                                                \
            const int key_ = nkey0 + tid;                                                      \
            dreg = key_ < T ? a.desc[key_] : int4{0, 0, 0, 0};                                 \
        }                                                                                      \
    }

    if (ntiles > 0) DQ_LOAD_TILE(0);

    for (int t = 0; t < ntiles; ++t) {
        const int key0 = nkey0;
        const bool need_mask = nmask;

        lds_barrier();   // every wave is done reading the previous tile
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT, row = c >> 4, d0 = (c & 15) * 8;
            *reinterpret_cast<u32x4*>(&Kh[swz_off(row, d0)]) = bf16x8_to_f16x8_scaled(kreg[i], sK);
            *reinterpret_cast<u32x4*>(&Vh[swz_off(row, d0)]) = bf16x8_to_f16x8_scaled(vreg[i], sV);
        }
        if (!SPARSE && need_mask && tid < FWD_BN) Ds[tid] = dreg;
        lds_barrier();

        if (t + 1 < ntiles) DQ_LOAD_TILE(t + 1);

        // per 32-key half kb: S^T = K Q^T and dP^T = V dO^T (lane column = its query row,
        // rows = keys), dS^T, then dQ^T += (K * sK)^T (dS^T * sO) for those 32 keys
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 st, dpt;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                st[r] = 0.f;
                dpt[r] = 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int off = swz_off(kb * 32 + l32, 16 * ks + 8 * hf);
                st = mfma32h(*reinterpret_cast<const f16x8*>(&Kh[off]), qf[ks], st);
                dpt = mfma32h(*reinterpret_cast<const f16x8*>(&Vh[off]), df[ks], dpt);
            }
            // dS^T * sO = P^T * (dP^T * sO - D * sO), as B operands of two 16-key steps;
            // key slot (hf, e) of step kk is key kb*32 + 16*kk + 8*(e/4) + 4*hf + e%4
            f16x8 sb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                u32x4 pk;
#pragma unroll
                for (int e2 = 0; e2 < 8; e2 += 2) {
                    float v2[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int r = kk * 8 + e2 + j;
                        const int kidx = kb * 32 + acc_row(r, hf);
                        bool vis = true;
                        if (need_mask) {
                            if constexpr (SPARSE) {
                                vis = key0 + kidx < T;
                            } else {
                                const int4 d = Ds[kidx];
                                vis = (pos >= d.x && pos < d.y) || (pos >= d.z && pos < d.w);
                            }
                        }
                        const float p = vis ? fast_exp2(fmaf(st[r], cS, -lse2)) : 0.f;
                        v2[j] = p * fmaf(dpt[r], inv_sV, -dd);
                    }
                    pk[e2 >> 1] = pack_f16(v2[0], v2[1]);
                }
                sb[kk] = as_f16x8(pk);
            }
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int k0 = kb * 32 + 16 * kk + 4 * hf;
                    acc[db] = mfma32h(tr_operand_swz(Kh, k0, k0 + 8, db * 32, lane), sb[kk], acc[db]);
                }
        }
    }
#undef DQ_LOAD_TILE

    if (row_ok) {
        const float unscale = a.scale / (sO * sK);
        float* op = a.dq + ((size_t)pos * a.Hq + head) * HEAD_DIM;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = db * 32 + 8 * i4 + 4 * hf;
                *reinterpret_cast<float4*>(op + d0) =
                    float4{acc[db][4 * i4] * unscale, acc[db][4 * i4 + 1] * unscale,
                           acc[db][4 * i4 + 2] * unscale, acc[db][4 * i4 + 3] * unscale};
            }
    }
}

hipError_t launch_bwd_pre(const Problem& P, const void* q, const void* k, const void* v, const void* o,
                          const void* o_lo, const void* dout, float* dbuf, hipStream_t s) {
    float* stats = reinterpret_cast<float*>(reinterpret_cast<char*>(dbuf) + bwd_stats_offset(P.Hq, P.T));
    hipLaunchKernelGGL(zero_stats_kernel, dim3(1), dim3(64), 0, s, stats);
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
                           const void* index, const float* dbuf, int parts, hipStream_t s) {
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
    if (parts & BWD_PART_DKDV) {
        if (!P.sparse) {
            hipLaunchKernelGGL((bwd_kernel<4, false>), dim3(P.Hk * P.nkt_b), dim3(512), 0, s, a);
        } else if (P.sblock == 64) {
            hipLaunchKernelGGL((bwd_kernel<2, true>), dim3(P.Hk * P.nb), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((bwd_kernel<4, true>), dim3(P.Hk * P.nb), dim3(512), 0, s, a);
        }
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (!(parts & BWD_PART_DQ)) return hipSuccess;

    // dQ pass on the forward's lists
    BwdArgs b = a;
    b.ptr = reinterpret_cast<const int*>(base + L.fwd_ptr);
    b.ent = reinterpret_cast<const int*>(base + L.fwd_ent);
    b.order = P.sparse ? nullptr : reinterpret_cast<const int*>(base + L.fwd_order);
    b.BMq = P.fBM;
    if (!P.sparse) {
        hipLaunchKernelGGL((dq_kernel<8, false>), dim3(P.Hk * P.nqt_f), dim3(512), 0, s, b);
    } else if (P.sblock == 64) {
        hipLaunchKernelGGL((dq_kernel<2, true>), dim3(P.Hk * P.G * P.nb), dim3(128), 0, s, b);
    } else {
        hipLaunchKernelGGL((dq_kernel<4, true>), dim3(P.Hk * P.G * P.nb), dim3(256), 0, s, b);
    }
    return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* in, void* out, size_t n, hipStream_t s) {
    hipLaunchKernelGGL(cast_kernel, dim3(2048), dim3(256), 0, s, in, static_cast<uint16_t*>(out), n);
    return hipGetLastError();
}

}  // namespace mlct
