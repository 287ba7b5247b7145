// Masked attention backward for gfx950.
//
//   D_i  = sum_c dO[i, c] O[i, c]                              (bwd_pre_kernel, HBM-bound)
//   P    = exp(scale * Q K^T - LSE)  on the non-empty tiles    (recomputed)
//   dV  += P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//   dK  += scale * dS^T Q,  dQ += scale * dS K                 (bwd_kernel)
//
// Work item = one workgroup = 32 * NW keys of one KV head. Each wave keeps its 32 keys'
// K and V rows in registers (B operands) and accumulates dK^T, dV^T for them over every
// non-empty query tile of the key tile's list and every query head of the group, so dK
// and dV are written once, without atomics. Query rows are processed 32 at a time: Q
// and dO are staged in LDS in natural layout (A operands of S and dP) and transposed
// (A operands of dK^T and dV^T); S is computed untransposed so P and dS come out of the
// accumulators already in the B-operand layout of the dK^T/dV^T products. dS goes
// through LDS once more for dQ = dS K (K^T kept in LDS for the whole work item); the dQ
// partial of each row block is added to the fp32 output with hardware float atomics.
#include "common.h"

namespace mlct {

constexpr int QS_LD = HEAD_DIM + 8;   // bf16 per Q / dO row in LDS
constexpr int QT_LD = 32 + 8;         // bf16 per Q^T / dO^T row (32 query rows + pad)

struct BwdArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const bf16* dout;
    const float* lse;
    const float* dbuf;   // D [Hq][T]
    float* dq;
    float* dk;
    float* dv;
    const int4* desc;
    const int* ptr;
    const int* ent;
    const int* order;
    int T, Hq, Hk, G, BMq, nb, sblock;
    float c;       // scale * log2(e)
    float scale;
};

// D[h][i] = sum_c dO[i][h][c] * O[i][h][c]; 16 lanes per (position, head) row.
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                      float* __restrict__ dbuf, int T, int Hq) {
    const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int part = threadIdx.x & 15;
    float s = 0.f;
    if (row < (long)T * Hq) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(o + row * HEAD_DIM + part * 8);
        const u32x4 y = *reinterpret_cast<const u32x4*>(dout + row * HEAD_DIM + part * 8);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            s += __uint_as_float(x[m] << 16) * __uint_as_float(y[m] << 16);
            s += __uint_as_float(x[m] & 0xffff0000u) * __uint_as_float(y[m] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (part == 0 && row < (long)T * Hq) {
        const int pos = (int)(row / Hq), head = (int)(row % Hq);
        dbuf[(size_t)head * T + pos] = s;
    }
}

__global__ void zero_kernel(float4* __restrict__ p, size_t n4) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n4; j += stride) p[j] = float4{0.f, 0.f, 0.f, 0.f};
}

__global__ void cast_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t j = i; j < n; j += stride) {
        const __bf16 b = (__bf16)in[j];
        out[j] = __builtin_bit_cast(uint16_t, b);
    }
}

template <int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void bwd_kernel(BwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int KEYS = NW * 32;
    constexpr int KT_LD = KEYS + 8;
    constexpr int DS_LD = KEYS + 8;

    __shared__ __attribute__((aligned(16))) bf16 Kt[HEAD_DIM * KT_LD];
    __shared__ __attribute__((aligned(16))) bf16 Qs[32 * QS_LD];
    __shared__ __attribute__((aligned(16))) bf16 dOs[32 * QS_LD];
    __shared__ __attribute__((aligned(16))) bf16 Qt[HEAD_DIM * QT_LD];
    __shared__ __attribute__((aligned(16))) bf16 dOt[HEAD_DIM * QT_LD];
    __shared__ __attribute__((aligned(16))) bf16 dSs[32 * DS_LD];
    __shared__ float lse_s[32];
    __shared__ float dd_s[32];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int g = blockIdx.x % a.Hk, y = blockIdx.x / a.Hk;
    const int T = a.T;

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

    // K^T of the whole key tile into LDS (B operand of dQ = dS K).
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
                *reinterpret_cast<uint32_t*>(&Kt[(d0 + 2 * m) * KT_LD + 2 * p]) = (x0[m] & 0xffffu) | (x1[m] << 16);
                *reinterpret_cast<uint32_t*>(&Kt[(d0 + 2 * m + 1) * KT_LD + 2 * p]) = (x0[m] >> 16) | (x1[m] & 0xffff0000u);
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

    for (int step = 0; step < nsteps; ++step) {
        const int e = a.ent[lb + step / RB];
        const int rb = step % RB;
        // (head, position) of row q (0..31) of this row block
        int qt = 0, hi = 0, qb = 0;
        bool full;
        if constexpr (SPARSE) {
            hi = e / a.nb;
            qb = e - hi * a.nb;
            full = true;
        } else {
            qt = e >> 1;
            full = (e & 1) != 0;
        }
        auto row_head = [&](int q) -> int {
            if constexpr (SPARSE) return g * a.G + hi;
            else return g * a.G + (rb * 32 + q) / a.BMq;
        };
        auto row_pos = [&](int q) -> int {
            if constexpr (SPARSE) return qb * a.sblock + rb * 32 + q;
            else return qt * a.BMq + (rb * 32 + q) % a.BMq;
        };

        __syncthreads();   // previous row block fully consumed
        // Stage Q and dO rows: natural [q][d] and transposed [d][q].
#pragma unroll
        for (int i = 0; i < 256 / NT; ++i) {
            const int u = tid + i * NT, rp = u & 15, d0 = (u >> 4) * 8;
            const int q0 = 2 * rp, q1 = q0 + 1;
            const int p0 = row_pos(q0), p1 = row_pos(q1);
            const size_t o0 = ((size_t)p0 * a.Hq + row_head(q0)) * HEAD_DIM + d0;
            const size_t o1 = ((size_t)p1 * a.Hq + row_head(q1)) * HEAD_DIM + d0;
            u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u}, y0 = {0u, 0u, 0u, 0u}, y1 = {0u, 0u, 0u, 0u};
            if (p0 < T) {
                x0 = *reinterpret_cast<const u32x4*>(a.q + o0);
                y0 = *reinterpret_cast<const u32x4*>(a.dout + o0);
            }
            if (p1 < T) {
                x1 = *reinterpret_cast<const u32x4*>(a.q + o1);
                y1 = *reinterpret_cast<const u32x4*>(a.dout + o1);
            }
            *reinterpret_cast<u32x4*>(&Qs[q0 * QS_LD + d0]) = x0;
            *reinterpret_cast<u32x4*>(&Qs[q1 * QS_LD + d0]) = x1;
            *reinterpret_cast<u32x4*>(&dOs[q0 * QS_LD + d0]) = y0;
            *reinterpret_cast<u32x4*>(&dOs[q1 * QS_LD + d0]) = y1;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                *reinterpret_cast<uint32_t*>(&Qt[(d0 + 2 * m) * QT_LD + q0]) = (x0[m] & 0xffffu) | (x1[m] << 16);
                *reinterpret_cast<uint32_t*>(&Qt[(d0 + 2 * m + 1) * QT_LD + q0]) = (x0[m] >> 16) | (x1[m] & 0xffff0000u);
                *reinterpret_cast<uint32_t*>(&dOt[(d0 + 2 * m) * QT_LD + q0]) = (y0[m] & 0xffffu) | (y1[m] << 16);
                *reinterpret_cast<uint32_t*>(&dOt[(d0 + 2 * m + 1) * QT_LD + q0]) = (y0[m] >> 16) | (y1[m] & 0xffff0000u);
            }
        }
        if (tid < 32) {
            const int p = row_pos(tid), h = row_head(tid);
            float l2 = INFINITY, dd = 0.f;   // rows past the end: P = 0
            if (p < T) {
                const float lse = a.lse[(size_t)h * T + p];
                l2 = lse == -INFINITY ? INFINITY : lse * LOG2E;   // fully masked row: P = 0
                dd = a.dbuf[(size_t)h * T + p];
            }
            lse_s[tid] = l2;
            dd_s[tid] = dd;
        }
        __syncthreads();

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

        float ds[16];
        bf16x8 pb[2], sb[2];
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
                    bool vis = key_ok;
                    if (!full) {
                        const int p = row_pos(q);
                        vis = vis && ((p >= kd.x && p < kd.y) || (p >= kd.z && p < kd.w));
                    }
                    const float p = vis ? fast_exp2(fmaf(sacc[r], a.c, -lse_s[q])) : 0.f;
                    pv[j] = p;
                    ds[r] = p * (dpacc[r] - dd_s[q]);
                }
                pk[e2 >> 1] = pack_bf16(pv[0], pv[1]);
                sk[e2 >> 1] = pack_bf16(ds[kk * 8 + e2], ds[kk * 8 + e2 + 1]);
            }
            pb[kk] = as_bf16x8(pk);
            sb[kk] = as_bf16x8(sk);
        }

        // dV^T += dO^T P and dK^T += Q^T dS: query slot (hf, e) of step kk is row
        // 16*kk + 8*(e/4) + 4*hf + e%4.
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const bf16* dtr = dOt + (db * 32 + l32) * QT_LD + 4 * hf;
            const bf16* qtr = Qt + (db * 32 + l32) * QT_LD + 4 * hf;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x2 a0 = *reinterpret_cast<const u32x2*>(dtr + 16 * kk);
                const u32x2 a1 = *reinterpret_cast<const u32x2*>(dtr + 16 * kk + 8);
                dv_acc[db] = mfma32(as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]}), pb[kk], dv_acc[db]);
                const u32x2 b0 = *reinterpret_cast<const u32x2*>(qtr + 16 * kk);
                const u32x2 b1 = *reinterpret_cast<const u32x2*>(qtr + 16 * kk + 8);
                dk_acc[db] = mfma32(as_bf16x8(u32x4{b0[0], b0[1], b1[0], b1[1]}), sb[kk], dk_acc[db]);
            }
        }

        // dS (bf16) to LDS as [q][key] for dQ.
#pragma unroll
        for (int r = 0; r < 16; ++r) dSs[acc_row(r, hf) * DS_LD + w * 32 + l32] = (__bf16)ds[r];
        __syncthreads();

        // dQ[q][d] += scale * sum_key dS[q][key] K[key][d]; wave w takes dim blocks w, w + NW, ...
        for (int db = w; db < 4; db += NW) {
            f32x16 qacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) qacc[r] = 0.f;
            const bf16* sr = dSs + l32 * DS_LD + 8 * hf;
            const bf16* kr = Kt + (db * 32 + l32) * KT_LD + 8 * hf;
#pragma unroll
            for (int ks = 0; ks < KEYS / 16; ++ks)
                qacc = mfma32(*reinterpret_cast<const bf16x8*>(sr + 16 * ks),
                              *reinterpret_cast<const bf16x8*>(kr + 16 * ks), qacc);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = acc_row(r, hf);
                const int p = row_pos(q);
                if (p < T)
                    unsafeAtomicAdd(a.dq + ((size_t)p * a.Hq + row_head(q)) * HEAD_DIM + db * 32 + l32,
                                    qacc[r] * a.scale);
            }
        }
    }

    if (key_ok) {
        float* dkp = a.dk + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM;
        float* dvp = a.dv + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = db * 32 + 8 * i4 + 4 * hf;
                *reinterpret_cast<float4*>(dkp + d0) =
                    float4{dk_acc[db][4 * i4] * a.scale, dk_acc[db][4 * i4 + 1] * a.scale,
                           dk_acc[db][4 * i4 + 2] * a.scale, dk_acc[db][4 * i4 + 3] * a.scale};
                *reinterpret_cast<float4*>(dvp + d0) =
                    float4{dv_acc[db][4 * i4], dv_acc[db][4 * i4 + 1], dv_acc[db][4 * i4 + 2], dv_acc[db][4 * i4 + 3]};
            }
    }
}

hipError_t launch_bwd_pre(const Problem& P, const void* o, const void* dout, float* dq, float* dbuf,
                          hipStream_t s) {
    const size_t n4 = (size_t)P.T * P.Hq * HEAD_DIM / 4;
    hipLaunchKernelGGL(zero_kernel, dim3(2048), dim3(256), 0, s, reinterpret_cast<float4*>(dq), n4);
    const long rows = (long)P.T * P.Hq;
    hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s,
                       static_cast<const bf16*>(o), static_cast<const bf16*>(dout), dbuf, P.T, P.Hq);
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
