// Masked attention backward for gfx950.
//
//   D_i  = sum_c dO[i, c] O[i, c]                              (bwd_stats_kernel, HBM-bound)
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
    const _Float16* qh;   // Q * sQ, dO * sO [T][Hq][128], K * sK, V * sV [T][Hk][128] (fp16)
    const _Float16* doh;
    const _Float16* kh;
    const _Float16* vh;
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
    int rev_lists;  // bwd_kernel walks its query lists from their end
    int splits;     // dense dK/dV: pieces per key tile (dkdv_splits)
    float* part;    // splits > 1: partial dK [splits][T][Hk][128], then partial dV
};

// Largest power of two s with bound * s <= 2^15 (1 when the bound is 0 or not finite).
__device__ __forceinline__ float pow2_scale(float bound) {
    if (!(bound > 0.f) || isinf(bound)) return 1.f;
    const float e = fminf(fmaxf(floorf(__log2f(32768.f / bound)), -120.f), 120.f);
    return exp2f(e);
}

// The power-of-two scales of the fp16 operands, from the preprocess bounds. dS is bounded
// by 2 max||dO_i|| max||V_j|| (|P| <= 1, |dP_ij| <= ||dO_i|| ||V_j||, |D_i| <= ||dO_i||), so
// dO's scale also keeps dS * sO in range.
struct OperandScales {
    float sQ, sK, sV, sO;
};
__device__ __forceinline__ OperandScales operand_scales(const float* stats) {
    const float nrm_do = sqrtf(stats[ST_DO_NORM2]), nrm_v = sqrtf(stats[ST_V_NORM2]);
    OperandScales r;
    r.sO = pow2_scale(fmaxf(2.f * nrm_do * nrm_v, nrm_do));
    r.sQ = pow2_scale(stats[ST_Q_ABS]);
    r.sK = pow2_scale(stats[ST_K_ABS]);
    r.sV = pow2_scale(nrm_v);
    return r;
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

// The four bound slots = 0 (a kernel rather than a memset, so the sequence can be captured).
__global__ void zero_stats_kernel(float* __restrict__ stats) {
    if (threadIdx.x < BWD_STATS) stats[threadIdx.x] = 0.f;
}

// One pass over the rows of O, O_lo, dO, Q ([T][Hq][128]) and of K, V ([T][Hk][128]):
//   D[h][i] = sum_c dO[i][h][c] * (O + O_lo)[i][h][c],
//   the bounds max_i ||dO_i||^2, max |Q|, max |K|, max_j ||V_j||^2.
// 16 lanes per row, grid-stride loops over groups of 16 rows (their bounds are uniform over
// the workgroup, so every lane reaches the shuffles); each workgroup then reduces its four
// maxima and raises the slots to them with one conditional atomic max each.
__global__ __launch_bounds__(256) void bwd_stats_kernel(const bf16* __restrict__ o, const bf16* __restrict__ o_lo,
                                                        const bf16* __restrict__ dout, const bf16* __restrict__ q,
                                                        const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                        float* __restrict__ dbuf, float* __restrict__ stats, int T,
                                                        int Hq, int Hk) {
    const int part = threadIdx.x & 15;
    float b_do = 0.f, b_q = 0.f, b_k = 0.f, b_v = 0.f;
    const long nq = (long)T * Hq, nk = (long)T * Hk;
    for (long base = (long)blockIdx.x * 16; base < nq; base += (long)gridDim.x * 16) {
        const long row = base + (threadIdx.x >> 4);
        float sd = 0.f, n2 = 0.f;
        if (row < nq) {
            const size_t off = (size_t)row * HEAD_DIM + part * 8;
            const u32x4 x = *reinterpret_cast<const u32x4*>(o + off);
            const u32x4 y = *reinterpret_cast<const u32x4*>(dout + off);
            const u32x4 qq = *reinterpret_cast<const u32x4*>(q + off);
            u32x4 z = {0u, 0u, 0u, 0u};
            if (o_lo) z = *reinterpret_cast<const u32x4*>(o_lo + off);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float d0 = bf16_lo(y[m]), d1 = bf16_hi(y[m]);
                sd += d0 * (bf16_lo(x[m]) + bf16_lo(z[m])) + d1 * (bf16_hi(x[m]) + bf16_hi(z[m]));
                n2 += d0 * d0 + d1 * d1;
                b_q = fmaxf(b_q, fmaxf(fabsf(bf16_lo(qq[m])), fabsf(bf16_hi(qq[m]))));
            }
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {
            sd += __shfl_xor(sd, off);
            n2 += __shfl_xor(n2, off);
        }
        if (part == 0 && row < nq) {
            const int pos = (int)(row / Hq), head = (int)(row % Hq);
            dbuf[(size_t)head * T + pos] = sd;
        }
        b_do = fmaxf(b_do, n2);
    }
    for (long base = (long)blockIdx.x * 16; base < nk; base += (long)gridDim.x * 16) {
        const long row = base + (threadIdx.x >> 4);
        float n2 = 0.f;
        if (row < nk) {
            const size_t off = (size_t)row * HEAD_DIM + part * 8;
            const u32x4 kk = *reinterpret_cast<const u32x4*>(k + off);
            const u32x4 vv = *reinterpret_cast<const u32x4*>(v + off);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                b_k = fmaxf(b_k, fmaxf(fabsf(bf16_lo(kk[m])), fabsf(bf16_hi(kk[m]))));
                n2 += bf16_lo(vv[m]) * bf16_lo(vv[m]) + bf16_hi(vv[m]) * bf16_hi(vv[m]);
            }
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) n2 += __shfl_xor(n2, off);
        b_v = fmaxf(b_v, n2);
    }
    // workgroup maxima (blockDim.x = 256, 4 waves), one conditional atomic per slot
    __shared__ float part_max[4][4];
    const float vals[4] = {wave_max(b_do), wave_max(b_v), wave_max(b_q), wave_max(b_k)};
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part_max[j][threadIdx.x >> 6] = vals[j];
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        const int j = threadIdx.x;   // ST_DO_NORM2, ST_V_NORM2, ST_Q_ABS, ST_K_ABS
        const float m = fmaxf(fmaxf(part_max[j][0], part_max[j][1]), fmaxf(part_max[j][2], part_max[j][3]));
        atomic_max_nonneg(stats + j, m);
    }
}

// 8 bf16 (one 16-byte chunk) -> 8 fp16 scaled by s.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_scaled(u32x4 x, float s) {
    u32x4 r;
#pragma unroll
    for (int m = 0; m < 4; ++m) r[m] = pack_f16(bf16_lo(x[m]) * s, bf16_hi(x[m]) * s);
    return r;
}

// Q, dO, K, V -> fp16 times their scales, once per backward pass (HBM-bound), so the main
// kernels stage their operands by plain copies.
__global__ __launch_bounds__(256) void to_f16_kernel(const u32x4* __restrict__ q, const u32x4* __restrict__ dout,
                                                     const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                     u32x4* __restrict__ qh, u32x4* __restrict__ doh,
                                                     u32x4* __restrict__ kh, u32x4* __restrict__ vh, size_t nq8,
                                                     size_t nk8, const float* __restrict__ stats) {
    const OperandScales sc = operand_scales(stats);
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = i0; i < nq8; i += stride) {
        qh[i] = bf16x8_to_f16x8_scaled(q[i], sc.sQ);
        doh[i] = bf16x8_to_f16x8_scaled(dout[i], sc.sO);
    }
    for (size_t i = i0; i < nk8; i += stride) {
        kh[i] = bf16x8_to_f16x8_scaled(k[i], sc.sK);
        vh[i] = bf16x8_to_f16x8_scaled(v[i], sc.sV);
    }
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

// Work item: NWK blocks of 32 keys of one KV head, 2 * NWK waves. Waves 0..NWK-1 ("A")
// compute S -> P and own dV^T; waves NWK..2*NWK-1 ("B") compute dP, receive P through LDS,
// form dS and own dK^T. Wave w and w + NWK handle the same 32 keys and share a SIMD. All
// products run on fp16 operands (the preprocess's scaled copies of Q, K, V, dO).
//
// The roles run one step apart, so a step (32 query rows) needs a single barrier:
//   step s, A: dV^T += dO_s^T P_s (P_s kept in registers from step s - 1),
//              S and P of step s + 1 (P -> LDS slot (s+1)%2 and registers),
//              stage Q, LSE of step s + 2 into Q slot (s+2)%3, load step s + 2 + PD;
//   step s, B: dS_s = P_s * (dP_s - D_s) with P_s from LDS slot s%2 and dP_s kept in
//              registers from step s - 1, dK^T += Q_s^T dS_s, then dP_{s+1} = dO_{s+1} V^T,
//              stage dO, D of step s + 2 into slot (s+2)%3, load step s + 2 + PD.
// The row loads run PD steps ahead of their stores (PD = 2 for the dense masks, whose
// 256-row tiles stream from HBM, with two register stages; 1 for block-sparse), so a
// load has PD whole steps to arrive before the store waits for it.
// Each wave thus alternates a vector phase with a run of 16 MFMAs, in opposite order to its
// partner on the SIMD: B forms dS while A issues its dV and S MFMAs, and A forms P while B
// issues its dK and dP MFMAs.
// Q_j is read in steps j - 1 (A) and j (B), dO_j in steps j - 1 (B) and j (A), and both are
// written in step j - 2, hence three slots each; P_j is read in step j and written in step
// j - 1, hence two. Every slot is rewritten only after the barrier that ends the last step
// reading its old content.
template <int NWK, bool SPARSE>
__global__ __launch_bounds__(NWK * 128) void bwd_kernel(BwdArgs a) {
    constexpr int NR = NWK * 64;          // threads per role
    constexpr int KEYS = NWK * 32;
    constexpr int CPT = 512 / NR;         // 16-byte chunks per thread per staged row block

    // staged rows: skewed (512-byte pitch) for 4 key blocks; the XOR swizzle (256-byte rows)
    // for 2, whose smaller LDS footprint keeps two work items per CU
    constexpr bool SKEW = NWK == 4;
    constexpr int PITCH = SKEW ? SKEW_PITCH : HEAD_DIM;
    __shared__ __attribute__((aligned(16))) _Float16 Qh[3][32 * PITCH];
    __shared__ __attribute__((aligned(16))) _Float16 dOh[3][32 * PITCH];
    auto roff = [](int q, int col) { return SKEW ? skew_off(q, col) : swz_off(q, col); };
    auto rtr = [](const _Float16* M, int rb16, int c0, int ln) {
        if constexpr (SKEW) return tr_rows_skew(M, rb16, c0, ln);
        else return tr_rows_swz(M, rb16 + 4 * (ln >> 5), rb16 + 8 + 4 * (ln >> 5), c0, ln);
    };
    __shared__ __attribute__((aligned(16))) _Float16 Ps[2][NWK * 2 * 64 * 8]; // [kb][kk][lane][8]
    __shared__ __attribute__((aligned(16))) float lse_s[3][32];
    __shared__ __attribute__((aligned(16))) float dd_s[3][32];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index made uniform (SGPR), so the role branches are scalar branches
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const bool is_a = w < NWK;
    const int kb = is_a ? w : w - NWK;
    const int rt = is_a ? tid : tid - NR;   // thread index within the role
    // Dense masks: workgroups go round-robin to the 8 XCDs, and XCD x takes the key tiles of
    // KV heads x * Hk / 8, x * Hk / 8 + 1, ... one head after another (at Hk = 8: KV head x),
    // so the key tiles running together on an XCD stage one head's Q and dO rows and share
    // them through its L2 (MHA 64:64 at FULL 8K: 5-6 % faster than KV head fastest, which is
    // the same order at Hk = 8 and stays for Hk not a multiple of 8).
    // Block-sparse: KV-head-major, so the whole chip works on one KV head's key blocks at a
    // time and the random lists of all CUs draw on that head's fp16 Q and dO rows (256 MiB
    // at 64K, within the 256 MB Infinity Cache) instead of eight heads' rows at once (one
    // head per XCD, whose L2 serves few of them: the lists share no order).
    int g, y;
    if constexpr (SPARSE) {
        g = (int)blockIdx.x / a.nb;
        y = (int)blockIdx.x % a.nb;
    } else if (a.Hk > 8 && (a.Hk & 7) == 0) {
        const int n = (int)gridDim.x / a.Hk;          // key tiles per KV head
        const int j = (int)blockIdx.x >> 3, hl = j / n;
        g = ((int)blockIdx.x & 7) * (a.Hk >> 3) + hl;
        y = j - hl * n;
    } else {
        g = (int)blockIdx.x % a.Hk;
        y = (int)blockIdx.x / a.Hk;
    }
    const int T = a.T;

    const OperandScales sc = operand_scales(a.stats);
    const float sO = sc.sO, sQ = sc.sQ, sK = sc.sK, sV = sc.sV;
    const float cS = a.c / (sQ * sK);       // exponent scale for the scaled scores
    const float inv_sV = 1.f / sV;

    int key_base, col, piece = 0;
    if constexpr (!SPARSE) {
        const int yy = y / a.splits;        // pieces of one key tile are consecutive items
        piece = y - yy * a.splits;
        const int kt = a.order[yy];
        key_base = kt * KEYS;
        col = kt;
    } else {
        key_base = y * a.sblock;
        col = g * a.nb + y;
    }
    // this item's piece of the key tile's list: entries [lb, le)
    const int lb0 = a.ptr[col], n0 = a.ptr[col + 1] - lb0;
    const int lb = lb0 + (int)((long)piece * n0 / a.splits), le = lb0 + (int)((long)(piece + 1) * n0 / a.splits);
    const int my_key = key_base + kb * 32 + l32;
    const bool key_ok = my_key < T;
    const size_t kv_row = (size_t)a.Hk * HEAD_DIM;

    const int lgRB = SPARSE ? (a.sblock == 128 ? 2 : 1) : 3;   // 32-row blocks per list entry
    const int RB = 1 << lgRB;
    const int nsteps = (le - lb) * RB;

    // K rows (A: B operand of S) or V rows (B: B operand of dP), fp16 scaled
    f16x8 kvf[8];
    {
        const _Float16* rowp = (is_a ? a.kh : a.vh) + (size_t)g * HEAD_DIM + (size_t)min(my_key, T - 1) * kv_row + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4 x = *reinterpret_cast<const u32x4*>(rowp + 16 * ks);
            if (!key_ok) x = u32x4{0u, 0u, 0u, 0u};
            kvf[ks] = as_f16x8(x);
        }
    }
    int4 kd = {0, 0, 0, 0};
    if (!SPARSE && is_a && key_ok) kd = a.desc[my_key];

    // The order of a key tile's query tiles is free. For the masks whose lists are suffixes
    // (CAUSAL, PREFIX LM CAUSAL, SHARED QUESTION) the lists are walked from their end: the
    // key tiles of a KV head that run together then stage the same query rows at about the
    // same time, so the rows are read from L2 instead of once per key tile from memory.
    EntryStream es;           // list entries of the staged row loads (2 + PD steps ahead)
    es.init(a.ent, lb, le - lb, lane, a.rev_lists != 0);
    EntryStream esc;          // A: list entries of the steps whose P it forms
    esc.init(a.ent, lb, le - lb, lane, a.rev_lists != 0);

    // Staging of this role's tensor (A: Q and LSE, B: dO and D). Rows past the end are
    // read from a valid row and get LSE = +inf (P = 0) and D = 0 when stored.
    const _Float16* src = is_a ? a.qh : a.doh;
    const float* ssrc = is_a ? a.lse : a.dbuf;
    const int span = SPARSE ? a.sblock : a.BMq;   // positions per list entry
    // rows in flight: PD register stages, loaded PD steps before they are stored (two for the
    // dense masks, whose long lists of 256-row tiles stream from HBM; one for block-sparse,
    // where the b = 64 instance is at the two-waves-per-SIMD register limit and b = 128 gains
    // nothing)
    constexpr int PD = (NWK == 4 && !SPARSE) ? 2 : 1;
    using Second = BoolTag<PD == 2>;   // register stage of odd steps
    u32x4 pre[2][CPT];
    float praw[2] = {0.f, 0.f};
    bool pvalid[2] = {false, false};
    auto load_rows = [&](int st, auto bt) {
        constexpr int BUF = decltype(bt)::value;
        const int e = es.get(st >> lgRB, lane), rb = st & (RB - 1);
        const RowMap m = row_map<SPARSE>(a, g, e);
        if (m.pbase + span <= T) {
            // one base per step plus small per-lane offsets
            const _Float16* base = src + ((size_t)m.pbase * a.Hq + m.hbase) * HEAD_DIM;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = rt + i * NR, R = rb * 32 + (c >> 4);
                const unsigned off = (unsigned)((((R & m.mask) * a.Hq + (R >> m.lg)) * HEAD_DIM) + (c & 15) * 8);
                pre[BUF][i] = *reinterpret_cast<const u32x4*>(base + off);
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = rt + i * NR, R = rb * 32 + (c >> 4);
                const int p = min(m.pos(R), T - 1);
                pre[BUF][i] = *reinterpret_cast<const u32x4*>(src + ((size_t)p * a.Hq + m.head(R)) * HEAD_DIM + (c & 15) * 8);
            }
        }
        if (rt < 32) {
            const int R = rb * 32 + rt, p = m.pos(R);
            pvalid[BUF] = p < T;
            praw[BUF] = ssrc[(size_t)m.head(R) * T + min(p, T - 1)];
        }
    };
    auto store_rows = [&](int slot, auto bt) {
        constexpr int BUF = decltype(bt)::value;
        _Float16* dst = is_a ? Qh[slot] : dOh[slot];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = rt + i * NR;
            *reinterpret_cast<u32x4*>(&dst[roff(c >> 4, (c & 15) * 8)]) = pre[BUF][i];
        }
        if (rt < 32) {
            if (is_a)
                lse_s[slot][rt] = (!pvalid[BUF] || praw[BUF] == -INFINITY) ? INFINITY : praw[BUF] * LOG2E;
            else
                dd_s[slot][rt] = pvalid[BUF] ? praw[BUF] * sO : 0.f;
        }
    };
    constexpr BoolTag<false> B0{};

    // A: S = Q K^T and P for step st (entry e) from Q slot qs; P -> LDS slot st % 2 and pb.
    // P slots (hf, e) of 16-row step kk are rows 16*kk + 8*(e/4) + 4*hf + e%4.
    auto s_and_p = [&](int st, int e, int qs, f16x8 (&pb)[2]) {
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        const _Float16* qh = Qh[qs];
        mfma_pipelined<8>(
            [&](int ks) { return *reinterpret_cast<const u32x4*>(&qh[roff(l32, 16 * ks + 8 * hf)]); },
            [&](int ks, u32x4 op) { sacc = mfma32h(as_f16x8(op), kvf[ks], sacc); });
        const bool full = SPARSE ? true : ((e & 1) != 0);
        const bool all_vis = full && key_base + KEYS <= T;   // no element of the step masked
        uint32_t vis = key_ok ? 0xffffu : 0u;
        if (!full && key_ok) {
            const RowMap rm = row_map<SPARSE>(a, g, e);
            const int rb = st & (RB - 1);
            if (rm.mask >= 31) {
                // the step's 32 rows are 32 consecutive positions from p0: this key's two
                // row intervals as a bit mask over them, then the lane's 16 rows
                // (bits 8q + 4hf + i, q, i < 4) packed into bits 4q + i
                const int p0 = rm.pbase + ((rb * 32) & rm.mask);
                uint32_t m = (interval_bits(kd.x, kd.y, p0) | interval_bits(kd.z, kd.w, p0)) >> (4 * hf);
                m &= 0x0F0F0F0Fu;
                m = (m | (m >> 4)) & 0x00FF00FFu;
                vis = (m | (m >> 8)) & 0xFFFFu;
            } else {
                vis = 0u;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int p = rm.pos(rb * 32 + acc_row(r, hf));
                    const bool v = (p >= kd.x && p < kd.y) || (p >= kd.z && p < kd.w);
                    vis |= (uint32_t)v << r;
                }
            }
        }
        _Float16* ps = Ps[st & 1];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float4 l0 = *reinterpret_cast<const float4*>(&lse_s[qs][16 * kk + 4 * hf]);
            const float4 l1 = *reinterpret_cast<const float4*>(&lse_s[qs][16 * kk + 8 + 4 * hf]);
            const float lr[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            u32x4 pk;
            if (all_vis) {
#pragma unroll
                for (int e2 = 0; e2 < 8; e2 += 2) {
                    const int r0 = kk * 8 + e2;
                    pk[e2 >> 1] = pack_f16(fast_exp2(fmaf(sacc[r0], cS, -lr[e2])),
                                           fast_exp2(fmaf(sacc[r0 + 1], cS, -lr[e2 + 1])));
                }
            } else {
#pragma unroll
                for (int e2 = 0; e2 < 8; e2 += 2) {
                    const int r0 = kk * 8 + e2, r1 = r0 + 1;
                    const float p0 = fast_exp2(fmaf(sacc[r0], cS, -lr[e2]));
                    const float p1 = fast_exp2(fmaf(sacc[r1], cS, -lr[e2 + 1]));
                    pk[e2 >> 1] = pack_f16(((vis >> r0) & 1u) ? p0 : 0.f, ((vis >> r1) & 1u) ? p1 : 0.f);
                }
            }
            pb[kk] = as_f16x8(pk);
            *reinterpret_cast<u32x4*>(&ps[((kb * 2 + kk) * 64 + lane) * 8]) = pk;
        }
    };

    f32x16 acc[4];   // A: dV^T, B: dK^T (dims db*32 + acc_row(r, hf), key = lane column)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    // B: dP = (dO * sO) V^T of the rows in dO slot os (scaled by sO * sV)
    auto dp_of = [&](int os) {
        f32x16 d;
#pragma unroll
        for (int r = 0; r < 16; ++r) d[r] = 0.f;
        const _Float16* doh = dOh[os];
        mfma_pipelined<8>(
            [&](int ks) { return *reinterpret_cast<const u32x4*>(&doh[roff(l32, 16 * ks + 8 * hf)]); },
            [&](int ks, u32x4 op) { d = mfma32h(as_f16x8(op), kvf[ks], d); });
        return d;
    };

    // prologue: A stages Q_0 and Q_1, B stages dO_0 and dO_1; then A forms P_0 and B dP_0,
    // and both load the rows of step 2
    if (nsteps > 0) {
        load_rows(0, B0);
        store_rows(0, B0);
        if (nsteps > 1) {
            load_rows(1, Second{});
            store_rows(1, Second{});
        }
    }
    lds_barrier();
    f16x8 pb_cur[2];   // A: P of the step being finished
    f32x16 dpacc;      // B: dP of the step being finished
    if (nsteps > 0) {
        // settle the one-time loads here, so no step waits for them behind its prefetches
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (is_a) s_and_p(0, esc.get(0, lane), 0, pb_cur);
        else dpacc = dp_of(0);
        // register stage (s % PD) holds the rows of step s + 2 at the top of step s
        if (nsteps > 2) load_rows(2, B0);
        if (PD == 2 && nsteps > 3) load_rows(3, Second{});
    }
    lds_barrier();

    if (is_a) {
        int qs1 = 1;   // Q slot of step s + 1
        int os = 0;    // dO slot of step s
        auto a_step = [&](int step, auto bt) {
            // dV^T += (dO * sO)^T P of this step first (P from the previous step), then S and
            // P of the next step: the exponentials then run while the B wave on the same SIMD
            // issues its dK and dP MFMAs, and B's dS work while this wave issues MFMAs
            const _Float16* doh = dOh[os];
            mfma_pipelined<8>(
                [&](int i) { return rtr(doh, 16 * (i & 1), (i >> 1) * 32, lane); },
                [&](int i, u32x4 op) { acc[i >> 1] = mfma32h(as_f16x8(op), pb_cur[i & 1], acc[i >> 1]); });
            if (step + 1 < nsteps) s_and_p(step + 1, esc.get((step + 1) >> lgRB, lane), qs1, pb_cur);

            const int qs2 = qs1 == 2 ? 0 : qs1 + 1;   // Q slot of step s + 2
            if (step + 2 < nsteps) store_rows(qs2, bt);
            if (step + 2 + PD < nsteps) load_rows(step + 2 + PD, bt);
            qs1 = qs2;
            os = os == 2 ? 0 : os + 1;
            lds_barrier();
        };
        for (int step = 0; step < nsteps; step += 2) {
            a_step(step, B0);
            if (step + 1 < nsteps) a_step(step + 1, Second{});
        }
    } else {
        int qs0 = 0;   // Q and dO slot of step s
        auto b_step = [&](int step, auto bt) {
            const int cb = step & 1;
            // dS * sO = P * (dP * sO - D * sO); dK^T += (Q * sQ)^T (dS * sO)
            f16x8 sb[2];
            const _Float16* ps = Ps[cb];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const f16x8 ph = as_f16x8(*reinterpret_cast<const u32x4*>(&ps[((kb * 2 + kk) * 64 + lane) * 8]));
                const float4 d0v = *reinterpret_cast<const float4*>(&dd_s[qs0][16 * kk + 4 * hf]);
                const float4 d1v = *reinterpret_cast<const float4*>(&dd_s[qs0][16 * kk + 8 + 4 * hf]);
                const float dr[8] = {d0v.x, d0v.y, d0v.z, d0v.w, d1v.x, d1v.y, d1v.z, d1v.w};
                // (dP - D) in fp32, rounded to fp16, times P in packed fp16
                f16x8 sk;
#pragma unroll
                for (int e2 = 0; e2 < 8; e2 += 2) {
                    const int r0 = kk * 8 + e2, r1 = r0 + 1;
                    f16x2 t, pp;
                    t[0] = (_Float16)fmaf(dpacc[r0], inv_sV, -dr[e2]);
                    t[1] = (_Float16)fmaf(dpacc[r1], inv_sV, -dr[e2 + 1]);
                    pp[0] = ph[e2];
                    pp[1] = ph[e2 + 1];
                    const f16x2 x = t * pp;
                    sk[e2] = x[0];
                    sk[e2 + 1] = x[1];
                }
                sb[kk] = sk;
            }
            const _Float16* qh = Qh[qs0];
            mfma_pipelined<8>(
                [&](int i) { return rtr(qh, 16 * (i & 1), (i >> 1) * 32, lane); },
                [&](int i, u32x4 op) { acc[i >> 1] = mfma32h(as_f16x8(op), sb[i & 1], acc[i >> 1]); });
            const int qs1 = qs0 == 2 ? 0 : qs0 + 1, qs2 = qs1 == 2 ? 0 : qs1 + 1;
            // dP of the next step (its dO rows were staged a step earlier)
            if (step + 1 < nsteps) dpacc = dp_of(qs1);
            if (step + 2 < nsteps) store_rows(qs2, bt);
            if (step + 2 + PD < nsteps) load_rows(step + 2 + PD, bt);
            qs0 = qs1;
            lds_barrier();
        };
        for (int step = 0; step < nsteps; step += 2) {
            b_step(step, B0);
            if (step + 1 < nsteps) b_step(step + 1, Second{});
        }
    }

    if (key_ok) {
        const float unscale = is_a ? 1.f / sO : a.scale / (sQ * sO);
        // split key tiles write their piece's partial sums, which dkdv_reduce_kernel adds up
        float* dst = is_a ? a.dv : a.dk;
        if (!SPARSE && a.splits > 1)
            dst = a.part + ((size_t)(is_a ? a.splits : 0) + piece) * ((size_t)T * kv_row);
        float* outp = dst + (size_t)my_key * kv_row + (size_t)g * HEAD_DIM;
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
// and dS^T straight from the accumulators as the B operand. Operands are the preprocess's
// fp16 copies, scaled by the same powers of two as in the dK/dV kernel.
//
// K, V and the column descriptors are double-buffered in LDS: while tile t is computed
// from slot t % 2, tile t + 1 (loaded one tile earlier) is stored into the other slot and
// the loads of tile t + 2 are issued; one barrier per tile.
//
// PAIR (block-sparse, b = 64, four waves): one work item is query blocks 2p (waves 0, 1)
// and 2p + 1 (waves 2, 3) of one head, walking the union of their two ascending key lists
// so that a key block both keep is staged once; each staged tile is computed by the waves
// whose block keeps it (uniform per wave; every wave runs every iteration and barrier).
template <int NW, bool SPARSE, bool PAIR = false>
__global__ __launch_bounds__(NW * 64) void dq_kernel(BwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int CPT = 1024 / NT;               // 16-byte chunks per thread per tile per tensor
    constexpr int TPE = PAIR ? 1 : SPARSE ? NW / 2 : 1;   // 64-key tiles per list entry

    // Padded rows (fp16 per row): K is read as rows (S^T) and transposed (dQ^T), V as rows
    // only. Every operand read is a per-lane base plus a compile-time offset, which measured
    // faster than an XOR swizzle of 256-byte rows (whose lane-dependent addresses cost
    // vector instructions). No stride serves both of K's patterns at full rate: 152 keeps its
    // row reads conflict-free and its transposed reads 2-way (160 would free the transposed
    // reads and make the row reads 4-way); V's 136 is conflict-free for row reads.
    constexpr int KLD = HEAD_DIM + 24, VLD = HEAD_DIM + 8;
    __shared__ __attribute__((aligned(16))) _Float16 Kh[2][FWD_BN * KLD];
    __shared__ __attribute__((aligned(16))) _Float16 Vh[2][FWD_BN * VLD];
    __shared__ int4 Ds[2][FWD_BN];
    __shared__ __attribute__((aligned(16))) uint32_t Mb[NW][FWD_BN];   // per wave: key -> position bits

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int g = blockIdx.x % a.Hk, y = blockIdx.x / a.Hk;
    const int T = a.T;

    const OperandScales sc = operand_scales(a.stats);
    const float sO = sc.sO, sQ = sc.sQ, sK = sc.sK, sV = sc.sV;
    const float cS = a.c / (sQ * sK);
    const float inv_sV = 1.f / sV;

    int head, pos, lb, le, le2 = 0;
    int p_base = 0;   // the wave's rows cover positions p_base + (0 .. 31) (dense masks)
    if constexpr (!SPARSE) {
        const int qt = a.order[y];
        const int R = w * 32 + l32;
        head = g * a.G + (R >> a.lgBMq);
        pos = qt * a.BMq + (R & (a.BMq - 1));
        p_base = qt * a.BMq + ((w * 32) & (a.BMq - 1));
        lb = a.ptr[qt];
        le = a.ptr[qt + 1];
    } else {
        const int span = PAIR ? (a.nb + 1) >> 1 : a.nb;   // work items per head
        const int hi = y / span, item = y - hi * span;
        const int qb = PAIR ? 2 * item + (w >> 1) : item;
        head = g * a.G + hi;
        pos = qb * a.sblock + (PAIR ? (w & 1) : w) * 32 + l32;
        const int r = head * a.nb + (PAIR ? 2 * item : item);
        lb = a.ptr[r];
        le = a.ptr[r + 1];
        // PAIR: the second block's list follows the first's in the CSR; empty when the
        // pair's second block lies past the last one
        le2 = (PAIR && 2 * item + 1 < a.nb) ? a.ptr[r + 2] : le;
    }
    const bool row_ok = pos < T;
    const int ntiles = (le - lb) * TPE;   // (not PAIR: there the union's length is found while walking)

    // this lane's row: LSE (base 2), D * sO, Q * sQ and dO * sO as B operands
    float lse2 = INFINITY, dd = 0.f;
    f16x8 qf[8], df[8];
    {
        const size_t ro = ((size_t)min(pos, T - 1) * a.Hq + head) * HEAD_DIM + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = as_f16x8(*reinterpret_cast<const u32x4*>(a.qh + ro + 16 * ks));
            df[ks] = as_f16x8(*reinterpret_cast<const u32x4*>(a.doh + ro + 16 * ks));
        }
        const float l = a.lse[(size_t)head * T + min(pos, T - 1)];
        const float d = a.dbuf[(size_t)head * T + min(pos, T - 1)];
        // rows past the end: P = 0
        lse2 = (!row_ok || l == -INFINITY) ? INFINITY : l * LOG2E;
        dd = row_ok ? d * sO : 0.f;
    }

    f32x16 acc[4];   // dQ^T: dims db*32 + acc_row(r, hf), query = lane column
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    const _Float16* kbase = a.kh + (size_t)g * HEAD_DIM;
    const _Float16* vbase = a.vh + (size_t)g * HEAD_DIM;
    const size_t kv_row = (size_t)a.Hk * HEAD_DIM;

    EntryStream es;
    es.init(a.ent, lb, le - lb, lane);
    // first key and "needs per-element masking" of tiles t (cur) and t + 1 (nxt)
    int key0_cur = 0, key0_nxt = 0;
    bool mask_cur = false, mask_nxt = false;
    // PAIR: second list, entries consumed of each list, tiles issued, and whether block 2p
    // (a) / 2p + 1 (b) keeps tiles t (cur) and t + 1 (nxt)
    EntryStream es2;
    const int na = le - lb, nb2 = le2 - le;
    int ia = 0, ib = 0, issued = 0;
    if constexpr (PAIR) es2.init(a.ent, le, nb2, lane);
    bool ka_cur = true, ka_nxt = true, kb_cur = true, kb_nxt = true;

    // Rows past the end are read from row T - 1 (finite data; such keys are masked).
    u32x4 kreg[CPT], vreg[CPT];
    int4 dreg = {0, 0, 0, 0};
    bool dzero = false;
    // the fixed part of each chunk's offset: chunk c = tid + i * NT is row c / 16 of the
    // tile, dims 8 (c % 16) .. + 7
    unsigned lofs[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        lofs[i] = (unsigned)((c >> 4) * kv_row + (c & 15) * 8);
    }
    auto load_tile = [&](int t) {
        int e;
        if constexpr (PAIR) {
            // the smaller head of the two lists (uniform: read through readlane)
            const int ea = ia < na ? es.get(ia, lane) : 0x7fffffff;
            const int eb = ib < nb2 ? es2.get(ib, lane) : 0x7fffffff;
            e = min(ea, eb);
            ka_cur = ka_nxt;
            kb_cur = kb_nxt;
            ka_nxt = ea == e;
            kb_nxt = eb == e;
            ia += ka_nxt;
            ib += kb_nxt;
            ++issued;
        } else {
            e = es.get(t / TPE, lane);
        }
        int key0;
        bool full;
        if constexpr (SPARSE) {
            key0 = e * a.sblock + (t % TPE) * FWD_BN;
            full = true;
        } else {
            key0 = (e >> 1) * FWD_BN;
            full = (e & 1) != 0;
        }
        key0_cur = key0_nxt;
        mask_cur = mask_nxt;
        key0_nxt = key0;
        mask_nxt = !full || key0 + FWD_BN > T;
        const int k0u = __builtin_amdgcn_readfirstlane(key0);
        if (k0u + FWD_BN <= T) {
            // a whole tile: uniform tile base plus the lane's fixed offsets
            const _Float16* kt0 = kbase + (size_t)k0u * kv_row;
            const _Float16* vt0 = vbase + (size_t)k0u * kv_row;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                kreg[i] = *reinterpret_cast<const u32x4*>(kt0 + lofs[i]);
                vreg[i] = *reinterpret_cast<const u32x4*>(vt0 + lofs[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = tid + i * NT, key = min(key0 + (c >> 4), T - 1);
                const size_t o = (size_t)key * kv_row + (c & 15) * 8;
                kreg[i] = *reinterpret_cast<const u32x4*>(kbase + o);
                vreg[i] = *reinterpret_cast<const u32x4*>(vbase + o);
            }
        }
        if (!SPARSE && tid < FWD_BN) {
            const int key = key0 + tid;
            dreg = a.desc[min(key, T - 1)];
            dzero = key >= T;
        }
    };
    auto store_tile = [&](int slot) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT, row = c >> 4, d0 = (c & 15) * 8;
            *reinterpret_cast<u32x4*>(&Kh[slot][row * KLD + d0]) = kreg[i];
            *reinterpret_cast<u32x4*>(&Vh[slot][row * VLD + d0]) = vreg[i];
        }
        if (!SPARSE && tid < FWD_BN) Ds[slot][tid] = dzero ? int4{0, 0, 0, 0} : dreg;
    };

    // PAIR: entries left in either list (uniform)
    auto more = [&]() { return ia < na || ib < nb2; };
    if (PAIR ? more() : ntiles > 0) {
        load_tile(0);
        store_tile(0);
        if (PAIR ? more() : ntiles > 1) load_tile(1);
    }
    lds_barrier();

    for (int t = 0; PAIR ? t < issued : t < ntiles; ++t) {
        const int cb = t & 1;
        const bool have1 = PAIR ? t + 1 < issued : t + 1 < ntiles;   // tile t + 1 exists
        const int key0 = have1 ? key0_cur : key0_nxt;
        const bool need_mask = have1 ? mask_cur : mask_nxt;
        const bool mine = (w >> 1) == 0 ? (have1 ? ka_cur : ka_nxt) : (have1 ? kb_cur : kb_nxt);
        const _Float16* kt = Kh[cb];
        const _Float16* vt = Vh[cb];
        if (!SPARSE && need_mask) {
            // lane j: key j's two row intervals as a bit mask over the wave's positions
            const int4 d = Ds[cb][lane];
            Mb[w][lane] = interval_bits(d.x, d.y, p_base) | interval_bits(d.z, d.w, p_base);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's masks written
        }
        // per 32-key half kb: S^T = K Q^T and dP^T = V dO^T (lane column = its query row,
        // rows = keys), dS^T, then dQ^T += (K * sK)^T (dS^T * sO) for those 32 keys
        if (!PAIR || mine) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 st, dpt;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    st[r] = 0.f;
                    dpt[r] = 0.f;
                }
                mfma_pipelined<16>(
                    [&](int i) {
                        const int r = kb * 32 + l32, c = 16 * (i >> 1) + 8 * hf;
                        return *reinterpret_cast<const u32x4*>((i & 1) ? vt + r * VLD + c : kt + r * KLD + c);
                    },
                    [&](int i, u32x4 op) {
                        if (i & 1) dpt = mfma32h(as_f16x8(op), df[i >> 1], dpt);
                        else st = mfma32h(as_f16x8(op), qf[i >> 1], st);
                    });
                // dS^T * sO = P^T * (dP^T * sO - D * sO), as B operands of two 16-key steps;
                // key slot (hf, e) of step kk is key kb*32 + 16*kk + 8*(e/4) + 4*hf + e%4
                f16x8 sb[2];
                // two copies of the element loop, so that a FULL tile carries no mask test
                auto form_ds = [&](auto masked_tag) {
                    constexpr bool masked = decltype(masked_tag)::value;
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
                                float p = fast_exp2(fmaf(st[r], cS, -lse2));
                                if constexpr (masked) {
                                    bool vis;
                                    if constexpr (SPARSE) vis = key0 + kidx < T;
                                    else vis = (int)(Mb[w][kidx] << (31 - (pos - p_base))) < 0;
                                    p = vis ? p : 0.f;
                                }
                                v2[j] = p * fmaf(dpt[r], inv_sV, -dd);
                            }
                            pk[e2 >> 1] = pack_f16(v2[0], v2[1]);
                        }
                        sb[kk] = as_f16x8(pk);
                    }
                };
                if (need_mask) form_ds(BoolTag<true>{});
                else form_ds(BoolTag<false>{});
                mfma_pipelined<8>(
                    [&](int i) {
                        const int k0 = kb * 32 + 16 * (i & 1) + 4 * hf;
                        return tr_rows_ld(kt, KLD, k0, k0 + 8, (i >> 1) * 32, lane);
                    },
                    [&](int i, u32x4 op) { acc[i >> 1] = mfma32h(as_f16x8(op), sb[i & 1], acc[i >> 1]); });
            }
        }
        // tile t + 1 into the other slot (its readers of tile t - 1 passed the last
        // barrier), loads of tile t + 2
        if (have1) store_tile(cb ^ 1);
        if (PAIR ? more() : t + 2 < ntiles) load_tile(t + 2);
        lds_barrier();
    }

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

// dK and dV of split key tiles: the sum of the S partial results, in piece order (n4 = T * Hk *
// 128 / 4 float4 per tensor; part holds dK's S pieces, then dV's).
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float4* __restrict__ part, float4* __restrict__ dk,
                                                          float4* __restrict__ dv, size_t n4, int S) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        float4 a = part[i], b = part[(size_t)S * n4 + i];
        for (int p = 1; p < S; ++p) {
            const float4 x = part[(size_t)p * n4 + i], y = part[(size_t)(S + p) * n4 + i];
            a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
            b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
        }
        dk[i] = a;
        dv[i] = b;
    }
}

int launch_bwd_pre(const Problem& P, const void* q, const void* k, const void* v, const void* o,
                   const void* o_lo, const void* dout, float* dbuf, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const BwdLayout W = bwd_layout(P.Hq, P.Hk, P.T, dkdv_splits(P));
    char* ws = reinterpret_cast<char*>(dbuf);
    float* stats = reinterpret_cast<float*>(ws + W.stats);
    hipLaunchKernelGGL(zero_stats_kernel, dim3(1), dim3(64), 0, s, stats);
    const long groups = ((long)P.T * P.Hq + 15) / 16;
    hipLaunchKernelGGL(bwd_stats_kernel, dim3((unsigned)(groups < 4096 ? groups : 4096)), dim3(256), 0, s,
                       static_cast<const bf16*>(o), static_cast<const bf16*>(o_lo), static_cast<const bf16*>(dout),
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v), dbuf,
                       stats, P.T, P.Hq, P.Hk);
    const size_t nq8 = (size_t)P.T * P.Hq * HEAD_DIM / 8, nk8 = (size_t)P.T * P.Hk * HEAD_DIM / 8;
    hipLaunchKernelGGL(to_f16_kernel, dim3(2048), dim3(256), 0, s, static_cast<const u32x4*>(q),
                       static_cast<const u32x4*>(dout), static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
                       reinterpret_cast<u32x4*>(ws + W.qh), reinterpret_cast<u32x4*>(ws + W.doh),
                       reinterpret_cast<u32x4*>(ws + W.kh), reinterpret_cast<u32x4*>(ws + W.vh), nq8, nk8, stats);
    return (int)hipGetLastError();
}

int launch_bwd_main(const Problem& P, const void* q, const void* k, const void* v, const float* lse,
                    const void* dout, float* dq, float* dk, float* dv, const int32_t* desc, const void* index,
                    float* dbuf, int parts, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const IndexLayout L = index_layout(P);
    const char* base = static_cast<const char*>(index);
    BwdArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.dout = static_cast<const bf16*>(dout);
    a.lse = lse;
    a.dbuf = dbuf;
    const int S = dkdv_splits(P);
    const BwdLayout W = bwd_layout(P.Hq, P.Hk, P.T, S);
    char* ws = reinterpret_cast<char*>(dbuf);
    a.stats = reinterpret_cast<const float*>(ws + W.stats);
    a.qh = reinterpret_cast<const _Float16*>(ws + W.qh);
    a.doh = reinterpret_cast<const _Float16*>(ws + W.doh);
    a.kh = reinterpret_cast<const _Float16*>(ws + W.kh);
    a.vh = reinterpret_cast<const _Float16*>(ws + W.vh);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.desc = reinterpret_cast<const int4*>(desc);
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
    a.rev_lists = !P.sparse && (P.kind == ATTN_MASK_CAUSAL || P.kind == ATTN_MASK_PREFIX_LM_CAUSAL ||
                                P.kind == ATTN_MASK_SHARED_QUESTION);
    a.splits = S;
    a.part = S > 1 ? reinterpret_cast<float*>(ws + W.part) : nullptr;
    if (parts & BWD_PART_DKDV) {
        if (!P.sparse) {
            hipLaunchKernelGGL((bwd_kernel<4, false>), dim3(P.Hk * P.nkt_b * S), dim3(512), 0, s, a);
            if (S > 1) {
                const size_t n4 = (size_t)P.T * P.Hk * HEAD_DIM / 4, nblk = (n4 + 255) / 256;
                hipLaunchKernelGGL(dkdv_reduce_kernel, dim3((unsigned)(nblk < 2048 ? nblk : 2048)), dim3(256), 0, s,
                                   reinterpret_cast<const float4*>(a.part), reinterpret_cast<float4*>(dk),
                                   reinterpret_cast<float4*>(dv), n4, S);
            }
        } else if (P.sblock == 64) {
            hipLaunchKernelGGL((bwd_kernel<2, true>), dim3(P.Hk * P.nb), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((bwd_kernel<4, true>), dim3(P.Hk * P.nb), dim3(512), 0, s, a);
        }
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
    }
    if (!(parts & BWD_PART_DQ)) return 0;

    // dQ pass on the forward's lists
    BwdArgs b = a;
    b.ptr = reinterpret_cast<const int*>(base + L.fwd_ptr);
    b.ent = reinterpret_cast<const int*>(base + L.fwd_ent);
    b.order = P.sparse ? nullptr : reinterpret_cast<const int*>(base + L.fwd_order);
    b.BMq = P.fBM;
    if (!P.sparse) {
        hipLaunchKernelGGL((dq_kernel<8, false>), dim3(P.Hk * P.nqt_f), dim3(512), 0, s, b);
    } else if (P.sblock == 64) {
        hipLaunchKernelGGL((dq_kernel<4, true, true>), dim3(P.Hk * P.G * ((P.nb + 1) / 2)), dim3(256), 0, s, b);
    } else {
        hipLaunchKernelGGL((dq_kernel<4, true>), dim3(P.Hk * P.G * P.nb), dim3(256), 0, s, b);
    }
    return (int)hipGetLastError();
}

int launch_cast_bf16(const float* in, void* out, size_t n, void* stream) {
    hipLaunchKernelGGL(cast_kernel, dim3(2048), dim3(256), 0, static_cast<hipStream_t>(stream), in,
                       static_cast<uint16_t*>(out), n);
    return (int)hipGetLastError();
}

}  // namespace mlct
