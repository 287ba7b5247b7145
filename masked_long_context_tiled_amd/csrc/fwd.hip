// Masked attention forward for gfx950.
//
// Work item = one workgroup = 32 * NW (head, position) rows that walk the same list of
// 64-key tiles. Dense masks (fwd_dense_kernel, NW = 8): the rows are the G query heads
// of one KV head times 256/G consecutive positions (one query tile of the tile index),
// so every K/V tile staged in LDS is reused by the whole GQA group. Block-sparse
// (fwd_sparse_kernel, four waves): at b = 128 the rows are one (query head, query block)
// row of the keep matrix; at b = 64 they are two such rows of one head (query blocks 2p
// and 2p + 1), which walk the union of their key lists.
//
// Each wave owns 32 rows and computes the transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in registers), so a lane holds
// one query row and 16 keys per 32-key block: the row max and row sum are mostly
// in-lane, with one exchange between the two wave halves. The probabilities P^T then
// feed O^T += V^T P^T directly as the B operand (no register shuffles); the A operand
// V^T comes from LDS.
//
// Per tile: EMPTY tiles are not in the list; FULL tiles skip all mask work; on PARTIAL
// tiles (and the ragged last tile) each key's two visible row intervals become one bit
// mask over the wave's positions, which every lane tests for its own row (block-sparse
// tiles only mask keys past the end). Online softmax runs in base 2 with a lazy rescale:
// the running max used for the exponent is only raised when a row's new max exceeds it by
// more than 8 (so P <= 2^8), which keeps the O rescale off the common path; O / l and
// LSE = (m + log2 l) * ln 2 are exact whatever max was used.
#include "common.h"

namespace mlct {

constexpr float RESCALE_SLACK = 8.0f; // log2 units the running max may lag behind

struct FwdArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    bf16* o_lo;   // optional: bf16 residual of the fp32 O (O_fp32 - O)
    float* lse;
    const int4* desc;
    const int* ptr;
    const int* ent;
    const int* order;
    int T, Hq, Hk, G, BMq, lgBMq, nb, sblock;
    float c;   // scale * log2(e)
};

// LDS row strides (16-bit elements). The MFMA operand patterns read at full LDS rate only
// at some strides (measured, eight waves per CU): 16-byte row reads (lane l: row l % 32)
// are conflict-free at 8 mod 16 (136, 152, ...; 2-way at 144, 4-way at 160), transposed
// reads of a row-major tile (ds_read_b64_tr_b16: per 16 lanes 4 rows x 16 columns) at 160
// and 224 (about 180 B/clk against 128 at 144..216). K is read as rows only, V (staged
// row-major, V^T read transposed, no transposing stores) transposed only. Every MFMA's LDS
// operand is read three MFMAs ahead.
constexpr int K_LD = HEAD_DIM + 8;    // bf16 per K row in LDS
constexpr int V_LD = HEAD_DIM + 32;   // bf16 per V row in LDS

// Block-sparse work items, four waves: at b = 128 one (query head, query block) row of the
// keep matrix, each list entry a 128-key block walked as two 64-key tiles; at b = 64 (PAIR,
// below) two rows, each list entry one 64-key tile. K and V are staged row-major
// (V^T read with transposed LDS reads, as in the dense kernel), single-buffered with two
// barriers per tile (the small LDS footprint keeps four work items per CU).
//
// PAIR (b = 64, four waves): one work item is query blocks 2p (waves 0, 1) and 2p + 1
// (waves 2, 3) of one head. It walks the union of their two ascending key lists, so a key
// block both keep is staged once; each staged tile is computed by the waves whose query
// block keeps it (the choice is uniform per wave, and the loop's trip count is uniform per
// work item, so every wave meets every barrier).
template <int NW, bool PAIR = false>
__global__ __launch_bounds__(NW * 64) void fwd_sparse_kernel(FwdArgs a) {
    constexpr int NT = NW * 64;
    constexpr int CPT = 1024 / NT;            // 16-byte chunks per thread per tile per tensor
    constexpr int TPE = PAIR ? 1 : NW / 2;    // 64-key tiles per list entry

    __shared__ __attribute__((aligned(16))) bf16 Ks[FWD_BN * K_LD];
    __shared__ __attribute__((aligned(16))) bf16 Vs[FWD_BN * V_LD];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    // 1-D grid, KV head fastest: consecutive workgroups go to different XCDs, so all
    // work items of one KV head share an XCD (and its L2) when Hk is a multiple of 8.
    const int g = blockIdx.x % a.Hk, y = blockIdx.x / a.Hk;
    const int T = a.T;

    const int span = PAIR ? (a.nb + 1) >> 1 : a.nb;   // work items per head
    const int hi = y / span, item = y - hi * span;
    const int sub = PAIR ? w >> 1 : 0;                // PAIR: which block of the pair
    const int qb = PAIR ? 2 * item + sub : item;
    const int head = g * a.G + hi;
    const int pos = qb * a.sblock + (PAIR ? (w & 1) : w) * 32 + l32;
    const int r0 = head * a.nb + (PAIR ? 2 * item : item);
    // the (first) block's list; PAIR: the second block's list follows it in the CSR and is
    // empty when the pair's second block lies past the last one
    const int lb = a.ptr[r0], le = a.ptr[r0 + 1];
    const int le2 = (PAIR && 2 * item + 1 < a.nb) ? a.ptr[r0 + 2] : le;
    const bool row_ok = pos < T;
    const int ntiles = (le - lb) * TPE;   // (not PAIR)

    // Q row fragments: B operand, lane holds dims 16*ks + 8*hf .. +7 of its row; the loads
    // complete before the loop (left pending, the first wait in the loop would also cover
    // the K/V loads issued behind them)
    bf16x8 qf[8];
    {
        const bf16* qp = a.q + ((size_t)min(pos, T - 1) * a.Hq + head) * HEAD_DIM + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * ks));
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(as_u32x4(qf[ks])));
    }

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m2 = -INFINITY, lsum[2] = {0.f, 0.f};

    const bf16* kbase = a.k + (size_t)g * HEAD_DIM;
    const bf16* vbase = a.v + (size_t)g * HEAD_DIM;
    const size_t kv_row = (size_t)a.Hk * HEAD_DIM;

    // list entries from registers filled a chunk of 64 ahead (no tile waits on a freshly
    // loaded entry before it can address its K/V loads)
    EntryStream es, es2;
    es.init(a.ent, lb, le - lb, lane);
    int ia = 0, ib = 0;                    // PAIR: entries of each list consumed
    const int na = le - lb, nb2 = le2 - le;
    if constexpr (PAIR) es2.init(a.ent, le, nb2, lane);
    bool nka = true, nkb = true;           // PAIR: the loaded tile is kept by block 2p / 2p + 1

    // Rows past the end are read from row T - 1 (finite data; such keys are masked).
    u32x4 kreg[CPT], vreg[CPT];
    int nkey0 = 0;
    // the fixed part of each chunk's offset: chunk c = tid + i * NT is row c / 16 of the
    // tile, dims 8 (c % 16) .. + 7 (every instance launched has four waves, so both block
    // sizes use it; a two-wave instance would need eight offsets per thread, which would
    // cost it its second wave per SIMD)
    constexpr bool FIXED_OFS = NW == 4;
    unsigned lofs[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tid + i * NT;
        lofs[i] = FIXED_OFS ? (unsigned)((c >> 4) * kv_row + (c & 15) * 8) : 0u;
    }
    auto load_tile = [&](int t) {
        int e;
        if constexpr (PAIR) {
            // the smaller head of the two lists (uniform: read through readlane)
            const int ea = ia < na ? es.get(ia, lane) : 0x7fffffff;
            const int eb = ib < nb2 ? es2.get(ib, lane) : 0x7fffffff;
            e = min(ea, eb);
            nka = ea == e;
            nkb = eb == e;
            ia += nka;
            ib += nkb;
        } else {
            e = es.get(t / TPE, lane);
        }
        const int k0 = e * a.sblock + (t % TPE) * FWD_BN;
        nkey0 = FIXED_OFS ? __builtin_amdgcn_readfirstlane(k0) : k0;   // uniform either way
        if (FIXED_OFS && nkey0 + FWD_BN <= T) {
            // a whole tile: uniform tile base plus the lane's fixed offsets
            const bf16* kt0 = kbase + (size_t)nkey0 * kv_row;
            const bf16* vt0 = vbase + (size_t)nkey0 * kv_row;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                kreg[i] = *reinterpret_cast<const u32x4*>(kt0 + lofs[i]);
                vreg[i] = *reinterpret_cast<const u32x4*>(vt0 + lofs[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = tid + i * NT, key = min(nkey0 + (c >> 4), T - 1);
                const size_t o = (size_t)key * kv_row + (c & 15) * 8;
                kreg[i] = *reinterpret_cast<const u32x4*>(kbase + o);
                vreg[i] = *reinterpret_cast<const u32x4*>(vbase + o);
            }
        }
    };

    bool have = PAIR ? na + nb2 > 0 : ntiles > 0;
    if (have) load_tile(0);

    for (int t = 0; have; ++t) {
        const int key0 = nkey0;
        const bool need_mask = key0 + FWD_BN > T;
        const bool mine = sub == 0 ? nka : nkb;   // PAIR: this wave's block keeps the tile

        __syncthreads();   // every wave is done reading the previous tile
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT, row = c >> 4, col = (c & 15) * 8;
            *reinterpret_cast<u32x4*>(&Ks[row * K_LD + col]) = kreg[i];
            *reinterpret_cast<u32x4*>(&Vs[row * V_LD + col]) = vreg[i];
        }
        lds_barrier();

        have = PAIR ? (ia < na || ib < nb2) : t + 1 < ntiles;
        if (have) load_tile(t + 1);
        if (PAIR && !mine) continue;

        // S^T = K Q^T for the two 32-key halves of the tile
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const bf16* kr = Ks + l32 * K_LD + 8 * hf;
        mfma_pipelined<16>(
            [&](int i) { return *reinterpret_cast<const u32x4*>(kr + (i & 1) * 32 * K_LD + 16 * (i >> 1)); },
            [&](int i, u32x4 op) { s[i & 1] = mfma32(as_bf16x8(op), qf[i >> 1], s[i & 1]); });

        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // the last tile of the sequence: keys past the end
                    if (key0 + kb * 32 + acc_row(r, hf) >= T) s[kb][r] = -INFINITY;
                }
        }

        // online softmax (base 2), lazy rescale
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2)
                mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[kb][r], s[kb][r + 1]));
        if (__ballot(mx * a.c > m2 + RESCALE_SLACK) != 0ull) {
            mx = fmaxf(mx, swap_halves(mx));
            const float mnew = fmaxf(m2, mx * a.c);
            const float alpha = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mnew);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            lsum[0] *= alpha;
            lsum[1] *= alpha;
            m2 = mnew;
        }
        const float msub = (m2 == -INFINITY) ? 0.f : m2;

        bf16x8 pb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 pk;
#pragma unroll
            for (int e2 = 0; e2 < 8; e2 += 2) {
                const float p0 = fast_exp2(fmaf(s[kk >> 1][(kk & 1) * 8 + e2], a.c, -msub));
                const float p1 = fast_exp2(fmaf(s[kk >> 1][(kk & 1) * 8 + e2 + 1], a.c, -msub));
                lsum[kk & 1] += p0 + p1;
                pk[e2 >> 1] = pack_bf16(p0, p1);
            }
            pb[kk] = as_bf16x8(pk);
        }

        // O^T += V^T P^T: key slot (hf, e) of step kk is key 16*kk + 8*(e/4) + 4*hf + e%4.
        mfma_pipelined<16>(
            [&](int i) {
                const int kk = i >> 2, db = i & 3;
                return tr_rows_ld(Vs, V_LD, 16 * kk + 4 * hf, 16 * kk + 8 + 4 * hf, db * 32, lane);
            },
            [&](int i, u32x4 op) { acc[i & 3] = mfma32(as_bf16x8(op), pb[i >> 2], acc[i & 3]); });
    }

    const float lrow = lsum[0] + lsum[1];
    const float ltot = lrow + swap_halves(lrow);
    if (row_ok) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        bf16* op = a.o + ((size_t)pos * a.Hq + head) * HEAD_DIM;
        bf16* olp = a.o_lo ? a.o_lo + ((size_t)pos * a.Hq + head) * HEAD_DIM : nullptr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = db * 32 + 8 * i4 + 4 * hf;
                const float v0 = acc[db][4 * i4 + 0] * inv, v1 = acc[db][4 * i4 + 1] * inv;
                const float v2 = acc[db][4 * i4 + 2] * inv, v3 = acc[db][4 * i4 + 3] * inv;
                u32x2 pk;
                pk[0] = pack_bf16(v0, v1);
                pk[1] = pack_bf16(v2, v3);
                *reinterpret_cast<u32x2*>(op + d0) = pk;
                if (olp) {
                    u32x2 lo;
                    lo[0] = pack_bf16(v0 - bf16_lo(pk[0]), v1 - bf16_hi(pk[0]));
                    lo[1] = pack_bf16(v2 - bf16_lo(pk[1]), v3 - bf16_hi(pk[1]));
                    *reinterpret_cast<u32x2*>(olp + d0) = lo;
                }
            }
        if (hf == 0)
            a.lse[(size_t)head * T + pos] = ltot > 0.f ? (m2 + fast_log2(ltot)) * LN2 : -INFINITY;
    }
}

// Dense work items (the G heads of one KV head x 256/G positions, 8 waves of 32 rows).
// Same arithmetic as fwd_sparse_kernel, with these differences:
//  - K, V and the column descriptors are double-buffered in LDS by stages of two
//    64-key tiles (two list entries): while stage u is computed from slot u % 2, stage
//    u + 1 (loaded one stage earlier) is stored into the other slot and the loads of stage
//    u + 2 are issued; one barrier per stage;
//  - PARTIAL tiles are masked through per-key bit masks over the wave's positions;
//  - list entries are read from registers filled a chunk ahead, so no load waits on a
//    freshly loaded entry;
//  - the in-lane row max covers half of a row's keys; the two halves are combined only
//    when the running max has to move (the lazy rescale).
__global__ __launch_bounds__(512) void fwd_dense_kernel(FwdArgs a) {
    constexpr int NT = 512;
    constexpr int SUB = 2;                   // list entries (64-key tiles) staged together
    constexpr int CPT = SUB * 1024 / NT;     // 16-byte chunks per thread per stage per tensor

    __shared__ __attribute__((aligned(16))) bf16 Kb[2][SUB * FWD_BN * K_LD];
    __shared__ __attribute__((aligned(16))) bf16 Vb[2][SUB * FWD_BN * V_LD];
    __shared__ int4 Db[2][SUB * FWD_BN];
    __shared__ __attribute__((aligned(16))) uint32_t Mb[8][FWD_BN];   // per wave: key -> position bits

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int g = blockIdx.x % a.Hk, y = blockIdx.x / a.Hk;
    const int T = a.T;

    const int qt = a.order[y];
    const int R = w * 32 + l32;
    const int head = g * a.G + (R >> a.lgBMq);
    const int pos = qt * a.BMq + (R & (a.BMq - 1));
    const int lb = a.ptr[qt], le = a.ptr[qt + 1];
    const bool row_ok = pos < T;
    const int n = le - lb;
    // the wave's rows cover positions p_base + (0 .. 31) (fewer when a query tile has under
    // 32 positions); this row's bit in a per-key position mask is pos - p_base
    const int p_base = qt * a.BMq + ((w * 32) & (a.BMq - 1));
    const int bit_shift = 31 - (pos - p_base);

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m2 = -INFINITY, lsum[2] = {0.f, 0.f};

    // Q row fragments: B operand, lane holds dims 16*ks + 8*hf .. +7 of its row.
    bf16x8 qf[8];
    {
        const bf16* qp = a.q + ((size_t)min(pos, T - 1) * a.Hq + head) * HEAD_DIM + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * ks));
        // Complete the Q loads here. Left pending into the loop, the wait the compiler puts
        // before the first MFMAs that read Q also covers every K/V prefetch issued behind
        // them, so each tile would stall on the next tile's loads.
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(as_u32x4(qf[ks])));
    }

    const bf16* kbase = a.k + (size_t)g * HEAD_DIM;
    const bf16* vbase = a.v + (size_t)g * HEAD_DIM;
    const size_t kv_row = (size_t)a.Hk * HEAD_DIM;

    EntryStream es;
    es.init(a.ent, lb, n, lane);
    // A stage is SUB consecutive list entries (the last stage may hold fewer; its missing
    // entries repeat the last one and are not computed); e_cur / e_nxt hold the entries of
    // stages u and u + 1.
    const int nst = (n + SUB - 1) / SUB;
    int e_cur[SUB] = {}, e_nxt[SUB] = {};

    // Rows past the end are read from row T - 1 (finite data; such keys are masked).
    u32x4 kreg[CPT], vreg[CPT];
    int4 dreg = {0, 0, 0, 0};
    bool dzero = false;
    // the fixed part of each chunk's offset: chunk c = tid + i * NT is row (c % 1024) / 16 of
    // its sub-tile, dims 8 (c % 16) .. + 7
    unsigned lofs[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int cc = (tid + i * NT) & 1023;
        lofs[i] = (unsigned)((cc >> 4) * kv_row + (cc & 15) * 8);
    }
    auto load_stage = [&](int u) {
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
            e_cur[sb] = e_nxt[sb];
            const int t = SUB * u + sb;
            e_nxt[sb] = t < n ? es.get(t, lane) : e_nxt[sb > 0 ? sb - 1 : 0];
        }
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
            const int key0 = __builtin_amdgcn_readfirstlane((e_nxt[sb] >> 1) * FWD_BN);   // uniform
            if (key0 + FWD_BN <= T) {
                // a whole tile: scalar tile base plus the lane's fixed 32-bit offset
                const bf16* kt0 = kbase + (size_t)key0 * kv_row;
                const bf16* vt0 = vbase + (size_t)key0 * kv_row;
#pragma unroll
                for (int i = sb * (CPT / SUB); i < (sb + 1) * (CPT / SUB); ++i) {
                    kreg[i] = *reinterpret_cast<const u32x4*>(kt0 + lofs[i]);
                    vreg[i] = *reinterpret_cast<const u32x4*>(vt0 + lofs[i]);
                }
            } else {
#pragma unroll
                for (int i = sb * (CPT / SUB); i < (sb + 1) * (CPT / SUB); ++i) {
                    const int cc = (tid + i * NT) & 1023;
                    const int key = min(key0 + (cc >> 4), T - 1);
                    const size_t o = (size_t)key * kv_row + (cc & 15) * 8;
                    kreg[i] = *reinterpret_cast<const u32x4*>(kbase + o);
                    vreg[i] = *reinterpret_cast<const u32x4*>(vbase + o);
                }
            }
        }
        if (tid < SUB * FWD_BN) {
            const int sb = tid / FWD_BN;
            const int key = (e_nxt[sb] >> 1) * FWD_BN + (tid % FWD_BN);
            dreg = a.desc[min(key, T - 1)];
            dzero = key >= T;
        }
    };
    auto store_stage = [&](int slot) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT, row = c >> 4, col = (c & 15) * 8;
            *reinterpret_cast<u32x4*>(&Kb[slot][row * K_LD + col]) = kreg[i];
            *reinterpret_cast<u32x4*>(&Vb[slot][row * V_LD + col]) = vreg[i];
        }
        if (tid < SUB * FWD_BN) Db[slot][tid] = dzero ? int4{0, 0, 0, 0} : dreg;
    };

    if (nst > 0) {
        load_stage(0);
        store_stage(0);
        if (nst > 1) load_stage(1);
    }
    lds_barrier();

    for (int u = 0; u < nst; ++u) {
      const int cb = u & 1;
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        if (SUB * u + sb >= n) break;
        const int e = u + 1 < nst ? e_cur[sb] : e_nxt[sb];
        const int key0 = (e >> 1) * FWD_BN;
        const bool need_mask = (e & 1) == 0 || key0 + FWD_BN > T;

        // S^T = K Q^T for the two 32-key halves of the tile
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const bf16* kr = Kb[cb] + (sb * FWD_BN + l32) * K_LD + 8 * hf;
        mfma_pipelined<16>(
            [&](int i) { return *reinterpret_cast<const u32x4*>(kr + (i & 1) * 32 * K_LD + 16 * (i >> 1)); },
            [&](int i, u32x4 op) { s[i & 1] = mfma32(as_bf16x8(op), qf[i >> 1], s[i & 1]); });

        if (need_mask) {
            // Lane j turns key j's two row intervals into a bit mask over the wave's (at
            // most 32) distinct positions p_base .. p_base + 31; every lane then tests its
            // own position's bit in the masks of the 32 keys it holds.
            const int4 d = Db[cb][sb * FWD_BN + lane];
            Mb[w][lane] = interval_bits(d.x, d.y, p_base) | interval_bits(d.z, d.w, p_base);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's masks written
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const u32x4 m4 = *reinterpret_cast<const u32x4*>(&Mb[w][kb * 32 + 8 * q4 + 4 * hf]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool vis = (int)(m4[i] << bit_shift) < 0;
                        s[kb][4 * q4 + i] = vis ? s[kb][4 * q4 + i] : -INFINITY;
                    }
                }
        }

        // online softmax (base 2), lazy rescale; the IEEE maximum (v_maximum3_f32) needs
        // no input canonicalisation, unlike fmaxf on MFMA results
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2)
                mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[kb][r], s[kb][r + 1]));
        if (__ballot(mx * a.c > m2 + RESCALE_SLACK) != 0ull) {
            mx = fmaxf(mx, swap_halves(mx));
            const float mnew = fmaxf(m2, mx * a.c);
            const float alpha = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mnew);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            lsum[0] *= alpha;
            lsum[1] *= alpha;
            m2 = mnew;
        }
        const float msub = (m2 == -INFINITY) ? 0.f : m2;

        bf16x8 pb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 pk;
#pragma unroll
            for (int e2 = 0; e2 < 8; e2 += 2) {
                const float p0 = fast_exp2(fmaf(s[kk >> 1][(kk & 1) * 8 + e2], a.c, -msub));
                const float p1 = fast_exp2(fmaf(s[kk >> 1][(kk & 1) * 8 + e2 + 1], a.c, -msub));
                lsum[kk & 1] += p0 + p1;
                pk[e2 >> 1] = pack_bf16(p0, p1);
            }
            pb[kk] = as_bf16x8(pk);
        }

        // O^T += V^T P^T: key slot (hf, e) of step kk is key 16*kk + 8*(e/4) + 4*hf + e%4.
        const bf16* vt = Vb[cb] + sb * FWD_BN * V_LD;
        mfma_pipelined<16>(
            [&](int i) {
                const int kk = i >> 2, db = i & 3;
                return tr_rows_ld(vt, V_LD, 16 * kk + 4 * hf, 16 * kk + 8 + 4 * hf, db * 32, lane);
            },
            [&](int i, u32x4 op) { acc[i & 3] = mfma32(as_bf16x8(op), pb[i >> 2], acc[i & 3]); });

      }
        // stage u + 1 into the other slot (its readers of stage u - 1 passed the last
        // barrier), loads of stage u + 2
        if (u + 1 < nst) store_stage(cb ^ 1);
        if (u + 2 < nst) load_stage(u + 2);
        lds_barrier();
    }

    const float lrow = lsum[0] + lsum[1];
    const float ltot = lrow + swap_halves(lrow);
    if (row_ok) {
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        bf16* op = a.o + ((size_t)pos * a.Hq + head) * HEAD_DIM;
        bf16* olp = a.o_lo ? a.o_lo + ((size_t)pos * a.Hq + head) * HEAD_DIM : nullptr;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = db * 32 + 8 * i4 + 4 * hf;
                const float v0 = acc[db][4 * i4 + 0] * inv, v1 = acc[db][4 * i4 + 1] * inv;
                const float v2 = acc[db][4 * i4 + 2] * inv, v3 = acc[db][4 * i4 + 3] * inv;
                u32x2 pk;
                pk[0] = pack_bf16(v0, v1);
                pk[1] = pack_bf16(v2, v3);
                *reinterpret_cast<u32x2*>(op + d0) = pk;
                if (olp) {
                    u32x2 lo;
                    lo[0] = pack_bf16(v0 - bf16_lo(pk[0]), v1 - bf16_hi(pk[0]));
                    lo[1] = pack_bf16(v2 - bf16_lo(pk[1]), v3 - bf16_hi(pk[1]));
                    *reinterpret_cast<u32x2*>(olp + d0) = lo;
                }
            }
        if (hf == 0)
            a.lse[(size_t)head * T + pos] = ltot > 0.f ? (m2 + fast_log2(ltot)) * LN2 : -INFINITY;
    }
}

int launch_fwd(const Problem& P, const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse,
               const int32_t* desc, const void* index, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const IndexLayout L = index_layout(P);
    const char* base = static_cast<const char*>(index);
    FwdArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.o = static_cast<bf16*>(o);
    a.o_lo = static_cast<bf16*>(o_lo);
    a.lse = lse;
    a.desc = reinterpret_cast<const int4*>(desc);
    a.ptr = reinterpret_cast<const int*>(base + L.fwd_ptr);
    a.ent = reinterpret_cast<const int*>(base + L.fwd_ent);
    a.order = P.sparse ? nullptr : reinterpret_cast<const int*>(base + L.fwd_order);
    a.T = P.T;
    a.Hq = P.Hq;
    a.Hk = P.Hk;
    a.G = P.G;
    a.BMq = P.fBM;
    a.lgBMq = P.lgBM;
    a.nb = P.nb;
    a.sblock = P.sblock;
    a.c = P.scale * LOG2E;
    if (!P.sparse) {
        hipLaunchKernelGGL(fwd_dense_kernel, dim3(P.Hk * P.nqt_f), dim3(512), 0, s, a);
    } else if (P.sblock == 64) {
        hipLaunchKernelGGL((fwd_sparse_kernel<4, true>), dim3(P.Hk * P.G * ((P.nb + 1) / 2)), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL((fwd_sparse_kernel<4>), dim3(P.Hk * P.G * P.nb), dim3(256), 0, s, a);
    }
    return (int)hipGetLastError();
}

}  // namespace mlct
