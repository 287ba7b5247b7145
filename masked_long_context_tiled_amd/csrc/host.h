// Host-side problem description, buffer layouts and the kernel launchers' declarations:
// plain C++ with no HIP types, shared by the C-ABI entry points (host.cpp) and the launch
// code next to each kernel. Layout helpers are constexpr, so device code can use them too.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/attn.h"

namespace mlct {

constexpr int HEAD_DIM = 128;
constexpr int FWD_BN = 64;          // keys per forward tile
constexpr int BWD_BN = 128;         // keys per dense backward tile (4 waves x 32 keys)
constexpr int ROWS_PER_WG = 256;    // (head, position) rows per dense forward work item

// Round an offset up to 256 bytes.
constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// One problem after validation.
struct Problem {
    int T, Hq, Hk, G;
    int kind;
    int sblock;         // block-sparse block edge (0 otherwise)
    float scale;
    bool sparse;
    // dense tiles
    int fBM, fBN, bBM, bBN;
    int lgBM;           // log2(fBM) = log2(bBM)
    int nqt_f, nkt_f, nqt_b, nkt_b;
    // block-sparse
    int nb;
};

// Pieces per key tile of the dense dK/dV pass. A short sequence has fewer key tiles (Hk * nkt_b
// work items) than the chip runs at once, and the longest list then sets the time, so each
// key tile's query list is cut into S consecutive pieces (S a power of two up to 8, the
// smallest with Hk * nkt_b * S >= 512) whose partial dK / dV a reduction adds in a fixed
// order. Block-sparse problems have enough work items and take S = 1.
constexpr int dkdv_splits(const Problem& P) {
    int S = 1;
    if (!P.sparse)
        while (S < 8 && (long)P.Hk * P.nkt_b * S < 512) S *= 2;
    return S;
}

// Backward workspace, in order (each part 256-byte aligned):
//   D [Hq][T] fp32 | BWD_STATS fp32 bounds of the operands | Q, dO [T][Hq][128] and
//   K, V [T][Hk][128] as fp16 multiplied by their power-of-two scales | with S > 1 dK/dV
//   pieces, their partial dK [S][T][Hk][128] and dV [S][T][Hk][128] in fp32.
constexpr int BWD_STATS = 4;
struct BwdLayout {
    size_t stats, qh, doh, kh, vh, part, total;
};
constexpr BwdLayout bwd_layout(int Hq, int Hk, int T, int S) {
    BwdLayout L{};
    const size_t qbytes = align256((size_t)T * Hq * 128 * 2), kbytes = align256((size_t)T * Hk * 128 * 2);
    L.stats = align256((size_t)Hq * T * 4);
    L.qh = L.stats + 256;
    L.doh = L.qh + qbytes;
    L.kh = L.doh + qbytes;
    L.vh = L.kh + kbytes;
    L.part = L.vh + kbytes;
    L.total = L.part + (S > 1 ? align256((size_t)2 * S * T * Hk * 128 * 4) : 0);
    return L;
}

struct IndexLayout {
    size_t fwd_cls, fwd_ptr, fwd_ent, fwd_order;
    size_t bwd_cls, bwd_ptr, bwd_ent, bwd_order;
    size_t total;
};

attn_status validate_problem(const attn_problem* p, Problem* out);
IndexLayout index_layout(const Problem& P);

// Block selection workspace: the fp32 block means of Q [Hq][nb][128], then of K [Hk][nb][128].
constexpr int SEL_MAX_NB = 4096;   // longest row of blocks the selection kernel sorts
constexpr size_t select_qbar_bytes(const Problem& P) { return align256((size_t)P.Hq * P.nb * HEAD_DIM * 4); }
constexpr size_t select_workspace_bytes(const Problem& P) {
    return select_qbar_bytes(P) + align256((size_t)P.Hk * P.nb * HEAD_DIM * 4);
}

// Kernel launchers, defined next to their kernels. Each returns the HIP runtime's error
// code after queueing its launches (0 = success); stream is a hipStream_t; desc points to
// the int32 [T][4] column-interval descriptor on the device.
// The column-interval descriptor of mp (whose cu_seqlens, if used, points to device memory).
int launch_desc(const attn_mask_params& mp, int32_t T, int32_t* desc, void* stream);
int launch_index_dense(const Problem& P, const int32_t* desc, void* index, void* stream);
int launch_index_sparse(const Problem& P, const uint8_t* keep, void* index, void* stream);
int launch_fwd(const Problem& P, const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse,
               const int32_t* desc, const void* index, void* stream);
int launch_bwd_pre(const Problem& P, const void* q, const void* k, const void* v, const void* o,
                   const void* o_lo, const void* dout, float* dbuf, void* stream);
enum { BWD_PART_DKDV = 1, BWD_PART_DQ = 2 };
int launch_bwd_main(const Problem& P, const void* q, const void* k, const void* v, const float* lse,
                    const void* dout, float* dq, float* dk, float* dv, const int32_t* desc, const void* index,
                    float* dbuf, int parts, void* stream);
int launch_cast_bf16(const float* in, void* out, size_t n, void* stream);
int launch_block_select(const Problem& P, int mode, int topk, float topp, int keep_diag, const void* q,
                        const void* k, float* scores, uint8_t* keep, void* ws, void* stream);
// The same launches with the workspace in the library's static per-GPU array (at most
// SEL_SCRATCH_BYTES; the caller checks the size first). Looks the array up on the device
// of the stream at its first use there.
constexpr size_t SEL_SCRATCH_BYTES = size_t(ATTN_SELECT_SCRATCH_BYTES);
int launch_block_select_scratch(const Problem& P, int mode, int topk, float topp, int keep_diag, const void* q,
                                const void* k, float* scores, uint8_t* keep, void* stream);
int launch_lse_merge(const Problem& P, void* o, void* o_lo, float* lse, const void* o_part,
                     const void* o_part_lo, const float* lse_part, void* stream);

}  // namespace mlct
