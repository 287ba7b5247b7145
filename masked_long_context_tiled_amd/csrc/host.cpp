// C-ABI entry points: argument validation, the host column-interval descriptor builder,
// the Variable Block expansion, the tile-index layout and the calls of the kernel
// launchers. Plain C++ (no HIP types): the launchers are declared in host.h and defined
// next to their kernels. No allocation, no global state.
#include <math.h>
#include <string.h>

#include "desc.h"
#include "host.h"

namespace mlct {

static bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

attn_status validate_problem(const attn_problem* p, Problem* out) {
    if (!p) return ATTN_ERR_INVALID_ARG;
    if (p->T < 1 || p->T > (1 << 24) || p->Hq < 1 || p->Hk < 1) return ATTN_ERR_INVALID_ARG;
    if (p->Hq % p->Hk != 0) return ATTN_ERR_INVALID_ARG;
    if (p->mask_kind < ATTN_MASK_FULL || p->mask_kind > ATTN_MASK_BLOCK_CAUSAL_DOCUMENT)
        return ATTN_ERR_INVALID_ARG;
    if (p->head_dim != HEAD_DIM) return ATTN_ERR_UNSUPPORTED;
    if (!(p->scale == p->scale) || isinf(p->scale)) return ATTN_ERR_INVALID_ARG;
    const int G = p->Hq / p->Hk;
    if (!is_pow2(G) || G > ROWS_PER_WG) return ATTN_ERR_UNSUPPORTED;
    Problem P{};
    P.T = p->T;
    P.Hq = p->Hq;
    P.Hk = p->Hk;
    P.G = G;
    P.kind = p->mask_kind;
    P.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)HEAD_DIM);
    P.sparse = p->mask_kind == ATTN_MASK_BLOCK_SPARSE;
    if (P.sparse) {
        if (p->sparse_block != 64 && p->sparse_block != 128) return ATTN_ERR_UNSUPPORTED;
        P.sblock = p->sparse_block;
        P.nb = (P.T + P.sblock - 1) / P.sblock;
        // the keep matrix and the block lists are indexed with 32-bit integers
        if ((size_t)P.Hq * P.nb * P.nb > (size_t)INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    } else {
        P.fBM = ROWS_PER_WG / G;
        P.lgBM = 0;
        while ((1 << P.lgBM) < P.fBM) ++P.lgBM;
        P.fBN = FWD_BN;
        P.bBM = ROWS_PER_WG / G;
        P.bBN = BWD_BN;
        P.nqt_f = (P.T + P.fBM - 1) / P.fBM;
        P.nkt_f = (P.T + P.fBN - 1) / P.fBN;
        P.nqt_b = (P.T + P.bBM - 1) / P.bBM;
        P.nkt_b = (P.T + P.bBN - 1) / P.bBN;
        if ((size_t)P.nqt_f * P.nkt_f > (size_t)INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
    }
    if (out) *out = P;
    return ATTN_OK;
}

IndexLayout index_layout(const Problem& P) {
    IndexLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    if (!P.sparse) {
        const size_t nf = (size_t)P.nqt_f * P.nkt_f, nb = (size_t)P.nqt_b * P.nkt_b;
        L.fwd_cls = take(nf);
        L.fwd_ptr = take(((size_t)P.nqt_f + 1) * 4);
        L.fwd_ent = take(nf * 4);
        L.fwd_order = take((size_t)P.nqt_f * 4);
        L.bwd_cls = take(nb);
        L.bwd_ptr = take(((size_t)P.nkt_b + 1) * 4);
        L.bwd_ent = take(nb * 4);
        L.bwd_order = take((size_t)P.nkt_b * 4);
    } else {
        const size_t rows = (size_t)P.Hq * P.nb, cols = (size_t)P.Hk * P.nb;
        const size_t all = rows * P.nb;
        L.fwd_ptr = take((rows + 1) * 4);
        L.fwd_ent = take(all * 4);
        L.bwd_ptr = take((cols + 1) * 4);
        L.bwd_ent = take(all * 4);
    }
    L.total = align256(off);
    return L;
}

// Descriptor of the n x n chunk pair at (q_offset, k_offset), every column (host).
static void build_desc(const attn_mask_params* mp, int32_t T, int32_t q_offset, int32_t k_offset, int32_t n,
                       int32_t* out) {
    for (int jl = 0; jl < n; ++jl) desc_column(mp, T, q_offset, k_offset, n, jl, out + 4 * jl);
}

static attn_status validate_mask(const attn_mask_params* mp, int32_t T) {
    if (!mp || T < 1 || T > (1 << 24)) return ATTN_ERR_INVALID_ARG;
    switch (mp->kind) {
    case ATTN_MASK_FULL:
    case ATTN_MASK_CAUSAL:
        return ATTN_OK;
    case ATTN_MASK_FULL_DOCUMENT:
    case ATTN_MASK_CAUSAL_DOCUMENT:
    case ATTN_MASK_PREFIX_LM_DOCUMENT:
    case ATTN_MASK_BLOCK_CAUSAL_DOCUMENT: {
        if (mp->n_docs < 1 || !mp->cu_seqlens) return ATTN_ERR_INVALID_ARG;
        if (mp->kind == ATTN_MASK_PREFIX_LM_DOCUMENT && mp->prefix_len < 0) return ATTN_ERR_INVALID_ARG;
        if (mp->kind == ATTN_MASK_BLOCK_CAUSAL_DOCUMENT && mp->block_len < 1) return ATTN_ERR_INVALID_ARG;
        const int32_t* cu = mp->cu_seqlens;
        if (cu[0] != 0 || cu[mp->n_docs] != T) return ATTN_ERR_INVALID_ARG;
        for (int d = 0; d < mp->n_docs; ++d)
            if (cu[d + 1] <= cu[d]) return ATTN_ERR_INVALID_ARG;
        return ATTN_OK;
    }
    case ATTN_MASK_FULL_SLIDING_WINDOW:
    case ATTN_MASK_CAUSAL_SLIDING_WINDOW:
        return mp->window >= 1 ? ATTN_OK : ATTN_ERR_INVALID_ARG;
    case ATTN_MASK_SHARED_QUESTION:
        if (mp->question_len < 0 || mp->answer_len < 1 || mp->n_answers < 1) return ATTN_ERR_INVALID_ARG;
        if ((long)mp->question_len + (long)mp->n_answers * mp->answer_len != T) return ATTN_ERR_INVALID_ARG;
        return ATTN_OK;
    case ATTN_MASK_PREFIX_LM_CAUSAL:
        return (mp->prefix_len >= 0 && mp->prefix_len <= T) ? ATTN_OK : ATTN_ERR_INVALID_ARG;
    case ATTN_MASK_CAUSAL_BLOCKWISE:
        return (mp->block_len >= 1 && mp->final_block_len >= 0 && mp->final_block_len <= T)
                   ? ATTN_OK : ATTN_ERR_INVALID_ARG;
    case ATTN_MASK_GLOBAL_SLIDING:
        return (mp->global_len >= 0 && mp->global_len <= T && mp->window >= 1) ? ATTN_OK
                                                                                : ATTN_ERR_INVALID_ARG;
    default:
        return ATTN_ERR_INVALID_ARG;   // BLOCK_SPARSE has no descriptor; unknown kinds
    }
}

static attn_status hip_status(int e) { return e == 0 ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace mlct

using namespace mlct;

extern "C" {

const char* attn_status_string(attn_status s) {
    switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_ERR_UNKNOWN";
    }
}

attn_status attn_mask_desc_build(const attn_mask_params* p, int32_t T, int32_t* desc_out) {
    if (!desc_out) return ATTN_ERR_INVALID_ARG;
    attn_status st = validate_mask(p, T);
    if (st != ATTN_OK) return st;
    build_desc(p, T, 0, 0, T, desc_out);
    return ATTN_OK;
}

attn_status attn_mask_desc_build_device(const attn_mask_params* p, int32_t T, const int32_t* cu_seqlens_dev,
                                        int32_t* desc_dev, void* stream) {
    if (!desc_dev) return ATTN_ERR_INVALID_ARG;
    attn_status st = validate_mask(p, T);
    if (st != ATTN_OK) return st;
    attn_mask_params d = *p;
    const bool docs = p->kind == ATTN_MASK_FULL_DOCUMENT || p->kind == ATTN_MASK_CAUSAL_DOCUMENT ||
                      p->kind == ATTN_MASK_PREFIX_LM_DOCUMENT || p->kind == ATTN_MASK_BLOCK_CAUSAL_DOCUMENT;
    if (docs && !cu_seqlens_dev) return ATTN_ERR_INVALID_ARG;
    d.cu_seqlens = docs ? cu_seqlens_dev : nullptr;
    return hip_status(launch_desc(d, T, desc_dev, stream));
}

attn_status attn_mask_desc_build_chunk(const attn_mask_params* p, int32_t T, int32_t q_offset, int32_t k_offset,
                                       int32_t n, int32_t* desc_out) {
    if (!desc_out) return ATTN_ERR_INVALID_ARG;
    attn_status st = validate_mask(p, T);
    if (st != ATTN_OK) return st;
    if (n < 1 || q_offset < 0 || k_offset < 0 || (long)q_offset + n > T || (long)k_offset + n > T)
        return ATTN_ERR_INVALID_ARG;
    build_desc(p, T, q_offset, k_offset, n, desc_out);
    return ATTN_OK;
}

attn_status attn_lse_merge(const attn_problem* prob, void* o, void* o_lo, float* lse, const void* o_part,
                           const void* o_part_lo, const float* lse_part, void* stream) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!o || !lse || !o_part || !lse_part) return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_lse_merge(P, o, o_lo, lse, o_part, o_part_lo, lse_part, stream));
}

attn_status attn_block_select_workspace_size(const attn_problem* prob, size_t* bytes_out) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!bytes_out || !P.sparse) return ATTN_ERR_INVALID_ARG;
    *bytes_out = select_workspace_bytes(P);
    return ATTN_OK;
}

static attn_status validate_select(const attn_problem* prob, const attn_block_select_params* sp, const void* q,
                                   const void* k, const float* scores, const uint8_t* keep_out, Problem* P) {
    attn_status st = validate_problem(prob, P);
    if (st != ATTN_OK) return st;
    if (!P->sparse || !sp || !q || !k || !scores || !keep_out) return ATTN_ERR_INVALID_ARG;
    if (sp->mode == ATTN_SELECT_TOPK) {
        if (sp->topk < 1) return ATTN_ERR_INVALID_ARG;
    } else if (sp->mode == ATTN_SELECT_TOPP) {
        if (!(sp->topp > 0.f && sp->topp <= 1.f)) return ATTN_ERR_INVALID_ARG;
    } else {
        return ATTN_ERR_INVALID_ARG;
    }
    if (P->nb > SEL_MAX_NB) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

attn_status attn_block_select(const attn_problem* prob, const attn_block_select_params* sp, const void* q,
                              const void* k, float* scores, uint8_t* keep_out, void* ws, size_t ws_bytes,
                              void* stream) {
    Problem P;
    attn_status st = validate_select(prob, sp, q, k, scores, keep_out, &P);
    if (st != ATTN_OK) return st;
    if (!ws) return ATTN_ERR_INVALID_ARG;
    if (ws_bytes < select_workspace_bytes(P)) return ATTN_ERR_WORKSPACE;
    return hip_status(launch_block_select(P, sp->mode, sp->topk < P.nb ? sp->topk : P.nb, sp->topp,
                                          sp->keep_diagonal ? 1 : 0, q, k, scores, keep_out, ws,
                                          stream));
}

attn_status attn_block_select_noalloc(const attn_problem* prob, const attn_block_select_params* sp, const void* q,
                                      const void* k, float* scores, uint8_t* keep_out, void* stream) {
    Problem P;
    attn_status st = validate_select(prob, sp, q, k, scores, keep_out, &P);
    if (st != ATTN_OK) return st;
    if (select_workspace_bytes(P) > SEL_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    return hip_status(launch_block_select_scratch(P, sp->mode, sp->topk < P.nb ? sp->topk : P.nb, sp->topp,
                                                  sp->keep_diagonal ? 1 : 0, q, k, scores, keep_out, stream));
}

// Block edges 0 = off[0] < off[1] < ... < off[n] = T, the interior ones multiples of 64.
static bool valid_edges(const int32_t* off, int32_t n, int32_t T) {
    if (!off || n < 1 || off[0] != 0 || off[n] != T) return false;
    for (int32_t r = 0; r < n; ++r) {
        if (off[r + 1] <= off[r]) return false;
        if (r + 1 < n && off[r + 1] % 64 != 0) return false;
    }
    return true;
}

attn_status attn_variable_block_expand(int32_t T, int32_t Hq, const int32_t* row_off, int32_t n_rb,
                                       const int32_t* col_off, int32_t n_cb, const uint8_t* keep_var,
                                       uint8_t* keep_out) {
    if (T < 1 || T > (1 << 24) || Hq < 1 || !keep_var || !keep_out) return ATTN_ERR_INVALID_ARG;
    if (!valid_edges(row_off, n_rb, T) || !valid_edges(col_off, n_cb, T)) return ATTN_ERR_INVALID_ARG;
    const int64_t nt = (T + 63) / 64;
    if ((int64_t)Hq * nt * nt > (int64_t)INT32_MAX) return ATTN_ERR_UNSUPPORTED;
    for (int32_t h = 0; h < Hq; ++h) {
        int32_t r = 0;
        for (int64_t qt = 0; qt < nt; ++qt) {
            while (row_off[r + 1] <= qt * 64) ++r;   // the row block holding tile qt
            const uint8_t* kv = keep_var + ((size_t)h * n_rb + r) * n_cb;
            uint8_t* out = keep_out + ((size_t)h * nt + qt) * nt;
            int32_t c = 0;
            for (int64_t kt = 0; kt < nt; ++kt) {
                while (col_off[c + 1] <= kt * 64) ++c;
                out[kt] = kv[c] ? 1 : 0;
            }
        }
    }
    return ATTN_OK;
}

attn_status attn_tile_index_size(const attn_problem* prob, size_t* bytes_out) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!bytes_out) return ATTN_ERR_INVALID_ARG;
    *bytes_out = index_layout(P).total;
    return ATTN_OK;
}

attn_status attn_query_tile_shape(const attn_problem* prob, int32_t* fwd_bm, int32_t* fwd_bn,
                                  int32_t* bwd_bm, int32_t* bwd_bn) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (P.sparse) return ATTN_ERR_INVALID_ARG;
    if (!fwd_bm || !fwd_bn || !bwd_bm || !bwd_bn) return ATTN_ERR_INVALID_ARG;
    *fwd_bm = P.fBM;
    *fwd_bn = P.fBN;
    *bwd_bm = P.bBM;
    *bwd_bn = P.bBN;
    return ATTN_OK;
}

attn_status attn_tile_index_layout(const attn_problem* prob, attn_index_layout* out) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!out) return ATTN_ERR_INVALID_ARG;
    IndexLayout L = index_layout(P);
    if (P.sparse) {
        out->nqt_f = P.Hq * P.nb;
        out->nkt_f = P.nb;
        out->nqt_b = P.Hk * P.nb;
        out->nkt_b = P.nb;
    } else {
        out->nqt_f = P.nqt_f;
        out->nkt_f = P.nkt_f;
        out->nqt_b = P.nqt_b;
        out->nkt_b = P.nkt_b;
    }
    out->fwd_cls = L.fwd_cls;
    out->fwd_ptr = L.fwd_ptr;
    out->fwd_ent = L.fwd_ent;
    out->fwd_order = L.fwd_order;
    out->bwd_cls = L.bwd_cls;
    out->bwd_ptr = L.bwd_ptr;
    out->bwd_ent = L.bwd_ent;
    out->bwd_order = L.bwd_order;
    out->total_bytes = L.total;
    return ATTN_OK;
}

attn_status attn_tile_index_build(const attn_problem* prob, const int32_t* desc_dev, void* index_dev,
                                  size_t index_bytes, void* stream) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (P.sparse || !desc_dev || !index_dev) return ATTN_ERR_INVALID_ARG;
    if (index_bytes < index_layout(P).total) return ATTN_ERR_WORKSPACE;
    return hip_status(launch_index_dense(P, desc_dev, index_dev,
                                         stream));
}

attn_status attn_block_index_build(const attn_problem* prob, const uint8_t* keep_dev, void* index_dev,
                                   size_t index_bytes, void* stream) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!P.sparse || !keep_dev || !index_dev) return ATTN_ERR_INVALID_ARG;
    if (index_bytes < index_layout(P).total) return ATTN_ERR_WORKSPACE;
    return hip_status(launch_index_sparse(P, keep_dev, index_dev, stream));
}

attn_status attn_fwd_workspace_size(const attn_problem* prob, size_t* bytes_out) {
    attn_status st = validate_problem(prob, nullptr);
    if (st != ATTN_OK) return st;
    if (!bytes_out) return ATTN_ERR_INVALID_ARG;
    *bytes_out = 0;
    return ATTN_OK;
}

attn_status attn_bwd_workspace_size(const attn_problem* prob, size_t* bytes_out) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!bytes_out) return ATTN_ERR_INVALID_ARG;
    // D, operand bounds, scaled fp16 Q, dO, K, V (and partial dK / dV for short sequences)
    *bytes_out = bwd_layout(P.Hq, P.Hk, P.T, dkdv_splits(P)).total;
    return ATTN_OK;
}

attn_status attn_fwd(const attn_problem* prob, const void* q, const void* k, const void* v, void* o,
                     void* o_lo, float* lse, const int32_t* desc_dev, const void* index_dev, size_t index_bytes,
                     void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!q || !k || !v || !o || !lse || !index_dev) return ATTN_ERR_INVALID_ARG;
    if (!P.sparse && !desc_dev) return ATTN_ERR_INVALID_ARG;
    if (index_bytes < index_layout(P).total) return ATTN_ERR_WORKSPACE;
    return hip_status(launch_fwd(P, q, k, v, o, o_lo, lse, desc_dev, index_dev,
                                 stream));
}

static attn_status check_bwd_ws(const attn_problem* prob, const void* ws, size_t ws_bytes) {
    size_t need = 0;
    attn_bwd_workspace_size(prob, &need);
    return (!ws || ws_bytes < need) ? ATTN_ERR_WORKSPACE : ATTN_OK;
}

attn_status attn_bwd_preprocess(const attn_problem* prob, const void* q, const void* k, const void* v,
                                const void* o, const void* o_lo, const void* dout, void* ws, size_t ws_bytes,
                                void* stream) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!q || !k || !v || !o || !dout) return ATTN_ERR_INVALID_ARG;
    if ((st = check_bwd_ws(prob, ws, ws_bytes)) != ATTN_OK) return st;
    return hip_status(launch_bwd_pre(P, q, k, v, o, o_lo, dout, (float*)ws, stream));
}

static attn_status bwd_parts(const attn_problem* prob, const void* q, const void* k, const void* v,
                             const float* lse, const void* dout, float* dq, float* dk, float* dv,
                             const int32_t* desc_dev, const void* index_dev, size_t index_bytes, void* ws,
                             size_t ws_bytes, void* stream, int parts) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    if (!q || !k || !v || !lse || !dout || !index_dev) return ATTN_ERR_INVALID_ARG;
    if (((parts & BWD_PART_DQ) && !dq) || ((parts & BWD_PART_DKDV) && (!dk || !dv))) return ATTN_ERR_INVALID_ARG;
    if (!P.sparse && !desc_dev) return ATTN_ERR_INVALID_ARG;
    if (index_bytes < index_layout(P).total) return ATTN_ERR_WORKSPACE;
    if ((st = check_bwd_ws(prob, ws, ws_bytes)) != ATTN_OK) return st;
    return hip_status(launch_bwd_main(P, q, k, v, lse, dout, dq, dk, dv, desc_dev,
                                      index_dev, (float*)ws, parts, stream));
}

attn_status attn_bwd_main(const attn_problem* prob, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, float* dq, float* dk, float* dv,
                          const int32_t* desc_dev, const void* index_dev, size_t index_bytes, void* ws,
                          size_t ws_bytes, void* stream) {
    return bwd_parts(prob, q, k, v, lse, dout, dq, dk, dv, desc_dev, index_dev, index_bytes, ws, ws_bytes, stream,
                     BWD_PART_DKDV | BWD_PART_DQ);
}

attn_status attn_bwd_dkdv(const attn_problem* prob, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, float* dk, float* dv, const int32_t* desc_dev,
                          const void* index_dev, size_t index_bytes, void* ws, size_t ws_bytes,
                          void* stream) {
    return bwd_parts(prob, q, k, v, lse, dout, nullptr, dk, dv, desc_dev, index_dev, index_bytes, ws, ws_bytes,
                     stream, BWD_PART_DKDV);
}

attn_status attn_bwd_dq(const attn_problem* prob, const void* q, const void* k, const void* v,
                        const float* lse, const void* dout, float* dq, const int32_t* desc_dev,
                        const void* index_dev, size_t index_bytes, const void* ws, size_t ws_bytes, void* stream) {
    // the dQ pass only reads the workspace
    return bwd_parts(prob, q, k, v, lse, dout, dq, nullptr, nullptr, desc_dev, index_dev, index_bytes,
                     const_cast<void*>(ws), ws_bytes, stream, BWD_PART_DQ);
}

attn_status attn_bwd(const attn_problem* prob, const void* q, const void* k, const void* v, const void* o,
                     const void* o_lo, const float* lse, const void* dout, float* dq, float* dk, float* dv,
                     const int32_t* desc_dev, const void* index_dev, size_t index_bytes, void* ws,
                     size_t ws_bytes, void* stream) {
    Problem P;
    attn_status st = validate_problem(prob, &P);
    if (st != ATTN_OK) return st;
    // validate everything before the first launch
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !index_dev)
        return ATTN_ERR_INVALID_ARG;
    if (!P.sparse && !desc_dev) return ATTN_ERR_INVALID_ARG;
    if (index_bytes < index_layout(P).total) return ATTN_ERR_WORKSPACE;
    if ((st = check_bwd_ws(prob, ws, ws_bytes)) != ATTN_OK) return st;
    st = attn_bwd_preprocess(prob, q, k, v, o, o_lo, dout, ws, ws_bytes, stream);
    if (st != ATTN_OK) return st;
    return attn_bwd_main(prob, q, k, v, lse, dout, dq, dk, dv, desc_dev, index_dev, index_bytes, ws, ws_bytes,
                         stream);
}

attn_status attn_cast_bf16(const float* in, void* out, size_t n, void* stream) {
    if (n == 0) return ATTN_OK;
    if (!in || !out) return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_cast_bf16(in, out, n, stream));
}

}  // extern "C"
