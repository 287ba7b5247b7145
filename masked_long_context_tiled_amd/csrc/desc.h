// Column-interval mask descriptor, one key column at a time: the rule of every mask kind
// of attn.h restated in column form. constexpr, so the host builder (host.cpp) and the
// device builder (desc.hip) run the same code; cu_seqlens points to host or device memory
// accordingly.
#pragma once

#include <stdint.h>

#include "../../include/attn.h"

namespace mlct {

// For key column j the visible query rows are [a0, b0) U [a1, b1), written to iv.
constexpr void column_intervals(const attn_mask_params* mp, int32_t T, int j, long iv[4]) {
    const int k = mp->kind;
    auto set = [&](long a0, long b0, long a1, long b1) {
        iv[0] = a0;
        iv[1] = b0;
        iv[2] = a1;
        iv[3] = b1;
    };
    auto lmin = [](long a, long b) { return a < b ? a : b; };
    auto lmax = [](long a, long b) { return a > b ? a : b; };
    // document of j: cu[d] <= j < cu[d + 1]
    auto doc_of = [&](int x) {
        int lo = 0, hi = mp->n_docs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (mp->cu_seqlens[mid] <= x) lo = mid; else hi = mid - 1;
        }
        return lo;
    };
    switch (k) {
    case ATTN_MASK_FULL: set(0, T, 0, 0); return;
    case ATTN_MASK_CAUSAL: set(j, T, 0, 0); return;
    case ATTN_MASK_FULL_DOCUMENT:
    case ATTN_MASK_CAUSAL_DOCUMENT: {
        const int d = doc_of(j);
        const long s0 = mp->cu_seqlens[d], e0 = mp->cu_seqlens[d + 1];
        set(k == ATTN_MASK_FULL_DOCUMENT ? s0 : j, e0, 0, 0);
        return;
    }
    case ATTN_MASK_FULL_SLIDING_WINDOW: {
        const long w = mp->window;
        set(lmax(0, j - w + 1), lmin(T, j + w), 0, 0);
        return;
    }
    case ATTN_MASK_CAUSAL_SLIDING_WINDOW: set(j, lmin(T, (long)j + mp->window), 0, 0); return;
    case ATTN_MASK_SHARED_QUESTION: {
        const long Qn = mp->question_len, A = mp->answer_len;
        if (j < Qn) set(j, T, 0, 0);                                   // question key: every later row
        else set(j, lmin(T, Qn + ((j - Qn) / A + 1) * A), 0, 0);       // rest of its answer
        return;
    }
    case ATTN_MASK_PREFIX_LM_CAUSAL: set(j < mp->prefix_len ? 0 : j, T, 0, 0); return;
    case ATTN_MASK_CAUSAL_BLOCKWISE: {
        const long b = mp->block_len, F = (long)T - mp->final_block_len;
        if (j >= F) { set(j, T, 0, 0); return; }
        const long bend = lmin(T, ((long)j / b + 1) * b);              // rows of j's own block
        if (bend >= F) set(j, T, 0, 0);                                // touches the final block
        else set(j, bend, F, T);
        return;
    }
    case ATTN_MASK_GLOBAL_SLIDING: {
        const long Gl = mp->global_len, w = mp->window;
        if (j < Gl) { set(0, T, 0, 0); return; }                       // global key: every row
        const long lo = lmax(0, j - w + 1), hi = lmin(T, j + w);
        if (lo <= Gl) set(0, lmax(hi, Gl), 0, 0);                      // window meets the global rows
        else set(0, Gl, lo, hi);
        return;
    }
    case ATTN_MASK_PREFIX_LM_DOCUMENT: {
        const int d = doc_of(j);
        const long s0 = mp->cu_seqlens[d], e0 = mp->cu_seqlens[d + 1];
        set(j - s0 < mp->prefix_len ? s0 : j, e0, 0, 0);               // prefix key: its whole document
        return;
    }
    case ATTN_MASK_BLOCK_CAUSAL_DOCUMENT: {
        const int d = doc_of(j);
        const long s0 = mp->cu_seqlens[d], e0 = mp->cu_seqlens[d + 1], b = mp->block_len;
        set(s0 + (j - s0) / b * b, e0, 0, 0);                          // rows from the start of j's block on
        return;
    }
    default: set(0, 0, 0, 0); return;                                   // not reached: validated first
    }
}

// Descriptor entry of local key column jl of the n x n chunk pair (query rows q_offset..,
// key columns k_offset..) of a sequence of length T, in chunk coordinates: each global
// interval is clipped to the query chunk and shifted; empty intervals become [0, 0) and a
// lone interval comes first.
constexpr void desc_column(const attn_mask_params* mp, int32_t T, int32_t q_offset, int32_t k_offset, int32_t n,
                           int jl, int32_t* out) {
    long iv[4] = {0, 0, 0, 0};
    column_intervals(mp, T, k_offset + jl, iv);
    long a0 = iv[0] - q_offset, b0 = iv[1] - q_offset, a1 = iv[2] - q_offset, b1 = iv[3] - q_offset;
    a0 = a0 < 0 ? 0 : a0;
    a1 = a1 < 0 ? 0 : a1;
    b0 = b0 > n ? n : b0;
    b1 = b1 > n ? n : b1;
    if (a0 >= b0) { a0 = b0 = 0; }
    if (a1 >= b1) { a1 = b1 = 0; }
    if (a0 == b0 && a1 != b1) { a0 = a1; b0 = b1; a1 = b1 = 0; }
    out[0] = (int32_t)a0;
    out[1] = (int32_t)b0;
    out[2] = (int32_t)a1;
    out[3] = (int32_t)b1;
}

}  // namespace mlct
