/*
 * attn.h - C ABI of the masked long-context attention library (libattn.so, gfx950).
 *
 * The operator is bf16 masked softmax attention, forward and backward,
 *     O = softmax(scale * Q K^T + mask) V,
 * over grouped query heads (GQA: Hq query heads share Hk key/value heads in contiguous
 * groups of G = Hq / Hk; MHA is G = 1) at head dimension 128, for the mask families
 * benchmarked on "LongCA-bench: 长上下文注意力基准测试" (xllm-io paper-review blog):
 *   - section 三 "注意力掩码模式": the regular masks (FULL, CAUSAL, FULL/CAUSAL DOCUMENT
 *     over packed sequences, FULL/CAUSAL SLIDING WINDOW), the heterogeneous masks
 *     (SHARED QUESTION, PREFIX LM CAUSAL, CAUSAL BLOCKWISE, GLOBAL SLIDING, PREFIX LM
 *     DOCUMENT, BLOCK CAUSAL DOCUMENT) and the
 *     dynamic Uniform Block mask (block-sparse, fixed 64x64 or 128x128 blocks)
 *     and Variable Block (variable block sizes), with a TopK / TopP block selector;
 *   - section 三 "稀疏注意力内核": block size 64 and 128, GQA and MHA, forward and
 *     backward (the capability matrix of the sparse kernels);
 *   - section 四 "实验设置": bf16, head dim 128, GQA 64:8 and MHA 64:64, long sequences.
 * The pages give names only; the exact visibility rule of every mask is stated at
 * attn_mask_kind below.
 *
 * Layouts (all row-major, contiguous, batch 1, one packed sequence of length T):
 *   Q, dO, O : bf16  [T][Hq][128]        K, V : bf16 [T][Hk][128]
 *   LSE      : fp32  [Hq][T]  natural-log log-sum-exp of each query row's scaled scores
 *   dQ       : fp32  [T][Hq][128]        dK, dV : fp32 [T][Hk][128]
 *   desc     : int32 [T][4]  column-interval mask descriptor (attn_mask_desc_build)
 *   keep     : uint8 [Hq][nb][nb], nb = ceil(T / b): block-sparse keep matrix
 * Query head h uses key/value head h / G.
 *
 * Ownership and threading: the caller allocates and frees every buffer (inputs,
 * outputs, the tile index and the workspace); the library allocates nothing and keeps
 * no global state, so calls are reentrant. Device entry points are asynchronous on
 * the given stream (a hipStream_t passed as void*, NULL = the null stream) and return
 * after the launches are queued. All argument validation happens before any launch:
 * an error status means nothing was launched. A launch failure reported by the HIP
 * runtime is returned as ATTN_ERR_HIP. No C++ exception crosses this interface.
 *
 * Fully masked rows (possible only with a hand-built descriptor or keep matrix) get
 * O = 0, LSE = -inf and zero gradients.
 */
#ifndef MLCT_ATTN_H
#define MLCT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,  /* null pointer, bad size, Hq % Hk != 0, bad cu_seqlens, ... */
    ATTN_ERR_UNSUPPORTED = 2,  /* head_dim != 128, group size G not a power of two <= 256, ... */
    ATTN_ERR_WORKSPACE = 3,    /* workspace or index buffer smaller than the queried size */
    ATTN_ERR_HIP = 4           /* the HIP runtime reported a launch error */
} attn_status;

/*
 * Mask kinds. i = query position, j = key position, 0-based in the packed sequence.
 * visible(i, j) is the rule each kind implements (the readings of the page's names):
 *   FULL                     true
 *   CAUSAL                   j <= i
 *   FULL_DOCUMENT            doc(i) == doc(j)           doc from cu_seqlens
 *   CAUSAL_DOCUMENT          doc(i) == doc(j) && j <= i
 *   FULL_SLIDING_WINDOW      |i - j| < window
 *   CAUSAL_SLIDING_WINDOW    0 <= i - j < window
 *   SHARED_QUESTION          j <= i && (j < question_len || ans(i) == ans(j)),
 *                            ans(x) = (x - question_len) / answer_len for x >= question_len
 *   PREFIX_LM_CAUSAL         j < prefix_len || j <= i
 *   CAUSAL_BLOCKWISE         j <= i && (i >= T - final_block_len || i / block_len == j / block_len)
 *   GLOBAL_SLIDING           i < global_len || j < global_len || |i - j| < window
 *   BLOCK_SPARSE             keep[h][i / b][j / b] != 0 (per query head h, b = sparse_block)
 *   PREFIX_LM_DOCUMENT       doc(i) == doc(j) && (j - start(doc(j)) < prefix_len || j <= i):
 *                            every document has its own bidirectional prefix of
 *                            min(prefix_len, its length) positions, the rest causal
 *   BLOCK_CAUSAL_DOCUMENT    doc(i) == doc(j) && blk(i) >= blk(j),
 *                            blk(x) = (x - start(doc(x))) / block_len: blocks of block_len
 *                            positions (restarting at every document, the last one of a
 *                            document possibly shorter) see themselves fully and the
 *                            earlier blocks of their document
 * Every kind except BLOCK_SPARSE is head-independent and has at most two visible row
 * intervals per key column, which is what the descriptor stores.
 */
typedef enum attn_mask_kind {
    ATTN_MASK_FULL = 0,
    ATTN_MASK_CAUSAL = 1,
    ATTN_MASK_FULL_DOCUMENT = 2,
    ATTN_MASK_CAUSAL_DOCUMENT = 3,
    ATTN_MASK_FULL_SLIDING_WINDOW = 4,
    ATTN_MASK_CAUSAL_SLIDING_WINDOW = 5,
    ATTN_MASK_SHARED_QUESTION = 6,
    ATTN_MASK_PREFIX_LM_CAUSAL = 7,
    ATTN_MASK_CAUSAL_BLOCKWISE = 8,
    ATTN_MASK_GLOBAL_SLIDING = 9,
    ATTN_MASK_BLOCK_SPARSE = 10,
    ATTN_MASK_PREFIX_LM_DOCUMENT = 11,
    ATTN_MASK_BLOCK_CAUSAL_DOCUMENT = 12
} attn_mask_kind;

/* Mask parameters; fields a kind does not use are ignored. */
typedef struct attn_mask_params {
    int32_t kind;             /* attn_mask_kind */
    int32_t window;           /* sliding window width w >= 1 */
    int32_t prefix_len;       /* PREFIX_LM_CAUSAL: 0 <= prefix_len <= T; PREFIX_LM_DOCUMENT: >= 0 */
    int32_t question_len;     /* SHARED_QUESTION: T == question_len + n_answers * answer_len */
    int32_t answer_len;
    int32_t n_answers;
    int32_t block_len;        /* CAUSAL_BLOCKWISE: block_len >= 1, 0 <= final_block_len <= T;
                                 BLOCK_CAUSAL_DOCUMENT: block_len >= 1 */
    int32_t final_block_len;
    int32_t global_len;       /* GLOBAL_SLIDING: 0 <= global_len <= T, window >= 1 */
    int32_t n_docs;           /* the four DOCUMENT kinds: number of documents >= 1 */
    const int32_t* cu_seqlens;/* host pointer, n_docs + 1 strictly increasing entries, 0 .. T */
} attn_mask_params;

/* One attention problem. */
typedef struct attn_problem {
    int32_t T;                /* packed sequence length, 1 <= T <= 2^24 */
    int32_t Hq;               /* query heads */
    int32_t Hk;               /* key/value heads; G = Hq / Hk must be a power of two <= 256 */
    int32_t head_dim;         /* must be 128 */
    float scale;              /* softmax scale; <= 0 selects 1 / sqrt(head_dim) */
    int32_t mask_kind;        /* attn_mask_kind */
    int32_t sparse_block;     /* BLOCK_SPARSE only: 64 or 128 */
} attn_problem;

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(attn_status s);

/*
 * Column-interval mask descriptor (host, synchronous). For every key column j it
 * writes desc[j] = {a0, b0, a1, b1}: the query rows that see key j are exactly
 * [a0, b0) U [a1, b1), with 0 <= a0 <= b0 <= a1 <= b1 <= T (an empty interval has
 * a == b). This is the column-wise mask representation that the pages credit to
 * FlashMask (section 三 "密集注意力内核", section 四 "密集内核性能"), restricted to
 * two intervals, which every non-sparse kind above needs at most.
 *   p        : mask parameters (kind must not be BLOCK_SPARSE)
 *   T        : sequence length
 *   desc_out : host int32 [T][4], written entirely on success, untouched on error
 */
attn_status attn_mask_desc_build(const attn_mask_params* p, int32_t T, int32_t* desc_out);

/*
 * The same descriptor built on the device (asynchronous on stream): one thread per key
 * column runs the host builder's per-column rule, so a step that rebuilds its mask needs no
 * host work and no host-to-device copy, and can be captured in a HIP graph.
 *   p              : mask parameters, validated on the host as by attn_mask_desc_build
 *                    (p->cu_seqlens, if the kind uses documents, is read on the host for
 *                    the validation only)
 *   cu_seqlens_dev : device int32 [n_docs + 1], the same values as p->cu_seqlens; required
 *                    by the four DOCUMENT kinds, ignored by the others (may be NULL)
 *   desc_dev       : device int32 [T][4], written entirely by the launch
 * Errors: as attn_mask_desc_build, plus ATTN_ERR_INVALID_ARG for a null desc_dev or a
 * DOCUMENT kind without cu_seqlens_dev (nothing is launched then).
 */
attn_status attn_mask_desc_build_device(const attn_mask_params* p, int32_t T, const int32_t* cu_seqlens_dev,
                                        int32_t* desc_dev, void* stream);

/*
 * Context-parallel building block (the pages' ring / USP / LoongTrain methods exchange
 * K/V chunks of one long sequence between devices and combine per-chunk results; see
 * "LongCA-bench: 长上下文注意力基准测试", section 三 "分布式注意力机制" and section 四
 * "分布式注意力性能"). A chunk pair is the n x n block of the global mask with query rows
 * q_offset .. q_offset + n - 1 and key columns k_offset .. k_offset + n - 1 of a sequence
 * of length T. Its descriptor, in chunk coordinates, turns the pair into an ordinary
 * problem of length n: attn_tile_index_build / attn_fwd / attn_bwd run on it unchanged.
 *   p        : mask parameters of the whole sequence (kind must not be BLOCK_SPARSE)
 *   T        : global sequence length
 *   q_offset, k_offset : global positions of the chunks' first query / key, >= 0,
 *              q_offset + n <= T, k_offset + n <= T
 *   n        : chunk length >= 1
 *   desc_out : host int32 [n][4]: for local key j, the local query rows i with
 *              visible(q_offset + i, k_offset + j), as at most two half-open intervals;
 *              written entirely on success, untouched on error
 * The forward of a chunk pair gives the attention of the query chunk over that key chunk
 * only (O normalised over it, LSE over it; a row with no visible key in the chunk gets
 * O = 0, LSE = -inf); attn_lse_merge combines such partial results over key chunks. The
 * backward of a chunk pair, given the merged O (and O_lo) and LSE of the whole rows,
 * gives that pair's share of dQ (summed over key chunks) and of dK, dV (summed over query
 * chunks).
 */
attn_status attn_mask_desc_build_chunk(const attn_mask_params* p, int32_t T, int32_t q_offset, int32_t k_offset,
                                       int32_t n, int32_t* desc_out);

/*
 * Merge a partial attention result over another key set into an accumulated one, in
 * place: with m = max(LSE, LSE_part), w = exp(LSE - m), w_part = exp(LSE_part - m),
 *   O <- (w O + w_part O_part) / (w + w_part),   LSE <- m + ln(w + w_part)
 * (a row with both LSEs -inf keeps O = 0, LSE = -inf). This is exactly the attention over
 * the union of the key sets. Start the accumulator from the first chunk's result.
 *   prob          : T = chunk length, Hq; the other fields are validated but unused
 *   o, o_lo       : device bf16 [T][Hq][128] accumulated O and its optional bf16 residual
 *                   (O + O_lo is the fp32 value; o_lo may be NULL: then treated as 0 and
 *                   not written)
 *   lse           : device fp32 [Hq][T] accumulated LSE (natural log)
 *   o_part, o_part_lo, lse_part : the partial result, same layouts (o_part_lo may be NULL)
 * Errors: ATTN_ERR_INVALID_ARG for a null required pointer or a bad problem.
 */
attn_status attn_lse_merge(const attn_problem* prob, void* o, void* o_lo, float* lse, const void* o_part,
                           const void* o_part_lo, const float* lse_part, void* stream);

/*
 * Tile index: per-tile classes (EMPTY / PARTIAL / FULL) and the lists of non-empty
 * tiles the kernels walk, for the tile shapes the kernels use for this problem. EMPTY
 * tiles are skipped, FULL tiles run without per-element mask work, PARTIAL tiles
 * evaluate the interval descriptor per element. For BLOCK_SPARSE the same buffer holds
 * the block index built from the keep matrix instead.
 * attn_tile_index_size gives the bytes the caller must allocate (device memory,
 * 256-byte aligned); the size depends only on the problem.
 */
attn_status attn_tile_index_size(const attn_problem* prob, size_t* bytes_out);

/* Tile shapes (query positions x key positions) of the forward and backward kernels,
 * as used in the tile index. Valid for every mask kind except BLOCK_SPARSE. */
attn_status attn_query_tile_shape(const attn_problem* prob, int32_t* fwd_bm, int32_t* fwd_bn,
                                  int32_t* bwd_bm, int32_t* bwd_bn);

/* Byte offsets of the sections of a tile index (for inspection and tests):
 *   fwd_cls   uint8 [nqt_f][nkt_f]        class per forward tile (0 EMPTY, 1 PARTIAL, 2 FULL)
 *   fwd_ptr   int32 [nqt_f + 1]           CSR row pointers
 *   fwd_ent   int32 [nnz]                 (key tile << 1) | is_full, ascending per row
 *   fwd_order int32 [nqt_f]               query tiles by descending list length (launch order)
 *   bwd_cls   uint8 [nqt_b][nkt_b], bwd_ptr int32 [nkt_b + 1],
 *   bwd_ent   int32 [nnz]                 (query tile << 1) | is_full, ascending per column
 *   bwd_order int32 [nkt_b]               key tiles by descending list length
 * For BLOCK_SPARSE: fwd_ptr/fwd_ent are the CSR of keep over rows (h * nb + qb), entries
 * kb; bwd_ptr/bwd_ent the CSC over columns (g * nb + kb), entries (h - g*G) * nb + qb;
 * the cls and order sections are unused (offset 0). */
typedef struct attn_index_layout {
    int32_t nqt_f, nkt_f, nqt_b, nkt_b;
    size_t fwd_cls, fwd_ptr, fwd_ent, fwd_order;
    size_t bwd_cls, bwd_ptr, bwd_ent, bwd_order;
    size_t total_bytes;
} attn_index_layout;
attn_status attn_tile_index_layout(const attn_problem* prob, attn_index_layout* out);

/*
 * Build the tile index on the device from a descriptor (any kind but BLOCK_SPARSE).
 *   desc_dev  : device int32 [T][4] from attn_mask_desc_build
 *   index_dev : device buffer of attn_tile_index_size bytes
 */
attn_status attn_tile_index_build(const attn_problem* prob, const int32_t* desc_dev,
                                  void* index_dev, size_t index_bytes, void* stream);

/*
 * Build the block index on the device from a keep matrix (BLOCK_SPARSE only; the page's
 * "Uniform Block" dynamic mask, section 三 "动态掩码").
 *   keep_dev  : device uint8 [Hq][nb][nb], nb = ceil(T / sparse_block)
 *   index_dev : device buffer of attn_tile_index_size bytes
 */
attn_status attn_block_index_build(const attn_problem* prob, const uint8_t* keep_dev,
                                   void* index_dev, size_t index_bytes, void* stream);

/*
 * Dynamic block selection: the keep matrix of a block-sparse problem chosen from the
 * inputs themselves. The pages list Uniform Block as a dynamic mask (section 三
 * "注意力掩码模式", 动态掩码) and name TopK / TopP as the selection criterion of dynamic
 * block-sparse attention (the review's remarks on the paper's limitations); they give no
 * formula. The definition implemented here:
 *   block score  s[h][qb][kb] = scale * mean_Q[h][qb] . mean_K[h / G][kb], where
 *                mean_Q[h][qb] is the fp32 mean of the rows of query block qb of head h
 *                (the last block of a ragged T averages the rows it has), likewise mean_K;
 *   order        per (h, qb): block qb first if keep_diagonal, then the other blocks by
 *                descending score, equal scores by ascending kb;
 *   TOPK         keep the first min(topk, nb) blocks of the order;
 *   TOPP         keep the shortest prefix of the order whose mass under
 *                softmax_kb(s[h][qb][kb]) (natural exp, over all nb blocks) reaches topp.
 * Scores are fp32 (each a sequential FMA chain over the head dimension); the TopP masses
 * are fp32 sums, so a prefix whose mass lies within fp32 rounding of topp may end one
 * block earlier or later than an exact computation would.
 */
typedef enum attn_select_mode { ATTN_SELECT_TOPK = 0, ATTN_SELECT_TOPP = 1 } attn_select_mode;
typedef struct attn_block_select_params {
    int32_t mode;             /* attn_select_mode */
    int32_t topk;             /* TOPK: >= 1 (values above nb keep every block) */
    float topp;               /* TOPP: 0 < topp <= 1 */
    int32_t keep_diagonal;    /* nonzero: block (qb, qb) is always kept and counted first */
} attn_block_select_params;

/* Workspace bytes of attn_block_select (the fp32 block means of Q and K). */
attn_status attn_block_select_workspace_size(const attn_problem* prob, size_t* bytes_out);

/*
 *   prob      : a BLOCK_SPARSE problem (T, Hq, Hk, scale, sparse_block b); nb = ceil(T / b)
 *               must be <= 4096 (ATTN_ERR_UNSUPPORTED otherwise)
 *   q, k      : device bf16 [T][Hq][128], [T][Hk][128]
 *   scores    : device fp32 [Hq][nb][nb] output, the block scores
 *   keep_out  : device uint8 [Hq][nb][nb] output (0 / 1), ready for attn_block_index_build
 *   ws        : device workspace of attn_block_select_workspace_size bytes
 * Errors: ATTN_ERR_INVALID_ARG for a non-BLOCK_SPARSE problem, a null pointer, an unknown
 * mode, topk < 1 or topp outside (0, 1]; ATTN_ERR_WORKSPACE for a short workspace.
 */
attn_status attn_block_select(const attn_problem* prob, const attn_block_select_params* sp, const void* q,
                              const void* k, float* scores, uint8_t* keep_out, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * attn_block_select for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid allocation): the same selection, with
 * the same kernels and bit-identical results, but no workspace argument. The block means
 * live in a static device array of ATTN_SELECT_SCRATCH_BYTES (32 MiB), which every GPU the
 * library runs on holds from the module's load until the process ends; the first call on a
 * GPU looks up the array's device address (hipGetSymbolAddress; no allocation), later calls
 * reuse it. Nothing in the array needs clearing between calls (each call writes every mean
 * it reads). Calls on one GPU share the array and keep the last call's contents: calls that
 * overlap in time on one GPU (on different streams, or from several host threads) race and
 * must be serialised by the caller. Arguments and errors as attn_block_select, plus
 * ATTN_ERR_WORKSPACE when attn_block_select_workspace_size exceeds
 * ATTN_SELECT_SCRATCH_BYTES (64 query heads at T = 64K with b = 128 need 18.9 MB; with
 * b = 64, 37.7 MB exceeds it): nothing is launched then.
 */
#define ATTN_SELECT_SCRATCH_BYTES (32u << 20)
attn_status attn_block_select_noalloc(const attn_problem* prob, const attn_block_select_params* sp,
                                      const void* q, const void* k, float* scores, uint8_t* keep_out,
                                      void* stream);

/*
 * Variable Block mask (section 三 "注意力掩码模式", 动态掩码: block-sparse with variable
 * block sizes; no further definition on the pages). Row block r covers query positions
 * [row_off[r], row_off[r+1]), column block c key positions [col_off[c], col_off[c+1]), and
 *   visible(h, i, j) = keep_var[h][r(i)][c(j)] != 0.
 * With every block edge on a multiple of 64, each 64 x 64 tile lies inside one block
 * pair, so the mask is exactly the uniform 64-block mask this function writes (host,
 * synchronous); upload it and run the problem as BLOCK_SPARSE with sparse_block = 64.
 *   T          : sequence length
 *   Hq         : query heads
 *   row_off    : host int32 [n_rb + 1], 0 = row_off[0] < ... < row_off[n_rb] = T, the
 *                interior edges multiples of 64 (likewise col_off, n_cb)
 *   keep_var   : host uint8 [Hq][n_rb][n_cb]
 *   keep_out   : host uint8 [Hq][nt][nt], nt = ceil(T / 64), written entirely on success
 * Errors: ATTN_ERR_INVALID_ARG for null pointers, T out of range or edges that are not
 * as stated (nothing is written then).
 */
attn_status attn_variable_block_expand(int32_t T, int32_t Hq, const int32_t* row_off, int32_t n_rb,
                                       const int32_t* col_off, int32_t n_cb, const uint8_t* keep_var,
                                       uint8_t* keep_out);

/* Workspace bytes of attn_fwd / attn_bwd (0 means no workspace is needed). */
attn_status attn_fwd_workspace_size(const attn_problem* prob, size_t* bytes_out);
attn_status attn_bwd_workspace_size(const attn_problem* prob, size_t* bytes_out);

/*
 * Forward: O = softmax(scale * Q K^T + mask) V and LSE.
 *   q, k, v   : device bf16 inputs (layouts above)
 *   o         : device bf16 output [T][Hq][128] (the fp32 result rounded to nearest even)
 *   o_lo      : optional device bf16 output [T][Hq][128] (NULL: not written): the rounding
 *               residual O_fp32 - o, so that o + o_lo carries the forward's fp32 O. Passed
 *               to the backward it makes D = rowsum(dO * O) fp32-accurate.
 *   lse       : device fp32 output [Hq][T]
 *   desc_dev  : device descriptor (NULL for BLOCK_SPARSE)
 *   index_dev : tile / block index built for this problem
 *   ws        : workspace of attn_fwd_workspace_size bytes (may be NULL if that is 0)
 */
attn_status attn_fwd(const attn_problem* prob, const void* q, const void* k, const void* v,
                     void* o, void* o_lo, float* lse, const int32_t* desc_dev,
                     const void* index_dev, size_t index_bytes,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Backward: gradients of L with dL/dO = dout, given the forward's O and LSE.
 * Equivalent to attn_bwd_preprocess followed by attn_bwd_main.
 *   o, o_lo   : the forward's outputs (o_lo may be NULL: D then uses the bf16 O alone)
 *   dq        : device fp32 [T][Hq][128], overwritten
 *   dk, dv    : device fp32 [T][Hk][128], overwritten
 *   ws        : workspace of attn_bwd_workspace_size bytes (D = rowsum(dO * O), the operand
 *               bounds and the scaled fp16 operand copies of the preprocess; on short
 *               sequences also the partial dK / dV sums of split key tiles, see attn_bwd_main)
 * The three gradient products run on fp16 operands scaled by powers of two derived from
 * max |Q|, max |K|, max ||dO_i|| and max ||V_j|| (measured by the preprocess), which keeps
 * every operand in fp16 range; the scales are removed from the fp32 results.
 */
attn_status attn_bwd(const attn_problem* prob, const void* q, const void* k, const void* v,
                     const void* o, const void* o_lo, const float* lse, const void* dout,
                     float* dq, float* dk, float* dv, const int32_t* desc_dev,
                     const void* index_dev, size_t index_bytes,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Backward, first step: D[h][i] = sum_c dO[i][h][c] * (o + o_lo)[i][h][c] into the
 * workspace (fp32 [Hq][T]) and the operand bounds (max |Q|, max |K|, max ||dO_i||^2,
 * max ||V_j||^2) after it.
 */
attn_status attn_bwd_preprocess(const attn_problem* prob, const void* q, const void* k,
                                const void* v, const void* o, const void* o_lo,
                                const void* dout, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward, second step: recompute P on the non-empty tiles and write dV = P^T dO and
 * dK = scale * dS^T Q (key-tile major, each key written once) and dQ = scale * dS K
 * (query-tile major, each row written once), with dS = P * (dO V^T - D). No atomics: the
 * gradients are deterministic. Requires attn_bwd_preprocess on the same ws first (stream
 * order). When the dense key tiles are too few to fill the GPU (Hk times the key tiles
 * under 512, i.e. short sequences), each key tile's query list is cut into 2, 4 or 8
 * pieces whose partial dK / dV sums go to the end of ws and are then added in a fixed
 * order (still deterministic): ws is then written, so calls that share one ws must not
 * overlap.
 */
attn_status attn_bwd_main(const attn_problem* prob, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout,
                          float* dq, float* dk, float* dv, const int32_t* desc_dev,
                          const void* index_dev, size_t index_bytes,
                          void* ws, size_t ws_bytes, void* stream);

/* The two halves of attn_bwd_main, for callers that time or schedule them apart:
 * attn_bwd_dkdv writes dK and dV (key-tile major), attn_bwd_dq writes dQ (query-tile
 * major). Both read the inputs, the forward's LSE and the preprocessed workspace;
 * attn_bwd_dq only reads ws, attn_bwd_dkdv also writes the partial sums of split key tiles
 * into it on short sequences (as attn_bwd_main does). */
attn_status attn_bwd_dkdv(const attn_problem* prob, const void* q, const void* k, const void* v,
                          const float* lse, const void* dout, float* dk, float* dv,
                          const int32_t* desc_dev, const void* index_dev, size_t index_bytes,
                          void* ws, size_t ws_bytes, void* stream);
attn_status attn_bwd_dq(const attn_problem* prob, const void* q, const void* k, const void* v,
                        const float* lse, const void* dout, float* dq,
                        const int32_t* desc_dev, const void* index_dev, size_t index_bytes,
                        const void* ws, size_t ws_bytes, void* stream);

/* Optional cast of fp32 gradients to bf16: out[i] = bf16(in[i]), rounded to nearest with ties
 * to even (the largest finite values round to infinity; infinities keep their sign; a NaN
 * gives a NaN; subnormals are rounded, not flushed). in: device fp32 [n]; out: device bf16
 * [n]. n = 0 is a no-op; null pointers with n > 0 give ATTN_ERR_INVALID_ARG. */
attn_status attn_cast_bf16(const float* in, void* out, size_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLCT_ATTN_H */
