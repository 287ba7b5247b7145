// Shared device types, MFMA wrappers and the tile-index layout (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/attn.h"

namespace mlct {

constexpr int HEAD_DIM = 128;
constexpr int FWD_BN = 64;          // keys per forward tile
constexpr int BWD_BN = 128;         // keys per dense backward tile (4 waves x 32 keys)
constexpr int ROWS_PER_WG = 256;    // (head, position) rows per dense forward work item
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D = A * B + C for a 32x32 output tile with K = 16, bf16 inputs, fp32 accumulation.
// Lane l holds row (A) / column (B) l % 32 and the eight K-slots selected by l / 32;
// the accumulator holds column l % 32, rows 8*(r/4) + 4*(l/32) + r%4 for register r.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Same shape with fp16 inputs.
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row (within a 32-row block) held by accumulator register r of a lane in half hf.
__device__ __forceinline__ constexpr int acc_row(int r, int hf) {
    return 8 * (r >> 2) + 4 * hf + (r & 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// The two bf16 halves of a 32-bit word, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// Two fp32 -> packed fp16 pair (round to nearest even; v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Exchange a float with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its outstanding global loads, stores or atomics (register results of global loads are
// still waited for at their first use by the compiler).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Round an offset up to 256 bytes.
__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Host-side description of one problem after validation.
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

// Backward workspace: D [Hq][T] fp32, then BWD_STATS fp32 bounds used to pick the
// power-of-two scales of the fp16 operands (see bwd.hip).
constexpr int BWD_STATS = 4;
__host__ __device__ constexpr size_t bwd_stats_offset(int Hq, int T) { return align256((size_t)Hq * T * 4); }
__host__ __device__ constexpr size_t bwd_workspace_bytes(int Hq, int T) { return bwd_stats_offset(Hq, T) + 256; }

struct IndexLayout {
    size_t fwd_cls, fwd_ptr, fwd_ent, fwd_order;
    size_t bwd_cls, bwd_ptr, bwd_ent, bwd_order;
    size_t total;
};

attn_status validate_problem(const attn_problem* p, Problem* out);
IndexLayout index_layout(const Problem& P);

// Kernel launchers (defined next to their kernels).
hipError_t launch_index_dense(const Problem& P, const int4* desc, void* index, hipStream_t s);
hipError_t launch_index_sparse(const Problem& P, const uint8_t* keep, void* index, hipStream_t s);
hipError_t launch_fwd(const Problem& P, const void* q, const void* k, const void* v, void* o, void* o_lo,
                      float* lse, const int4* desc, const void* index, hipStream_t s);
hipError_t launch_bwd_pre(const Problem& P, const void* q, const void* k, const void* v, const void* o,
                          const void* o_lo, const void* dout, float* dbuf, hipStream_t s);
enum { BWD_PART_DKDV = 1, BWD_PART_DQ = 2 };
hipError_t launch_bwd_main(const Problem& P, const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, const int4* desc,
                           const void* index, const float* dbuf, int parts, hipStream_t s);
hipError_t launch_cast_bf16(const float* in, void* out, size_t n, hipStream_t s);

}  // namespace mlct
