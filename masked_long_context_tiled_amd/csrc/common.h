// Shared device types, MFMA wrappers and the tile-index layout (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "host.h"

namespace mlct {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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

// Compile-time flag passed to generic lambdas (decltype(tag)::value).
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Bits b = 0..31 with base + b in [lo, hi): the rows of a half-open row interval among 32
// consecutive positions starting at base.
__device__ __forceinline__ uint32_t interval_bits(int lo, int hi, int base) {
    const int a = min(max(lo - base, 0), 32), b = min(max(hi - base, 0), 32);
    const uint64_t m = ((1ull << b) - 1ull) & ~((1ull << a) - 1ull);
    return (uint32_t)m;
}

// Exchange a float with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its outstanding global loads, stores or atomics (register results of global loads are
// still waited for at their first use by the compiler).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, source lane s
// supplies the address of 4 consecutive 16-bit elements and output lane i receives
// element i % 4 of source lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12. With source lane s
// pointing at M[r0 + s/4][c0 + 4*(s%4)], output lane i gets M[r0 .. r0+3][c0 + i].
__device__ __forceinline__ u32x2 ds_read_tr16(const void* p) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// List entries of a work item, 64 per register: lane i of chunk register c holds entry
// 64 c + i. Entries are read in non-decreasing order; the chunk after the current one is
// loaded a whole chunk ahead and only touched (waited for) when the reader moves on to it.
// With rev, get(j) returns the list's entry n - 1 - j (the list walked from its end).
struct EntryStream {
    const int* ent;
    int first, dir, n, chunk, cur, nxt;
    __device__ __forceinline__ int load(int c, int lane) const {
        const int j = 64 * c + lane;
        return j < n ? ent[first + dir * j] : 0;
    }
    __device__ __forceinline__ void init(const int* e, int lb_, int n_, int lane, bool rev = false) {
        ent = e;
        first = rev ? lb_ + n_ - 1 : lb_;
        dir = rev ? -1 : 1;
        n = n_;
        chunk = 0;
        cur = load(0, lane);
        nxt = load(1, lane);
    }
    __device__ __forceinline__ int get(int j, int lane) {
        if ((j >> 6) != chunk) {
            cur = nxt;
            ++chunk;
            nxt = load(chunk + 1, lane);
        }
        return __builtin_amdgcn_readlane(cur, j & 63);
    }
};

// N MFMAs whose LDS operand (16 bytes per lane) is read three MFMAs ahead of its use. The
// scheduling fences keep that order; left alone, the compiler tends to wait for each read
// right before its MFMA.
template <int N, class Read, class Mma>
__device__ __forceinline__ void mfma_pipelined(Read read, Mma mma) {
    u32x4 ring[4];
    ring[0] = read(0);
    ring[1] = read(1);
    ring[2] = read(2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i + 3 < N) ring[(i + 3) & 3] = read(i + 3);
        mma(i, ring[i & 3]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Staged Q / dO rows: 128 fp16 (256 bytes) per row, the 16-byte chunk c of row q stored at
// chunk slot c ^ 4*(q % 4) ^ (q / 4 % 4). Sixteen consecutive rows of one chunk (row
// reads) and a 4-row x 4-chunk block (transposed reads) both land on distinct banks.
__device__ __forceinline__ int swz(int q, int c) { return c ^ (4 * (q & 3)) ^ ((q >> 2) & 3); }
__device__ __forceinline__ int swz_off(int q, int col) { return q * HEAD_DIM + swz(q, col >> 3) * 8 + (col & 7); }

// A operand (32 rows x 16 k) of 16-bit elements whose row m = lane % 32 is column c0 + m
// of a swizzled [rows][128] matrix M, k-slots e = 0..3 of the lane being rows r_lo + e and
// e = 4..7 rows r_hi + e - 4 (callers fold the lane half into r_lo / r_hi).
__device__ __forceinline__ u32x4 tr_rows_swz(const void* M, int r_lo, int r_hi, int c0, int lane) {
    const uint16_t* m = static_cast<const uint16_t*>(M);
    const int s = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const u32x2 lo = ds_read_tr16(m + swz_off(r_lo + (s >> 2), col));
    const u32x2 hi = ds_read_tr16(m + swz_off(r_hi + (s >> 2), col));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ f16x8 tr_operand_swz(const _Float16* M, int r_lo, int r_hi, int c0, int lane) {
    return as_f16x8(tr_rows_swz(M, r_lo, r_hi, c0, lane));
}

// A operand (32 rows x 16 k) of 16-bit elements whose row m = lane % 32 is column c0 + m
// of the row-major [rows][ld] matrix M; k-slots e = 0..3 are rows r_lo + e, e = 4..7 rows
// r_hi + e - 4 (callers fold the lane half into r_lo / r_hi).
__device__ __forceinline__ u32x4 tr_rows_ld(const void* Mv, int ld, int r_lo, int r_hi, int c0, int lane) {
    const uint16_t* M = static_cast<const uint16_t*>(Mv);
    const int s = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const u32x2 lo = ds_read_tr16(M + (r_lo + (s >> 2)) * ld + col);
    const u32x2 hi = ds_read_tr16(M + (r_hi + (s >> 2)) * ld + col);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Staged row blocks with a per-row skew instead of the XOR swizzle: row q of 128 fp16
// starts at element 256 q + 8 (4 (q mod 4) + (q / 4) mod 4), its 16-byte chunks in order,
// so a row takes 512 bytes of LDS. The skew puts 16 consecutive rows of one chunk, and a
// 4-row x 4-chunk block, on distinct banks (as the swizzle does), while every operand
// address is a per-lane row base plus a compile-time chunk offset.
constexpr int SKEW_PITCH = 256;
__device__ __forceinline__ int skew_off(int q, int col) {
    return q * SKEW_PITCH + 8 * (4 * (q & 3) + ((q >> 2) & 3)) + col;
}
// tr_rows_swz for a skewed block, with r_lo = rb16 + 4 hf, r_hi = r_lo + 8 (rb16 a
// multiple of 16): the skew of rows r_lo + s / 4 and r_hi + s / 4 depends on the lane only.
__device__ __forceinline__ u32x4 tr_rows_skew(const void* Mv, int rb16, int c0, int lane) {
    const uint16_t* M = static_cast<const uint16_t*>(Mv);
    const int s = lane & 15, g = (lane >> 4) & 1, hf = lane >> 5;
    const int lanepart = (4 * hf + (s >> 2)) * SKEW_PITCH + 8 * (4 * (s >> 2) + hf) + 16 * g + 4 * (s & 3);
    const uint16_t* p = M + lanepart + rb16 * SKEW_PITCH + c0;
    const u32x2 lo = ds_read_tr16(p);
    const u32x2 hi = ds_read_tr16(p + 8 * SKEW_PITCH + 16);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

}  // namespace mlct
