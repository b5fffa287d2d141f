// hh_common.h -- device-side helpers shared by the libhh kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (v_mfma_f32_16x16x32_bf16, one wave
// of 64 lanes, lane = 16 * g + r16 with g = lane / 16, r16 = lane % 16):
//   A operand (16 x 32, row-major M x K): lane holds row r16, K slots 8g .. 8g+7
//   B operand (32 x 16, K x N):          lane holds column r16, K slots 8g .. 8g+7
//   C/D accumulator (16 x 16):           lane holds column r16, rows 4g .. 4g+3
// The contraction only needs the A and B operands to agree on which K index
// sits in each (g, slot) position, so K may be permuted freely as long as both
// sides use the same permutation.  The kernels use this to feed an accumulator
// straight back in as an operand: two 16-row accumulator blocks (rows 0..15
// and 16..31 of a 32-wide K step) give lane group g the K indices
// {4g..4g+3, 16+4g..16+4g+3}, and the partner operand is read in that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hh {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint16_t bf16_t;  // raw storage of one bfloat16 in global memory

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int s = 0; s < 8; s++) z[s] = (__bf16)0.0f;
    return z;
}

__device__ __forceinline__ bf16x8 ones_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int s = 0; s < 8; s++) z[s] = (__bf16)1.0f;
    return z;
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4 &v) {
    bf16x4 r;
    r[0] = (__bf16)v[0];
    r[1] = (__bf16)v[1];
    r[2] = (__bf16)v[2];
    r[3] = (__bf16)v[3];
    return r;
}

__device__ __forceinline__ bf16x8 cat(const bf16x4 &lo, const bf16x4 &hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two accumulator blocks (K rows 0..15 and 16..31 of one K step) as a B or A operand.
__device__ __forceinline__ bf16x8 acc_pair_to_operand(const f32x4 &lo, const f32x4 &hi) {
    return cat(to_bf16x4(lo), to_bf16x4(hi));
}

__device__ __forceinline__ bf16x8 load8(const bf16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ bf16x4 load4(const bf16_t *p) {
    return *reinterpret_cast<const bf16x4 *>(p);
}
__device__ __forceinline__ void store4(bf16_t *p, const bf16x4 &v) {
    *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store8(bf16_t *p, const bf16x8 &v) {
    *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ float bf16_bits_to_float(bf16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ bf16_t float_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return *reinterpret_cast<bf16_t *>(&b);
}

// A tile whose rows feed the matrix cores in the K order of an accumulator pair (elements
// 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3 of each 32-wide K step, for lane group g) can be
// kept with each 32-column group reordered so that the 4-column runs g and g + 4 sit side by
// side at 8 g: each operand is then one 16-byte read.  Run r of a group goes to position 8 r
// (r < 4) or 8 (r - 4) + 4.
__device__ __forceinline__ int qperm_pos(int col) {
    const int r = (col & 31) >> 2;
    return (col & ~31) + (r < 4 ? 8 * r : 8 * (r - 4) + 4) + (col & 3);
}
// Eight consecutive columns col .. col + 7 (col a multiple of 8) of a reordered row.
__device__ __forceinline__ void store8_qperm(bf16_t *row, int col, const bf16x8 &x) {
    store4(row + qperm_pos(col), __builtin_shufflevector(x, x, 0, 1, 2, 3));
    store4(row + qperm_pos(col + 4), __builtin_shufflevector(x, x, 4, 5, 6, 7));
}

// Copy of N16 16-byte pieces from global memory into LDS by the NT threads of a workgroup
// (thread tid moves pieces tid, tid + NT, ...): piece e comes from src_of(e) (or is zero where
// live(e) is false) and goes to dst_of(e).  Every load is issued before the first store: a loop
// that stores each piece before loading the next waits one memory latency per piece.
template <int NT, int N16, typename Src, typename Dst, typename Live>
__device__ __forceinline__ void stage_pieces(int tid, Src src_of, Dst dst_of, Live live) {
    constexpr int PER = (N16 + NT - 1) / NT;
    bf16x8 tmp[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int e = tid + NT * i;
        tmp[i] = (N16 % NT == 0 || e < N16) && live(e) ? load8(src_of(e)) : zero_bf16x8();
    }
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int e = tid + NT * i;
        if (N16 % NT == 0 || e < N16) store8(dst_of(e), tmp[i]);
    }
}

// Workgroup -> (head bh, segment s) for grids of BH x nseg workgroups.  Workgroups are dealt to
// the eight XCDs round-robin (blockIdx mod 8); when BH is a multiple of 8, all segments of a head
// go to one XCD, so that the head's W (and its state slot) is fetched into that XCD's L2 once.
__device__ __forceinline__ void wg_head_segment(int nseg, int &bh, int &s) {
    const int b = blockIdx.x, BH = gridDim.x / nseg;
    if (BH % 8 == 0) {
        const int j = b >> 3;
        bh = (b & 7) + 8 * (j / nseg);
        s = j % nseg;
    } else {
        bh = b / nseg;
        s = b % nseg;
    }
}

}  // namespace hh
