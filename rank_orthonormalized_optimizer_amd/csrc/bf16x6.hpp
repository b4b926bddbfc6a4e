// fp32-accurate products on the bf16 matrix cores of gfx950 (v_mfma_f32_16x16x32_bf16).
//
// An fp32 value a is split exactly into three bf16 parts, a = (h + m) + l with h = RN(a),
// m = RN(a - h) and l = a - h - m (exact: at most eight significant bits are left).  The
// product a b is then the sum of the nine part products; the six kept here (hh, hm, mh, hl,
// lh, mm) leave out terms below 2^-24 |a b|, the size of one fp32 rounding, and the matrix
// core adds the kept products in fp32.  One bf16 MFMA does 16 x 16 x 32 at about 14 times the
// flop rate of the fp32 MFMA, so the six cost about 0.42 of the fp32 MFMA work.
//
// Split operands are stored as three planes [part][rows][kp] of bf16 (h, m, l), with kp the
// contraction length rounded up to a multiple of 32 and zero padding, so every row starts on
// a 64-byte boundary and a k-slab of 32 is four 16-byte chunks per row.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (measured on gfx950 with a one-wave probe):
//   A: lane l holds A[l % 16][8 (l / 16) + i], i = 0..7
//   B: lane l holds B[8 (l / 16) + i][l % 16]
//   D: lane l, element v holds D[4 (l / 16) + v][l % 16]  (as v_mfma_f32_16x16x4_f32)
// so a fragment is one 16-byte chunk of a k-contiguous row of either operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dion {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSplitK = 32;   // k-slab of one bf16 MFMA and padding unit of the planes

__host__ __device__ constexpr int64_t split_kp(int64_t k) { return (k + kSplitK - 1) / kSplitK * kSplitK; }

__device__ __forceinline__ void split3(float a, uint16_t& h, uint16_t& m, uint16_t& l) {
    const __bf16 bh = (__bf16)a;           // round to nearest even
    const float r1 = a - (float)bh;        // exact
    const __bf16 bm = (__bf16)r1;
    const float r2 = r1 - (float)bm;       // exact
    const __bf16 bl = (__bf16)r2;          // exact
    h = __builtin_bit_cast(uint16_t, bh);
    m = __builtin_bit_cast(uint16_t, bm);
    l = __builtin_bit_cast(uint16_t, bl);
}

// Element offset of 8-element chunk c (0..3) of row x in a 64 x 32 part tile in LDS.  Rows are
// 64 bytes, so rows x and x + 4 share banks; XORing the chunk with bits 2..3 of x spreads the 16
// rows a fragment read touches over all 64 banks, and a wave's tile store stays conflict-free.
__device__ __forceinline__ int part_off(int x, int c) { return x * kSplitK + ((c ^ ((x >> 2) & 3)) << 3); }

__device__ __forceinline__ f32x4 mma_bf16(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// The six kept part products, smallest first: (part of A, part of B) with 0 = h, 1 = m, 2 = l.
constexpr int kTermA[6] = {1, 0, 2, 0, 1, 0};
constexpr int kTermB[6] = {1, 2, 0, 1, 0, 0};

}  // namespace dion
