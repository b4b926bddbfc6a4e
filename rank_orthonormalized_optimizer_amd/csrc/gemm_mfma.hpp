// Batched MFMA GEMM building block for the Dion step on gfx950 (CDNA4).
//
// Every contraction of the step (B Q, P^T P, triangular solves and updates,
// B^T P, and the rank-r expansions of the momentum/weight pass) is
// C = alpha * op(A) op(B) + beta * C on one matrix of a stack, with operands
// read straight from the state buffers.  This header holds the shared tile
// engine: 256 threads = 4 wave64s in a 2 x 2 arrangement, each wave owning a
// (BM/2) x (BN/2) sub-tile built from 16 x 16 MFMA blocks
// (v_mfma_f64_16x16x4_f64 for double, v_mfma_f32_16x16x4_f32 for float).
//
// Operands are staged through LDS as [k][x] tiles (x = row of A or column of
// B), padded so the four 16-lane groups of a fragment read hit disjoint banks.
// Global loads are 4-element vectors along whichever index is contiguous in
// memory, prefetched into registers one k-tile ahead of the MFMA work.
//
// MFMA operand/result lane mapping (16 x 16 x 4, one block):
//   A: lane l holds A[l % 16][l / 16]      B: lane l holds B[l / 16][l % 16]
//   D: lane l, element v holds D[row][l % 16] with
//        row = 4 * (l / 16) + v   for v_mfma_f32_16x16x4_f32
//        row = (l / 16) + 4 * v   for v_mfma_f64_16x16x4_f64
//   (measured on gfx950 with a one-wave probe of each builtin).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dion {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma;
template <> struct Mfma<float> {
    using acc_t = f32x4;
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // row (within the 16 x 16 block) of result element v of lane `lane`
    static __device__ __forceinline__ int row(int lane, int v) { return 4 * (lane >> 4) + v; }
};
template <> struct Mfma<double> {
    using acc_t = f64x4;
    static __device__ __forceinline__ acc_t mma(double a, double b, acc_t c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lane, int v) { return (lane >> 4) + 4 * v; }
};

// Storage kinds an operand can be read from.
enum Src : int {
    SRC_F32 = 0,       // float
    SRC_F64 = 1,       // double
    SRC_BF16 = 2,      // bfloat16 bits
    SRC_SUM_F32 = 3,   // p0 (float) + p1 (float): B = M + G with G in fp32
    SRC_SUM_BF16 = 4   // p0 (float) + p1 (bf16):  B = M + G with G in bf16
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float -> bfloat16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One element at element offset `off`.  For the SUM kinds the two addends are
// widened to T first, so in double the sum is exact and in float it is rounded once.
template <typename T, int SRC>
__device__ __forceinline__ T load1(const void* p0, const void* p1, int64_t off) {
    if constexpr (SRC == SRC_F32) return (T)((const float*)p0)[off];
    else if constexpr (SRC == SRC_F64) return (T)((const double*)p0)[off];
    else if constexpr (SRC == SRC_BF16) return (T)bf16_bits_to_float(((const uint16_t*)p0)[off]);
    else if constexpr (SRC == SRC_SUM_F32) return (T)((const float*)p0)[off] + (T)((const float*)p1)[off];
    else return (T)((const float*)p0)[off] + (T)bf16_bits_to_float(((const uint16_t*)p1)[off]);
}

// Four consecutive elements; requires 4-element alignment of `off` and the base.
template <typename T, int SRC>
__device__ __forceinline__ void load4(const void* p0, const void* p1, int64_t off, T (&o)[4]) {
    if constexpr (SRC == SRC_F32) {
        float4 v = *(const float4*)((const float*)p0 + off);
        o[0] = (T)v.x; o[1] = (T)v.y; o[2] = (T)v.z; o[3] = (T)v.w;
    } else if constexpr (SRC == SRC_F64) {
        double2 a = *(const double2*)((const double*)p0 + off);
        double2 b = *(const double2*)((const double*)p0 + off + 2);
        o[0] = (T)a.x; o[1] = (T)a.y; o[2] = (T)b.x; o[3] = (T)b.y;
    } else if constexpr (SRC == SRC_BF16) {
        uint2 v = *(const uint2*)((const uint16_t*)p0 + off);
        o[0] = (T)bf16_bits_to_float(v.x & 0xffffu); o[1] = (T)bf16_bits_to_float(v.x >> 16);
        o[2] = (T)bf16_bits_to_float(v.y & 0xffffu); o[3] = (T)bf16_bits_to_float(v.y >> 16);
    } else if constexpr (SRC == SRC_SUM_F32) {
        float4 a = *(const float4*)((const float*)p0 + off);
        float4 b = *(const float4*)((const float*)p1 + off);
        o[0] = (T)a.x + (T)b.x; o[1] = (T)a.y + (T)b.y; o[2] = (T)a.z + (T)b.z; o[3] = (T)a.w + (T)b.w;
    } else {
        float4 a = *(const float4*)((const float*)p0 + off);
        uint2 b = *(const uint2*)((const uint16_t*)p1 + off);
        o[0] = (T)a.x + (T)bf16_bits_to_float(b.x & 0xffffu);
        o[1] = (T)a.y + (T)bf16_bits_to_float(b.x >> 16);
        o[2] = (T)a.z + (T)bf16_bits_to_float(b.y & 0xffffu);
        o[3] = (T)a.w + (T)bf16_bits_to_float(b.y >> 16);
    }
}

// Operand view: element (x, k) sits at base[x * ld + k] when KC (k contiguous)
// and at base[k * ld + x] otherwise.  x runs over [0, xext), k over [0, kext).
struct Operand {
    const void* p0;
    const void* p1;
    int64_t ld;
    int xext, kext;
    bool vec;   // 4-element vector loads are legal (base, ld and stride aligned)
};

// Register-staged loader of one BX x BK operand tile.
template <typename T, int BX, int BK, bool KC, int SRC>
struct TileLoader {
    static constexpr int GROUPS = BX * BK / 4;
    static_assert(GROUPS % 256 == 0, "tile must give every thread whole 4-element groups");
    static constexpr int PER = GROUPS / 256;
    T r[PER][4];

    __device__ __forceinline__ void load(const Operand& op, int x0, int k0) {
#pragma unroll
        for (int g = 0; g < PER; ++g) {
            const int idx = threadIdx.x + g * 256;
            int x, k;
            if constexpr (KC) { x = x0 + idx / (BK / 4); k = k0 + (idx % (BK / 4)) * 4; }
            else { k = k0 + idx / (BX / 4); x = x0 + (idx % (BX / 4)) * 4; }
            const int64_t off = KC ? (int64_t)x * op.ld + k : (int64_t)k * op.ld + x;
            const bool full = KC ? (x < op.xext && k + 3 < op.kext) : (k < op.kext && x + 3 < op.xext);
            if (op.vec && full) {
                load4<T, SRC>(op.p0, op.p1, off, r[g]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int xx = KC ? x : x + v;
                    const int kk = KC ? k + v : k;
                    r[g][v] = (xx < op.xext && kk < op.kext) ? load1<T, SRC>(op.p0, op.p1, off + v) : T(0);
                }
            }
        }
    }
    // LDS tile layout: s[k * LDX + x]
    template <int LDX>
    __device__ __forceinline__ void store(T* s) const {
#pragma unroll
        for (int g = 0; g < PER; ++g) {
            const int idx = threadIdx.x + g * 256;
            if constexpr (KC) {
                const int x = idx / (BK / 4), k = (idx % (BK / 4)) * 4;
#pragma unroll
                for (int v = 0; v < 4; ++v) s[(k + v) * LDX + x] = r[g][v];
            } else {
                const int k = idx / (BX / 4), x = (idx % (BX / 4)) * 4;
#pragma unroll
                for (int v = 0; v < 4; ++v) s[k * LDX + x + v] = r[g][v];
            }
        }
    }
};

// Tile geometry shared by the kernels.
template <typename T, int BM_, int BN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 16, PAD = 16;
    static constexpr int LDA = BM + PAD, LDB = BN + PAD;
    static constexpr int WTM = BM / 2, WTN = BN / 2;   // wave sub-tile
    static constexpr int FM = WTM / 16, FN = WTN / 16; // MFMA blocks per wave
    using acc_t = typename Mfma<T>::acc_t;
};

// acc[i][j] += A_frag[i] * B_frag[j] over one BK slab of LDS.
template <typename T, class C>
__device__ __forceinline__ void mma_slab(const T* As, const T* Bs, typename C::acc_t (&acc)[C::FM][C::FN],
                                         int wm, int wn, int lane) {
    const int lr = lane & 15, lk = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += 4) {
        T a[C::FM], b[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) a[i] = As[(kk + lk) * C::LDA + wm * C::WTM + i * 16 + lr];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) b[j] = Bs[(kk + lk) * C::LDB + wn * C::WTN + j * 16 + lr];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) acc[i][j] = Mfma<T>::mma(a[i], b[j], acc[i][j]);
    }
}

}  // namespace dion
