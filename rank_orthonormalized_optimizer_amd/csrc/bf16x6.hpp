// fp32-accurate products on the bf16 matrix cores of gfx950 (v_mfma_f32_16x16x32_bf16).
//
// An fp32 value a is split exactly into three bf16 parts, a = (h + m) + l with h = RN(a),
// m = RN(a - h) and l = a - h - m (exact: at most eight significant bits are left).  The
// product a b is then the sum of the nine part products; the six kept here (hh, hm, mh, hl,
// lh, mm) leave out terms below 2^-24 |a b|, the size of one fp32 rounding, and the matrix
// core adds the kept products in fp32.  One bf16 MFMA does 16 x 16 x 32 at about 14 times the
// flop rate of the fp32 MFMA, so the six cost about 0.42 of the fp32 MFMA work.
//
// Operands stay fp32 in memory and are split while they are staged into LDS, as three bf16
// part tiles (h, m, l) of one 32-k slab, with zeros beyond the contraction length.
//
// The same machinery runs plain bf16 products (operands rounded once to bf16, fp32
// accumulation) when the template parameter NP, the number of parts staged, is 1: only h is
// stored and only the hh product is issued.  That is the arithmetic of stacks whose weights
// are bf16, where the accepted error is that of bf16 (2^-8 relative per operand).
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

constexpr int kSplitK = 32;   // k-slab of one bf16 MFMA

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

namespace dion {

// ---------------------------------------------------------------------------
// Operand tiles of BX rows (x) by one 32-k slab, staged into LDS as three swizzled bf16 part
// tiles [x][32] (part_off).  Each of 256 staging threads (index t) owns a fixed share: load()
// fetches its raw values, split() turns them into bf16 parts in registers, store() writes them.
// ---------------------------------------------------------------------------
enum Src6 : int {
    S6_KC8 = 0,      // fp32 p0[x * ld + k], k contiguous, staged in chunks of eight k
    S6_KC = 1,       // fp32 p0[x * ld + k] (+ addend p1 at the same index), k contiguous
    S6_XC4 = 4,      // fp32 p0[k * ld + x] (+ addend p1 at the same index), x contiguous, staged as
                     // 16-byte row vectors (four x by four k per thread)
};
enum Add6 : int { A6_NONE = 0, A6_F32 = 1, A6_BF16 = 2 };

struct Op6 {
    const void* p0;
    const void* p1;     // addend (B = M + G), or null
    int64_t ld;         // pitch in elements between rows of the stored array
    int xext, kext;     // valid extents along x and k (outside: zeros)
    bool vec;           // S6_KC: 4-element vector loads are legal (ld, bases aligned)
};

// value of element (raw a, raw b) of a sum source: one fp32 addition (correctly rounded)
template <int ADD> struct Add6T { using t = float; };
template <> struct Add6T<A6_BF16> { using t = uint16_t; };
template <int ADD>
__device__ __forceinline__ float sum6(float a, typename Add6T<ADD>::t b) {
    if constexpr (ADD == A6_NONE) return a;
    else if constexpr (ADD == A6_BF16) return a + __uint_as_float((uint32_t)b << 16);
    else return a + b;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// two values at once: packed (h, m, l) parts, low half = first value
__device__ __forceinline__ void split3x2(float a0, float a1, uint32_t& h, uint32_t& m, uint32_t& l) {
    const f32x2_t a = {a0, a1};
    const bf16x2_t bh = __builtin_convertvector(a, bf16x2_t);
    const f32x2_t r1 = a - __builtin_convertvector(bh, f32x2_t);
    const bf16x2_t bm = __builtin_convertvector(r1, bf16x2_t);
    const f32x2_t r2 = r1 - __builtin_convertvector(bm, f32x2_t);
    const bf16x2_t bl = __builtin_convertvector(r2, bf16x2_t);
    h = __builtin_bit_cast(uint32_t, bh);
    m = __builtin_bit_cast(uint32_t, bm);
    l = __builtin_bit_cast(uint32_t, bl);
}

// four consecutive k, split: parts p[0..2] as packed pairs
struct Parts4 { u32x2 p[3]; };
__device__ __forceinline__ Parts4 split4(const float (&v)[4]) {
    Parts4 r;
    uint32_t h0, m0, l0, h1, m1, l1;
    split3x2(v[0], v[1], h0, m0, l0);
    split3x2(v[2], v[3], h1, m1, l1);
    r.p[0] = u32x2{h0, h1};
    r.p[1] = u32x2{m0, m1};
    r.p[2] = u32x2{l0, l1};
    return r;
}
// write them at k (k % 4 == 0 within the slab) of row x of the first NP part tiles
template <int NP>
__device__ __forceinline__ void store4(uint16_t* lds, int part_stride, int x, int k, const Parts4& q) {
    const int off = part_off(x, k >> 3) + (k & 7);
#pragma unroll
    for (int p = 0; p < NP; ++p) *(u32x2*)&lds[p * part_stride + off] = q.p[p];
}

// NT: the number of staging threads (256 or 512) that share one operand tile
template <int BX, int KIND, int ADD, int NT = 256>
struct Loader6;

// k-contiguous fp32, no addend, in chunks of eight k: BX * 4 chunks, BX / 64 per thread (four
// threads per row), so each part of a chunk is one 16-byte LDS write at its swizzled slot.
template <int BX, int ADD, int NT>
struct Loader6<BX, S6_KC8, ADD, NT> {
    static_assert(ADD == A6_NONE && NT == 256, "no addend, 256 threads");
    static constexpr int PER = BX / 64;
    float a[PER][8];
    __device__ __forceinline__ void load_fast(const Op6& op, int x0, int k0, int t) {
        const int xr = t >> 2, kk = 8 * (t & 3);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const float* src = (const float*)op.p0 + (int64_t)(x0 + xr + 64 * q) * op.ld + k0 + kk;
            const float4 v0 = *(const float4*)src, v1 = *(const float4*)(src + 4);
            a[q][0] = v0.x; a[q][1] = v0.y; a[q][2] = v0.z; a[q][3] = v0.w;
            a[q][4] = v1.x; a[q][5] = v1.y; a[q][6] = v1.z; a[q][7] = v1.w;
        }
    }
    static __device__ __forceinline__ bool interior(const Op6& op, int x0, int k0) {
        return op.vec && x0 + BX <= op.xext && k0 + kSplitK <= op.kext;
    }
    __device__ __forceinline__ void load(const Op6& op, int x0, int k0, int t) {
        if (interior(op, x0, k0)) { load_fast(op, x0, k0, t); return; }
        const int xr = t >> 2, kk = 8 * (t & 3);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int x = x0 + xr + 64 * q, k = k0 + kk;
            const int64_t o = (int64_t)(x < op.xext ? x : 0) * op.ld + k;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a[q][e] = (x < op.xext && k + e < op.kext) ? ((const float*)op.p0)[o + e] : 0.f;
        }
    }
    template <int NP = 3>
    __device__ __forceinline__ void split_store(uint16_t* lds, int t) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const float v0[4] = {a[q][0], a[q][1], a[q][2], a[q][3]};
            const float v1[4] = {a[q][4], a[q][5], a[q][6], a[q][7]};
            const Parts4 lo = split4(v0), hi = split4(v1);
            const int off = part_off((t >> 2) + 64 * q, t & 3);
#pragma unroll
            for (int p = 0; p < NP; ++p)
                *(u32x4*)&lds[p * BX * kSplitK + off] = u32x4{lo.p[p].x, lo.p[p].y, hi.p[p].x, hi.p[p].y};
        }
    }
};

// k-contiguous fp32 (+ addend): BX * 8 groups of four k, BX * 8 / NT per thread (8 threads per row).
// Interior tiles with vector-aligned rows take unchecked 4-element loads.
template <int BX, int ADD, int NT>
struct Loader6<BX, S6_KC, ADD, NT> {
    static constexpr int RP = NT / 8, PER = BX / RP;   // rows per pass, passes
    using AT = typename Add6T<ADD>::t;
    float a[PER][4];
    AT b[ADD == A6_NONE ? 1 : PER][4];
    Parts4 sp[PER];
    // interior tile (vector-legal, whole slab): no bounds tests
    __device__ __forceinline__ void load_fast(const Op6& op, int x0, int k0, int t) {
        const int xr = t >> 3, kk = 4 * (t & 7);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int64_t o = (int64_t)(x0 + xr + RP * q) * op.ld + k0 + kk;
            const float4 v = *(const float4*)((const float*)op.p0 + o);
            a[q][0] = v.x; a[q][1] = v.y; a[q][2] = v.z; a[q][3] = v.w;
            if constexpr (ADD == A6_F32) {
                const float4 w = *(const float4*)((const float*)op.p1 + o);
                b[q][0] = w.x; b[q][1] = w.y; b[q][2] = w.z; b[q][3] = w.w;
            } else if constexpr (ADD == A6_BF16) {
                const uint2 w = *(const uint2*)((const uint16_t*)op.p1 + o);
                b[q][0] = (uint16_t)w.x; b[q][1] = (uint16_t)(w.x >> 16);
                b[q][2] = (uint16_t)w.y; b[q][3] = (uint16_t)(w.y >> 16);
            }
        }
    }
    static __device__ __forceinline__ bool interior(const Op6& op, int x0, int k0) {
        return op.vec && x0 + BX <= op.xext && k0 + kSplitK <= op.kext;
    }
    __device__ __forceinline__ void load(const Op6& op, int x0, int k0, int t) {
        const int xr = t >> 3, kk = 4 * (t & 7);
        if (interior(op, x0, k0)) { load_fast(op, x0, k0, t); return; }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int x = x0 + xr + RP * q, k = k0 + kk;
            const int64_t o = (int64_t)(x < op.xext ? x : 0) * op.ld + k;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool in = x < op.xext && k + e < op.kext;
                a[q][e] = in ? ((const float*)op.p0)[o + e] : 0.f;
                if constexpr (ADD != A6_NONE) b[q][e] = in ? ((const AT*)op.p1)[o + e] : AT(0);
            }
        }
    }
    __device__ __forceinline__ void split() {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ADD == A6_NONE) v[e] = a[q][e];
                else v[e] = sum6<ADD>(a[q][e], b[q][e]);
            }
            sp[q] = split4(v);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int t) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) store4<3>(lds, BX * kSplitK, (t >> 3) + RP * q, 4 * (t & 7), sp[q]);
    }
    // split and store group by group (no register copy of the whole split slab)
    template <int NP = 3>
    __device__ __forceinline__ void split_store(uint16_t* lds, int t) const {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ADD == A6_NONE) v[e] = a[q][e];
                else v[e] = sum6<ADD>(a[q][e], b[q][e]);
            }
            store4<NP>(lds, BX * kSplitK, (t >> 3) + RP * q, 4 * (t & 7), split4(v));
        }
    }
};

// x-contiguous fp32 (+ addend): each thread owns XW consecutive x (4 with 256 staging threads,
// 2 with 512) and four consecutive k of the 128 x 32 tile, read as one XW-wide vector per k row
// (half that for a bf16 addend) when the rows allow it (op.vec: ld, x0 and the bases
// 4-element aligned); the split then writes each x's four k as one 8-byte chunk per part.
template <int BX, int ADD, int NT>
struct Loader6<BX, S6_XC4, ADD, NT> {
    static constexpr int XW = BX * kSplitK / (4 * NT), TX = BX / XW;   // x per thread, threads per k group
    static_assert(BX == 128 && (XW == 4 || XW == 2), "128 x 32 tile over 256 or 512 threads");
    using AT = typename Add6T<ADD>::t;
    float a[4 * XW];                      // [k][x]: a[XW k + x]
    AT b[ADD == A6_NONE ? 1 : 4 * XW];
    static __device__ __forceinline__ bool interior(const Op6& op, int x0, int k0) {
        return op.vec && x0 + BX <= op.xext && k0 + kSplitK <= op.kext;
    }
    // interior tile with vector-legal rows: no bounds tests
    __device__ __forceinline__ void load_fast(const Op6& op, int x0, int k0, int t) {
        const int64_t o = (int64_t)(k0 + 4 * (t / TX)) * op.ld + x0 + XW * (t % TX);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float* pa = (const float*)op.p0 + o + e * op.ld;
            if constexpr (XW == 4) {
                const float4 v = *(const float4*)pa;
                a[4 * e + 0] = v.x; a[4 * e + 1] = v.y; a[4 * e + 2] = v.z; a[4 * e + 3] = v.w;
            } else {
                const float2 v = *(const float2*)pa;
                a[2 * e + 0] = v.x; a[2 * e + 1] = v.y;
            }
            if constexpr (ADD == A6_F32) {
                const float* pb = (const float*)op.p1 + o + e * op.ld;
                if constexpr (XW == 4) {
                    const float4 w = *(const float4*)pb;
                    b[4 * e + 0] = w.x; b[4 * e + 1] = w.y; b[4 * e + 2] = w.z; b[4 * e + 3] = w.w;
                } else {
                    const float2 w = *(const float2*)pb;
                    b[2 * e + 0] = w.x; b[2 * e + 1] = w.y;
                }
            } else if constexpr (ADD == A6_BF16) {
                const uint16_t* pb = (const uint16_t*)op.p1 + o + e * op.ld;
                if constexpr (XW == 4) {
                    const uint2 w = *(const uint2*)pb;
                    b[4 * e + 0] = (uint16_t)w.x; b[4 * e + 1] = (uint16_t)(w.x >> 16);
                    b[4 * e + 2] = (uint16_t)w.y; b[4 * e + 3] = (uint16_t)(w.y >> 16);
                } else {
                    const uint32_t w = *(const uint32_t*)pb;
                    b[2 * e + 0] = (uint16_t)w; b[2 * e + 1] = (uint16_t)(w >> 16);
                }
            }
        }
    }
    __device__ __forceinline__ void load(const Op6& op, int x0, int k0, int t) {
        if (interior(op, x0, k0)) { load_fast(op, x0, k0, t); return; }
        // element loads from clamped addresses (element 0 is always valid), values selected
        const int x = x0 + XW * (t % TX), k = k0 + 4 * (t / TX);
#pragma unroll
        for (int q = 0; q < 4 * XW; ++q) {
            const int e = q / XW, i = q % XW;
            const bool in = x + i < op.xext && k + e < op.kext;
            const int64_t o = in ? (int64_t)(k + e) * op.ld + x + i : 0;
            const float va = ((const float*)op.p0)[o];
            a[XW * e + i] = in ? va : 0.f;
            if constexpr (ADD != A6_NONE) {
                const AT vb = ((const AT*)op.p1)[o];
                b[XW * e + i] = in ? vb : AT(0);
            }
        }
    }
    template <int NP = 3>
    __device__ __forceinline__ void split_store(uint16_t* lds, int t) const {
        const int xl = XW * (t % TX), kl = 4 * (t / TX);
#pragma unroll
        for (int i = 0; i < XW; ++i) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (ADD == A6_NONE) v[e] = a[XW * e + i];
                else v[e] = sum6<ADD>(a[XW * e + i], b[XW * e + i]);
            }
            store4<NP>(lds, BX * kSplitK, xl + i, kl, split4(v));
        }
    }
};

// acc[i][j] (wave sub-tile FM x FN blocks of 16 x 16) += A B over one 32-k slab from the part
// tiles: B fragments of all three parts held, A fragments one part at a time, the six kept
// products in increasing size.
// NP = 1: the single product of the h parts.
template <int BXA, int BXB, int FM, int FN, int NP = 3>
__device__ __forceinline__ void mma6_slab(const uint16_t* lA, const uint16_t* lB, f32x4 (&acc)[FM][FN], int ra,
                                          int rb, int fr, int fc) {
    u32x4 b[FN][NP];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int p = 0; p < NP; ++p)
            b[j][p] = *(const u32x4*)&lB[p * BXB * kSplitK + part_off(rb + 16 * j + fr, fc)];
    if constexpr (NP == 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const u32x4 a = *(const u32x4*)&lA[part_off(ra + 16 * i + fr, fc)];
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mma_bf16(a, b[j][0], acc[i][j]);
        }
        return;
    }
#pragma unroll
    for (int pa = NP - 1; pa >= 0; --pa) {
        u32x4 a[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = *(const u32x4*)&lA[pa * BXA * kSplitK + part_off(ra + 16 * i + fr, fc)];
#pragma unroll
        for (int pb = (NP - 1) - pa; pb >= 0; --pb)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mma_bf16(a[i], b[j][pb], acc[i][j]);
    }
}

// Two products sharing A (acc1 += A B1, acc2 += A B2) over one slab: A fragments of all three
// parts are read once, then per column block the B1 and B2 fragments of all three parts; the six
// kept products of each pair in the same increasing order as mma6_slab.
template <int BXA, int BXB, int FM, int FN, int NP = 3>
__device__ __forceinline__ void mma6_slab2(const uint16_t* lA, const uint16_t* lB1, const uint16_t* lB2,
                                           f32x4 (&acc1)[FM][FN], f32x4 (&acc2)[FM][FN], int ra, int rb, int fr,
                                           int fc) {
    u32x4 a[NP][FM];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < FM; ++i) a[p][i] = *(const u32x4*)&lA[p * BXA * kSplitK + part_off(ra + 16 * i + fr, fc)];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        u32x4 b1[NP], b2[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            b1[p] = *(const u32x4*)&lB1[p * BXB * kSplitK + part_off(rb + 16 * j + fr, fc)];
            b2[p] = *(const u32x4*)&lB2[p * BXB * kSplitK + part_off(rb + 16 * j + fr, fc)];
        }
#pragma unroll
        for (int pa = NP - 1; pa >= 0; --pa)
#pragma unroll
            for (int pb = (NP - 1) - pa; pb >= 0; --pb)
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    acc1[i][j] = mma_bf16(a[pa][i], b1[pb], acc1[i][j]);
                    acc2[i][j] = mma_bf16(a[pa][i], b2[pb], acc2[i][j]);
                }
    }
}

}  // namespace dion
