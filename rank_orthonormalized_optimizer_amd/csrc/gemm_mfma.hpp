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
// Operands are staged through LDS in their memory order: k-contiguous operands as
// [x][k] tiles, x-contiguous ones as [k][x] tiles (x = row of A or column of B),
// so every staging store is a contiguous 4-element vector.  Within a slab of BK,
// lane group g = lane / 16 of the MFMA feeds k = (BK / 4) g + s at step s, so a
// fragment of an [x][k] tile is BK / 4 consecutive k: two 16-byte LDS reads.
// Global loads are 4-element vectors along whichever index is contiguous in
// memory, prefetched into registers ahead of the MFMA work.
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

// Round-to-nearest-even float -> bfloat16 bits, by the hardware conversion (v_cvt_pk_bf16_f32;
// a NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two values rounded to bfloat16 and packed, a in the low half: one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Storage of an operand source: the raw element types read from p0 and p1.
template <int SRC> struct SrcStorage;
template <> struct SrcStorage<SRC_F32> { using S0 = float; using S1 = float; static constexpr bool two = false; };
template <> struct SrcStorage<SRC_F64> { using S0 = double; using S1 = double; static constexpr bool two = false; };
template <> struct SrcStorage<SRC_BF16> { using S0 = uint16_t; using S1 = uint16_t; static constexpr bool two = false; };
template <> struct SrcStorage<SRC_SUM_F32> { using S0 = float; using S1 = float; static constexpr bool two = true; };
template <> struct SrcStorage<SRC_SUM_BF16> { using S0 = float; using S1 = uint16_t; static constexpr bool two = true; };

template <typename T, typename S> __device__ __forceinline__ T widen(S v) { return (T)v; }
template <> __device__ __forceinline__ float widen<float, uint16_t>(uint16_t v) { return bf16_bits_to_float(v); }
template <> __device__ __forceinline__ double widen<double, uint16_t>(uint16_t v) {
    return (double)bf16_bits_to_float(v);
}

// Four consecutive raw elements; requires 4-element alignment of `off` and of the base.
template <typename S>
__device__ __forceinline__ void load4_raw(const void* p, int64_t off, S (&o)[4]) {
    if constexpr (sizeof(S) == 4) {
        const float4 v = *(const float4*)((const S*)p + off);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else if constexpr (sizeof(S) == 8) {
        const double2 a = *(const double2*)((const S*)p + off);
        const double2 b = *(const double2*)((const S*)p + off + 2);
        o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y;
    } else {
        const uint2 v = *(const uint2*)((const S*)p + off);
        o[0] = (S)(v.x & 0xffffu); o[1] = (S)(v.x >> 16); o[2] = (S)(v.y & 0xffffu); o[3] = (S)(v.y >> 16);
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

// Tile numbering that keeps neighbouring tiles on one XCD.  The dispatcher hands workgroups
// to the 8 XCDs round-robin by linear id, and each XCD has its own L2, so the tiles that share
// an operand panel (the column tiles of one row panel, all tiles of one matrix) would otherwise
// be spread over all eight L2s and fetch the panel eight times.  The linear id L (x fastest)
// is renumbered so that XCD x processes the contiguous range of tile ids of its share, in
// order; a bijection on [0, T) for any T.  Within a matrix, tile ids then run down bands of
// kTileBand rows, column by column, so the tiles resident on an XCD at one time (about 64)
// form a block about 8 x 8 whose row and column operand panels together fit in its L2.
constexpr int kTileBand = 8;
struct TileId { int x, y, z; };
__device__ __forceinline__ TileId xcd_tile_id() {
    constexpr int64_t NX = 8;
    const int64_t gx = gridDim.x, gy = gridDim.y;
    const int64_t T = gx * gy * (int64_t)gridDim.z;
    const int64_t L = blockIdx.x + gx * (blockIdx.y + gy * (int64_t)blockIdx.z);
    const int64_t q = T / NX, rem = T % NX, x = L % NX, slot = L / NX;
    const int64_t t = (x < rem) ? x * (q + 1) + slot : rem * (q + 1) + (x - rem) * q + slot;
    const int64_t per = gx * gy, z = t / per, w = t % per;
    const int64_t band = w / (kTileBand * gx), y0 = band * kTileBand;
    const int64_t rows = gy - y0 < kTileBand ? gy - y0 : kTileBand;
    const int64_t u = w - band * kTileBand * gx;     // position inside the band
    return TileId{(int)(u / rows), (int)(y0 + u % rows), (int)z};
}

// Register-staged loader of one BX x BK operand tile.  load() only issues the global
// loads of the raw storage values; store() widens them to T (adding the two addends of
// the SUM sources, exactly in double and with one rounding in float) and writes LDS.  So the
// loads stay in flight across the MFMAs placed between the two calls.
template <typename T, int BX, int BK, bool KC, int SRC>
struct TileLoader {
    using St = SrcStorage<SRC>;
    using S0 = typename St::S0;
    using S1 = typename St::S1;
    static constexpr int GROUPS = BX * BK / 4;
    static_assert(GROUPS % 256 == 0, "tile must give every thread whole 4-element groups");
    static_assert(!KC || BK % 4 == 0, "KC tiles are stored four k at a time");
    static constexpr int PER = GROUPS / 256;
    S0 r0[PER][4];
    S1 r1[St::two ? PER : 1][4];

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
                load4_raw<S0>(op.p0, off, r0[g]);
                if constexpr (St::two) load4_raw<S1>(op.p1, off, r1[g]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int xx = KC ? x : x + v;
                    const int kk = KC ? k + v : k;
                    const bool in = xx < op.xext && kk < op.kext;
                    r0[g][v] = in ? ((const S0*)op.p0)[off + v] : S0(0);
                    if constexpr (St::two) r1[g][v] = in ? ((const S1*)op.p1)[off + v] : S1(0);
                }
            }
        }
    }
    // Interior tiles with vector-legal operands: the same vector loads, with no bounds tests.
    // Branch-free, so the compiler can count the loads in flight and wait for exactly the
    // ones a store needs (the bounds-tested loader's paths force it to wait for all of them).
    __device__ __forceinline__ void load_fast(const Operand& op, int x0, int k0) {
#pragma unroll
        for (int g = 0; g < PER; ++g) {
            const int idx = threadIdx.x + g * 256;
            int x, k;
            if constexpr (KC) { x = x0 + idx / (BK / 4); k = k0 + (idx % (BK / 4)) * 4; }
            else { k = k0 + idx / (BX / 4); x = x0 + (idx % (BX / 4)) * 4; }
            const int64_t off = KC ? (int64_t)x * op.ld + k : (int64_t)k * op.ld + x;
            load4_raw<S0>(op.p0, off, r0[g]);
            if constexpr (St::two) load4_raw<S1>(op.p1, off, r1[g]);
        }
    }
    __device__ __forceinline__ T value(int g, int v) const {
        if constexpr (St::two) return widen<T, S0>(r0[g][v]) + widen<T, S1>(r1[g][v]);
        else return widen<T, S0>(r0[g][v]);
    }
    // LDS tile layout: s[x * LD + k] for KC operands, s[k * LD + x] otherwise (LD the pitch)
    template <int LD>
    __device__ __forceinline__ void store(T* s) const {
#pragma unroll
        for (int g = 0; g < PER; ++g) {
            const int idx = threadIdx.x + g * 256;
            if constexpr (KC) {
                const int x = idx / (BK / 4), k = (idx % (BK / 4)) * 4;
#pragma unroll
                for (int v = 0; v < 4; ++v) s[x * LD + k + v] = value(g, v);
            } else {
                const int k = idx / (BX / 4), x = (idx % (BX / 4)) * 4;
#pragma unroll
                for (int v = 0; v < 4; ++v) s[k * LD + x + v] = value(g, v);
            }
        }
    }
};

// Tile geometry shared by the kernels: BM x BN output tile, K slabs of BK, LDS tiles [k][x]
// padded by PAD elements per k-row or [x][k] padded by 16 bytes per x-row (which spreads the
// rows of a fragment read over the banks), two LDS stages (double buffering).
template <typename T, int BM_, int BN_, int BK_ = 16>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, PAD = 16;
    static constexpr int LDA = BM + PAD, LDB = BN + PAD;     // [k][x] pitches
    static constexpr int LDK = BK + 16 / (int)sizeof(T);     // [x][k] pitch
    static constexpr int WTM = BM / 2, WTN = BN / 2;   // wave sub-tile
    static constexpr int FM = WTM / 16, FN = WTN / 16; // MFMA blocks per wave
    static constexpr int KS = BK / 4;                  // MFMA steps per slab
    static constexpr int A_STAGE = BK * LDA > BM * LDK ? BK * LDA : BM * LDK;
    static constexpr int B_STAGE = BK * LDB > BN * LDK ? BK * LDB : BN * LDK;
    using acc_t = typename Mfma<T>::acc_t;
};

// The KS values of one fragment at row x of a tile: k = KS g + s, s = 0 .. KS - 1.
template <typename T, class C, bool KC, int LDX>
__device__ __forceinline__ void frag_k(const T* s, int x, int g, T (&v)[C::KS]) {
    if constexpr (KC) {
        typedef T t4 __attribute__((ext_vector_type(16 / sizeof(T))));
        constexpr int W = 16 / sizeof(T);
        const T* p = s + x * C::LDK + C::KS * g;
#pragma unroll
        for (int q = 0; q < C::KS / W; ++q) {
            const t4 u = *(const t4*)(p + W * q);
#pragma unroll
            for (int e = 0; e < W; ++e) v[W * q + e] = u[e];
        }
    } else {
#pragma unroll
        for (int q = 0; q < C::KS; ++q) v[q] = s[(C::KS * g + q) * LDX + x];
    }
}

// acc[i][j] += A_frag[i] * B_frag[j] over one BK slab of LDS.
template <typename T, class C, bool AKC, bool BKC>
__device__ __forceinline__ void mma_slab(const T* As, const T* Bs, typename C::acc_t (&acc)[C::FM][C::FN],
                                         int wm, int wn, int lane) {
    const int lr = lane & 15, lk = lane >> 4;
    T a[C::FM][C::KS], b[C::FN][C::KS];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) frag_k<T, C, AKC, C::LDA>(As, wm * C::WTM + i * 16 + lr, lk, a[i]);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) frag_k<T, C, BKC, C::LDB>(Bs, wn * C::WTN + j * 16 + lr, lk, b[j]);
#pragma unroll
    for (int q = 0; q < C::KS; ++q)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) acc[i][j] = Mfma<T>::mma(a[i][q], b[j][q], acc[i][j]);
}

// fp64 main loop of an interior tile whose K range is whole slabs: slab s in LDS buffer s % 2,
// register set s % 2 loaded two slabs ahead, and a steady loop with no conditional loads.
template <typename T, class C, bool AKC, int ASRC, bool BKC, int BSRC>
__device__ __forceinline__ void mainloop_fast2(const Operand& A, const Operand& B, int m0, int n0, int kbeg,
                                               int nslab, T* As, T* Bs, typename C::acc_t (&acc)[C::FM][C::FN]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    T* A0 = As;
    T* A1 = As + C::A_STAGE;
    T* B0 = Bs;
    T* B1 = Bs + C::B_STAGE;
    constexpr int LA = AKC ? C::LDK : C::LDA, LB = BKC ? C::LDK : C::LDB;
    TileLoader<T, C::BM, C::BK, AKC, ASRC> la0, la1;
    TileLoader<T, C::BN, C::BK, BKC, BSRC> lb0, lb1;
    la0.load_fast(A, m0, kbeg);
    lb0.load_fast(B, n0, kbeg);
    if (nslab > 1) { la1.load_fast(A, m0, kbeg + C::BK); lb1.load_fast(B, n0, kbeg + C::BK); }
    la0.template store<LA>(A0);
    lb0.template store<LB>(B0);
    __syncthreads();
    // invariant: LDS buffer 0 holds slab s, register set 1 slab s + 1
    int s = 0;
    for (; s + 3 < nslab; s += 2) {
        const int k2 = kbeg + (s + 2) * C::BK;
        la0.load_fast(A, m0, k2);
        lb0.load_fast(B, n0, k2);
        mma_slab<T, C, AKC, BKC>(A0, B0, acc, wm, wn, lane);
        la1.template store<LA>(A1);
        lb1.template store<LB>(B1);
        __syncthreads();
        la1.load_fast(A, m0, k2 + C::BK);
        lb1.load_fast(B, n0, k2 + C::BK);
        mma_slab<T, C, AKC, BKC>(A1, B1, acc, wm, wn, lane);
        la0.template store<LA>(A0);
        lb0.template store<LB>(B0);
        __syncthreads();
    }
    const int r = nslab - s;   // 1, 2 or 3 slabs left
    if (r == 3) { la0.load_fast(A, m0, kbeg + (s + 2) * C::BK); lb0.load_fast(B, n0, kbeg + (s + 2) * C::BK); }
    mma_slab<T, C, AKC, BKC>(A0, B0, acc, wm, wn, lane);
    if (r >= 2) {
        la1.template store<LA>(A1);
        lb1.template store<LB>(B1);
        __syncthreads();
        mma_slab<T, C, AKC, BKC>(A1, B1, acc, wm, wn, lane);
        if (r == 3) {
            la0.template store<LA>(A0);
            lb0.template store<LB>(B0);
            __syncthreads();
            mma_slab<T, C, AKC, BKC>(A0, B0, acc, wm, wn, lane);
        }
    }
    __syncthreads();
}

// Main loop over the K range [kbeg, kend), slab k in LDS buffer k % 2 (one barrier per slab).
// fp64: two register staging sets, the raw loads of slab k + 2 issued before slab k is
// multiplied, so each has two slabs of MFMA work to arrive.  fp32 (four times the MFMA rate,
// half the bytes) keeps one staging set: the second one costs it a wave of occupancy.
template <typename T, class C, bool AKC, int ASRC, bool BKC, int BSRC>
__device__ __forceinline__ void mainloop(const Operand& A, const Operand& B, int m0, int n0, int kbeg, int kend,
                                         T* As, T* Bs, typename C::acc_t (&acc)[C::FM][C::FN]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    if (kbeg >= kend) return;
    T* A0 = As;
    T* A1 = As + C::A_STAGE;
    T* B0 = Bs;
    T* B1 = Bs + C::B_STAGE;
    if constexpr (sizeof(T) == 8) {
        if (A.vec && B.vec && m0 + C::BM <= A.xext && n0 + C::BN <= B.xext && kend <= A.kext && kend <= B.kext &&
            (kend - kbeg) % C::BK == 0) {
            mainloop_fast2<T, C, AKC, ASRC, BKC, BSRC>(A, B, m0, n0, kbeg, (kend - kbeg) / C::BK, As, Bs, acc);
            return;
        }
        TileLoader<T, C::BM, C::BK, AKC, ASRC> la0, la1;
        TileLoader<T, C::BN, C::BK, BKC, BSRC> lb0, lb1;
        la0.load(A, m0, kbeg);
        lb0.load(B, n0, kbeg);
        if (kbeg + C::BK < kend) { la1.load(A, m0, kbeg + C::BK); lb1.load(B, n0, kbeg + C::BK); }
        la0.template store<AKC ? C::LDK : C::LDA>(A0);
        lb0.template store<BKC ? C::LDK : C::LDB>(B0);
        __syncthreads();
        for (int k0 = kbeg; k0 < kend; k0 += 2 * C::BK) {
            const int k1 = k0 + C::BK, k2 = k0 + 2 * C::BK, k3 = k0 + 3 * C::BK;
            if (k2 < kend) { la0.load(A, m0, k2); lb0.load(B, n0, k2); }
            mma_slab<T, C, AKC, BKC>(A0, B0, acc, wm, wn, lane);
            if (k1 < kend) {
                la1.template store<AKC ? C::LDK : C::LDA>(A1);
                lb1.template store<BKC ? C::LDK : C::LDB>(B1);
            }
            __syncthreads();
            if (k1 >= kend) break;
            if (k3 < kend) { la1.load(A, m0, k3); lb1.load(B, n0, k3); }
            mma_slab<T, C, AKC, BKC>(A1, B1, acc, wm, wn, lane);
            if (k2 < kend) {
                la0.template store<AKC ? C::LDK : C::LDA>(A0);
                lb0.template store<BKC ? C::LDK : C::LDB>(B0);
            }
            __syncthreads();
        }
    } else {
        TileLoader<T, C::BM, C::BK, AKC, ASRC> la;
        TileLoader<T, C::BN, C::BK, BKC, BSRC> lb;
        la.load(A, m0, kbeg);
        lb.load(B, n0, kbeg);
        la.template store<AKC ? C::LDK : C::LDA>(A0);
        lb.template store<BKC ? C::LDK : C::LDB>(B0);
        __syncthreads();
        int buf = 0;
        for (int k0 = kbeg; k0 < kend; k0 += C::BK) {
            const bool more = k0 + C::BK < kend;
            if (more) { la.load(A, m0, k0 + C::BK); lb.load(B, n0, k0 + C::BK); }
            mma_slab<T, C, AKC, BKC>(buf ? A1 : A0, buf ? B1 : B0, acc, wm, wn, lane);
            if (more) {
                la.template store<AKC ? C::LDK : C::LDA>(buf ? A0 : A1);
                lb.template store<BKC ? C::LDK : C::LDB>(buf ? B0 : B1);
            }
            __syncthreads();
            buf ^= 1;
        }
    }
}

}  // namespace dion
