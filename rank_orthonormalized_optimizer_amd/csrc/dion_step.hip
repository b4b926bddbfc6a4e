// Kernels and launch sequence of the Dion step on gfx950.
//
// Per matrix of the stack (shapes m x n, rank r), the step is
//   B = M + G;  P0 = B Q;  P = orth(P0);  R = B^T P;
//   M <- B - (1 - mu) P R^T;  Q <- R / (||r_j|| + eps);  X <- X - lr sqrt(m/n) P Q^T
// ("Dion e la fine del monopolio di Adam negli optimizer AI distribuiti",
// rivista.ai: low-rank orthonormalized update with error feedback, amortized
// power iteration with QR and Cholesky).
//
// orth() is CholeskyQR2: W = P0^T P0, L = chol(W), P1 = P0 L^-T, repeated once
// (the second pass by the near-identity series when P1^T P1 is close to I).
// In exact arithmetic it gives the same Q-factor (positive diagonal) as a
// Householder QR.  Two precision chains share the kernels:
//   fp32 chain  B rounded once to fp32, fp32 MFMA everywhere.  If a Cholesky
//               pivot fails or the diagonal ratio max(L_ii)/min(L_ii) of the
//               first pass exceeds kTau32, the matrix is handed to
//   fp64 chain  B = M + G exact in fp64, P0, the QR and R in fp64 MFMA.  If its
//               first Cholesky fails or its diagonal ratio exceeds kTau64, the
//               first pass is redone on W + s I (shifted CholeskyQR, Fukaya,
//               Kannan, Nakatsukasa, Yamamoto and Yanagisawa, SIAM J. Sci.
//               Comput. 2020) followed by two plain passes.
// The hand-over is a per-matrix state word in device memory: every kernel of a
// chain tests it and returns at once for matrices it does not own, so the host
// never synchronizes.  The momentum/weight pass then runs once for all
// matrices from P, R and the new Q rounded to fp32, with its two rank-r
// products on the bf16 matrix cores in the exact three-way split form
// (fp32 accuracy; see bf16x6.hpp).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "dion.h"
#include "dion_plan.h"
#include "gemm_mfma.hpp"
#include "bf16x6.hpp"

namespace dion {

// Diagonal-ratio thresholds of the first Cholesky pass (see the header comment).
constexpr double kTau32 = 64.0;
constexpr double kTau64 = 1.0e7;
// Re-orthonormalization passes, by eps = ||P^T P - I||_F.  fp32: F = Phi(E), S = F up to
// eps = 1e-4 (error ~ eps^2 <= 1e-8, below fp32 rounding).  fp64: the same first-order form up to
// eps = 3e-7 (error ~ eps^2 <= 1e-13); up to 1e-3 two fixed-point steps (error eps^2 (2 eps)^2
// <= 4e-12) and S up to F^3 (truncation eps^4 <= 1e-12); beyond, the Cholesky pass.
constexpr double kNearId32 = 1.0e-4;
constexpr double kNearId64 = 1.0e-6;
// Diagonal-ratio limit of a re-orthonormalization pass's Cholesky regime.  After a plain first
// pass accepted under kTau32 / kTau64, P1^T P1 is I + O(kappa^2 u) and the ratio stays near 1;
// after the shifted first pass kappa(P1) ~ sqrt(c_shift r) kappa(P0), which reached 5.6e4 on the
// full-rank 4096^2 stack (CPU emulation of its first step) and a few 1e4 on 8-decade spectra.
// A P0 that is singular to working precision (duplicate or zero columns) leaves P1 singular too,
// and its Cholesky then either fails or shows a ratio near u^-1/2 (1e8 in fp64): above the limit
// the pass counts as broken down, and the matrix goes on to the next fallback (fp32: the fp64
// chain; fp64: the Householder QR).
constexpr double kTauRe32 = 1.0e3;
constexpr double kTauRe64 = 1.0e6;

// ---------------------------------------------------------------------------
// generic batched GEMM:  C = alpha * A B + beta * C
// ---------------------------------------------------------------------------
struct GemmArgs {
    Operand a, b;              // per-matrix views (batch 0)
    int64_t sa0, sa1, sb0;     // batch strides in bytes of a.p0, a.p1, b.p0
    void* c;
    int64_t ldc, sc;           // ldc in elements, sc in bytes
    int M, N, K;
    double alpha, beta;
    const int* st;             // per-matrix state word; matrix runs iff (st & mask) == val
    int st_mask, st_val;
    int lower;                 // skip tiles strictly above the diagonal
    int zdiv;                  // tile z index = matrix * zdiv + group (0 or 1: no groups)
    int64_t ga0, gb0, gc;      // byte offsets between groups for a.p0, b.p0, c
    int kskip;                 // K range of a tile: 0 all; 1 k < n0 + BN (B = lower^T);
                               // 2 k >= n0 (B lower); 3 k < m0 + BM (A lower); 4 both 2 and 3
    int ksplit_total;          // > 0: group g covers K rows [g K, min((g + 1) K, ksplit_total)) of
                               // the operands (their base advanced by ga0 / gb0 per group)
    const void* csrc;          // beta term read from here instead of c (same layout), if set
};

// fp64 tiles are held to 128 registers a lane so that four workgroups share a CU (their LDS
// is 40 KB each): the fp64 MFMA has a long issue time, and more resident waves keep it fed
// across the per-slab barriers.
// One output tile (tx, ty) of matrix bz (group grp) of a batched GEMM; the workgroup synchronizes
// before returning only through mainloop's barriers, so a caller that reuses As / Bs for another
// tile must synchronize first.
template <typename T, int BM, int BN, int BK, bool AKC, int ASRC, bool BKC, int BSRC>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int bz, int grp, int tx, int ty, T* As, T* Bs) {
    using C = TileCfg<T, BM, BN, BK>;
    const int m0 = ty * BM, n0 = tx * BN;
    if (g.lower && n0 >= m0 + BM) return;
    int kbeg = 0, kend = g.K;
    if (g.kskip == 1) kend = min(g.K, n0 + BN);
    else if (g.kskip == 2) kbeg = (n0 / C::BK) * C::BK;
    else if (g.kskip == 3) kend = min(g.K, m0 + BM);
    else if (g.kskip == 4) { kbeg = (n0 / C::BK) * C::BK; kend = min(g.K, m0 + BM); }
    int kext = 0;
    if (g.ksplit_total > 0) {
        kext = min(g.K, g.ksplit_total - grp * g.K);
        kend = min(kend, kext);
    }

    Operand A = g.a, B = g.b;
    A.p0 = (const char*)A.p0 + bz * g.sa0 + grp * g.ga0;
    if (A.p1) A.p1 = (const char*)A.p1 + bz * g.sa1;
    B.p0 = (const char*)B.p0 + bz * g.sb0 + grp * g.gb0;
    if (g.ksplit_total > 0) { A.kext = kext; B.kext = kext; }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    typename C::acc_t acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::acc_t{0, 0, 0, 0};

    mainloop<T, C, AKC, ASRC, BKC, BSRC>(A, B, m0, n0, kbeg, kend, As, Bs, acc);

    T* Cp = (T*)((char*)g.c + bz * g.sc + grp * g.gc);
    const T* Sp = g.csrc ? (const T*)((const char*)g.csrc + bz * g.sc + grp * g.gc) : Cp;
    const T alpha = (T)g.alpha, beta = (T)g.beta;
    const bool need_src = beta != T(0);
    // all source loads of the tile before the first store (see the update kernel's epilogue)
    T sv[C::FM][C::FN][4];
    if (need_src) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = m0 + wm * C::WTM + i * 16 + Mfma<T>::row(lane, v);
                    const int col = n0 + wn * C::WTN + j * 16 + (lane & 15);
                    sv[i][j][v] = (row < g.M && col < g.N) ? Sp[(int64_t)row * g.ldc + col] : T(0);
                }
    }
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * C::WTM + i * 16 + Mfma<T>::row(lane, v);
                const int col = n0 + wn * C::WTN + j * 16 + (lane & 15);
                if (row < g.M && col < g.N) {
                    T val = alpha * acc[i][j][v];
                    if (need_src) val += beta * sv[i][j][v];
                    Cp[(int64_t)row * g.ldc + col] = val;
                }
            }
}

template <typename T, int BM, int BN, int BK, bool AKC, int ASRC, bool BKC, int BSRC>
__global__ __launch_bounds__(256, sizeof(T) == 8 ? 4 : 1) void gemm_kernel(GemmArgs g) {
    using C = TileCfg<T, BM, BN, BK>;
    const int zdiv = g.zdiv > 1 ? g.zdiv : 1;
    const TileId tid = xcd_tile_id();
    const int bz = tid.z / zdiv, grp = tid.z % zdiv;
    if (g.st && (g.st[bz] & g.st_mask) != g.st_val) return;
    // triangular K ranges: the longest tiles get the lowest dispatch order, so the launch does
    // not end on them
    const int tx = g.kskip == 1 ? (int)gridDim.x - 1 - tid.x : tid.x;
    const int ty = g.kskip == 3 ? (int)gridDim.y - 1 - tid.y : tid.y;
    __shared__ T As[2 * C::A_STAGE];
    __shared__ T Bs[2 * C::B_STAGE];
    gemm_tile<T, BM, BN, BK, AKC, ASRC, BKC, BSRC>(g, bz, grp, tx, ty, As, Bs);
}

// The same GEMM with a fixed number of workgroups per matrix (grid: workgroups x 1 x matrices),
// each looping over tiles, for the rarely taken paths: a launch that finds no matrix to work on
// then costs as little as a small grid, while a selected matrix still spreads over many CUs.
template <typename T, int BM, int BN, int BK, bool AKC, int ASRC, bool BKC, int BSRC>
__global__ __launch_bounds__(256, sizeof(T) == 8 ? 4 : 1) void gemm_stride_kernel(GemmArgs g) {
    using C = TileCfg<T, BM, BN, BK>;
    const int bz = blockIdx.z;
    if (g.st && (g.st[bz] & g.st_mask) != g.st_val) return;
    __shared__ T As[2 * C::A_STAGE];
    __shared__ T Bs[2 * C::B_STAGE];
    const int64_t tiles_x = (g.N + BN - 1) / BN, tiles = tiles_x * ((g.M + BM - 1) / BM);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        gemm_tile<T, BM, BN, BK, AKC, ASRC, BKC, BSRC>(g, bz, 0, (int)(t % tiles_x), (int)(t / tiles_x), As, Bs);
        __syncthreads();   // As / Bs are rewritten by the next tile
    }
}

template <typename T, int BM, int BN, int BK, bool AKC, int ASRC, bool BKC, int BSRC>
static hipError_t launch_gemm_tile(const GemmArgs& g, int64_t batch, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
    const int64_t zdiv = g.zdiv > 1 ? g.zdiv : 1;
    dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, (unsigned)(batch * zdiv));
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, AKC, ASRC, BKC, BSRC>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

constexpr int kRareGemmBlocks = 128;   // workgroups per matrix of a rare-path GEMM

template <typename T, bool AKC, int ASRC, bool BKC, int BSRC>
static hipError_t launch_gemm_rare(const GemmArgs& g, int64_t batch, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
    constexpr int BM = 64, BN = 64, BK = sizeof(T) == 8 ? 16 : 32;
    const int64_t tiles = ((g.N + BN - 1) / BN) * ((g.M + BM - 1) / BM);
    dim3 grid((unsigned)(tiles < kRareGemmBlocks ? tiles : kRareGemmBlocks), 1, (unsigned)batch);
    hipLaunchKernelGGL((gemm_stride_kernel<T, BM, BN, BK, AKC, ASRC, BKC, BSRC>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

// Tile choice.  The large tile is used when the grid still has at least kBigTileMinTiles
// tiles; otherwise (and for in-place column-panel updates, which need N <= 64) 64 x 64.
#ifndef DION_F64_BM
#define DION_F64_BM 64
#endif
#ifndef DION_F64_BN
#define DION_F64_BN 64
#endif
#ifndef DION_F64_BK
#define DION_F64_BK 16
#endif
#ifndef DION_F32_BM
#define DION_F32_BM 64
#endif
#ifndef DION_F32_BN
#define DION_F32_BN 64
#endif
#ifndef DION_F32_BK
#define DION_F32_BK 32
#endif
#ifndef DION_BIG_MIN_TILES
#define DION_BIG_MIN_TILES 256
#endif
constexpr int kBigTileMinTiles = DION_BIG_MIN_TILES;
#ifndef DION_PROD6
#define DION_PROD6 1
#endif
#ifndef DION_UPD_BIG_MIN_TILES
#define DION_UPD_BIG_MIN_TILES 256
#endif
constexpr int kUpdBigMinTiles = DION_UPD_BIG_MIN_TILES;

template <typename T, int BM, int BN, bool AKC, int ASRC, bool BKC, int BSRC>
static hipError_t launch_gemm(const GemmArgs& g, int64_t batch, hipStream_t s) {
    constexpr bool d = sizeof(T) == 8;
    constexpr int LBM = d ? DION_F64_BM : DION_F32_BM, LBN = d ? DION_F64_BN : DION_F32_BN;
    constexpr int LBK = d ? DION_F64_BK : DION_F32_BK, SBK = d ? 16 : 32;
    const int64_t zdiv = g.zdiv > 1 ? g.zdiv : 1;
    const int64_t big_tiles = ((g.M + LBM - 1) / LBM) * ((g.N + LBN - 1) / LBN) * batch * zdiv;
    if constexpr (LBM != 64 || LBN != 64 || LBK != SBK) {
        if (BM == 64 && BN == 64 && g.M >= LBM && g.N >= LBN && big_tiles >= kBigTileMinTiles)
            return launch_gemm_tile<T, LBM, LBN, LBK, AKC, ASRC, BKC, BSRC>(g, batch, s);
    }
    return launch_gemm_tile<T, 64, 64, SBK, AKC, ASRC, BKC, BSRC>(g, batch, s);
}

// ---------------------------------------------------------------------------
// diagonal block of the blocked Cholesky: factor, track the diagonal ratio,
// and invert the factor (both kept in LDS)
// ---------------------------------------------------------------------------
struct PotrfArgs {
    void* L; int64_t ldl, sL;   // factor (elements); the block is read from S (same layout), which may be L
    const void* S;
    void* Td; int64_t sTd;      // inverses of the diagonal blocks: block jblk at Td + jblk * blkTd, pitch ldTd
    int64_t ldTd, blkTd;
    int tdfull;                 // write the whole kNB x kNB block (zeros outside nbj x nbj), else nbj x nbj only
    int j0, nbj, jblk;
    int* st; int st_mask, st_val;
    double* kap;                // [batch][2] running min / max of diag(L)
    int first, last;
    double tau;                 // diagonal-ratio limit tested on the last block (<= 0: off)
    int fail_bit, tau_bit;
};

// The 64 x 64 diagonal block is factored in LDS by 16-column panels.  Per panel one wave sweeps
// the panel's columns (one row of the panel per lane, its 16 values in registers): the pivot
// and the next pivot travel by v_readlane, the scaled column by LDS, and a bad pivot is only
// recorded (checked after the sweep), so the sweep is one straight-line block in which the next
// pivot's reciprocal square root overlaps the current column's broadcast.  The trailing blocks
// are updated with 16 x 16 MFMA blocks spread over the four waves.  The inverse X = L^-1 then
// comes from the four 16 x 16 diagonal inverses (forward substitution, one wave each) and two
// levels of recursive doubling, X_VU = -X_VV (L_VU X_UU), again as MFMA blocks.
constexpr int kSB = 16, kDLD = kNB + 1;   // panel width; LDS pitch of the block

template <typename T>
struct DiagSmem {
    T a[kNB * kDLD];     // working block, then L (lower); its upper blocks park the doubling products
    T x[kNB * kDLD];     // L^-1 (lower)
    T col[2][64];        // column broadcast of the panel sweep
    T dg[kNB];           // diag(L)
    T rd[kNB];           // 1 / diag(L)
    int fail;
};

template <typename T>
__device__ __forceinline__ T read_lane(T v, int l) {
    if constexpr (sizeof(T) == 8) {
        const long long u = __double_as_longlong(v);
        const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffff), l);
        const int hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
        return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
    } else {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
    }
}

// 1 / sqrt(d): the hardware estimate and Newton steps y <- y (3/2 - d y^2 / 2), two in fp64
// (each doubles the correct bits of the estimate), one in fp32.
template <typename T>
__device__ __forceinline__ T rsqrt_newton(T d) {
    if constexpr (sizeof(T) == 8) {
        double y = __builtin_amdgcn_rsq(d);
        const double h = 0.5 * d;
        double t = y * y; t = __builtin_fma(-h, t, 1.5); y = y * t;
        t = y * y; t = __builtin_fma(-h, t, 1.5); y = y * t;
        return y;
    } else {
        float y = __builtin_amdgcn_rsqf(d);
        const float h = 0.5f * d;
        const float t = __builtin_fmaf(-h, y * y, 1.5f);
        return y * t;
    }
}

// acc += A B over K (a multiple of 16) for one 16 x 16 block held by the calling wave, with
// A(i,k) = a[i * ai + k * ak] and B(k,j) = b[k * bk + j * bj] in LDS; the operands of four
// k-steps are read before their four products.
template <typename T>
__device__ __forceinline__ void blk_mma(const T* a, int ai, int ak, const T* b, int bk, int bj, int K,
                                        typename Mfma<T>::acc_t& acc, int lane) {
    const int r = lane & 15, kk = lane >> 4;
    for (int k0 = 0; k0 < K; k0 += 16) {
        T av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[u] = a[r * ai + (k0 + 4 * u + kk) * ak];
            bv[u] = b[(k0 + 4 * u + kk) * bk + r * bj];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = Mfma<T>::mma(av[u], bv[u], acc);
    }
}

// Sweep of panel p by one wave: columns 16 p .. 16 p + 15, rows 16 p .. 63 (lane = row of the
// panel, its 16 values in registers).  False on a bad pivot.  Column K scales its column by the
// pivot's reciprocal square root and subtracts l_iK l_jK from the later columns j.  The pivot
// chain never waits for LDS: each lane also keeps its own diagonal element a_ll in a register
// (the same updates, l_lK^2, in the same order), so the next pivot is one v_readlane of it; the
// two following columns take this column's multipliers l_jK by v_readlane as well, and only the
// columns from K + 3 on take them from an LDS broadcast, whose reads are consumed one column
// later, behind the next pivot's reciprocal square root.  Every element receives the same fused
// multiply-adds in the same order as in a plain column-by-column sweep.
template <typename T>
__device__ bool panel_sweep(DiagSmem<T>& sm, int p, int lane) {
    const int o = kSB * p, R = o + lane;
    const bool valid = R < kNB;
    T a[kSB], dgv[kSB], rdv[kSB], pc[kSB];
#pragma unroll
    for (int j = 0; j < kSB; ++j) {
        a[j] = valid ? sm.a[R * kDLD + o + j] : T(0);
        pc[j] = T(0);
    }
    T dg = T(0);   // a_ll of this lane's row l = lane (lanes < 16)
#pragma unroll
    for (int j = 0; j < kSB; ++j) dg = (lane == j) ? a[j] : dg;
    T d = read_lane<T>(dg, 0), r = rsqrt_newton<T>(d), pl = T(0);
    bool bad = false;
#pragma unroll
    for (int K = 0; K < kSB; ++K) {
        bad |= !(d > T(0)) || !(d < T(INFINITY));
        const T lkk = d * r;
        const T l = lane > K ? a[K] * r : (lane == K ? lkk : T(0));
        a[K] = l;
        dgv[K] = lkk;
        rdv[K] = r;
        // next pivot: a_(K+1)(K+1) - l_(K+1)K^2 from lane K + 1's register alone, and the next
        // column's values, which take this column's multipliers by v_readlane
        dg = __builtin_fma(-l, l, dg);
        T dn = T(1), rn = T(1);
        if (K + 1 < kSB) {
            dn = read_lane<T>(dg, K + 1);
            a[K + 1] = __builtin_fma(-l, read_lane<T>(l, K + 1), a[K + 1]);
            rn = rsqrt_newton<T>(dn);
        }
        // the pivot chain above is issued before anything that waits for LDS
        __builtin_amdgcn_sched_barrier(0);
        // the previous column's LDS multipliers, read one column ago (columns j >= K + 2)
#pragma unroll
        for (int j = K + 2; j < kSB; ++j) a[j] = __builtin_fma(-pl, pc[j], a[j]);
        if (K + 2 < kSB) a[K + 2] = __builtin_fma(-l, read_lane<T>(l, K + 2), a[K + 2]);
        if (K + 3 < kSB) {
            T* c = &sm.col[K & 1][0];
            c[lane] = l;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int j = K + 3; j < kSB; ++j) pc[j] = c[j];
        }
        pl = l;
        d = dn;
        r = rn;
    }
    if (bad) return false;
    if (valid) {
#pragma unroll
        for (int j = 0; j < kSB; ++j) sm.a[R * kDLD + o + j] = (j <= lane) ? a[j] : T(0);
    }
    T dv = T(0), rv = T(0);
#pragma unroll
    for (int k = 0; k < kSB; ++k)
        if (lane == k) { dv = dgv[k]; rv = rdv[k]; }
    if (lane < kSB) { sm.dg[o + lane] = dv; sm.rd[o + lane] = rv; }
    return true;
}

// X_ww = L_ww^-1 for the 16 x 16 diagonal block w; lane c < 16 computes column c by forward
// substitution (two interleaved partial sums per row).
template <typename T>
__device__ void diag16_inverse(DiagSmem<T>& sm, int w, int lane) {
    const int o = kSB * w, c = lane & 15;
    T t[kSB];
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
        T s0 = (i == c) ? T(1) : T(0), s1 = T(0);
#pragma unroll
        for (int q = 0; q < i; ++q) {
            const T lv = sm.a[(o + i) * kDLD + o + q];
            if (q & 1) s1 = __builtin_fma(-lv, t[q], s1);
            else s0 = __builtin_fma(-lv, t[q], s0);
        }
        t[i] = (s0 + s1) * sm.rd[o + i];
    }
    if (lane < kSB) {
#pragma unroll
        for (int i = 0; i < kSB; ++i) sm.x[(o + i) * kDLD + o + c] = t[i];
    }
}

// L and X = L^-1 of the block in sm.a (lower part; rows and columns beyond the block's size
// hold the identity).  256 threads; false (in every thread) on a bad pivot.
template <typename T>
__device__ bool chol_inv64(DiagSmem<T>& sm) {
    using acc_t = typename Mfma<T>::acc_t;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, fr = lane & 15;
    if (tid == 0) sm.fail = 0;
    __syncthreads();
    for (int p = 0; p < 4; ++p) {
        const int o = kSB * p;
        if (wave == 0 && !panel_sweep<T>(sm, p, lane) && lane == 0) sm.fail = 1;
        __syncthreads();
        if (sm.fail) return false;
        if (p == 3) break;
        // trailing blocks (q, s), p < s <= q: A_qs -= L_qp L_sp^T
        int nb = 0;
        for (int q = p + 1; q < 4; ++q)
            for (int s2 = p + 1; s2 <= q; ++s2, ++nb) {
                if (nb % 4 != wave) continue;
                acc_t acc = {0, 0, 0, 0};
                blk_mma<T>(&sm.a[(kSB * q) * kDLD + o], kDLD, 1, &sm.a[(kSB * s2) * kDLD + o], 1, kDLD, kSB, acc, lane);
#pragma unroll
                for (int v = 0; v < 4; ++v) sm.a[(kSB * q + Mfma<T>::row(lane, v)) * kDLD + kSB * s2 + fr] -= acc[v];
            }
        __syncthreads();
    }
    diag16_inverse<T>(sm, wave, lane);
    __syncthreads();
    // doubling over 16-blocks: X_10 = -X_11 (L_10 X_00), X_32 = -X_33 (L_32 X_22); the products
    // L_VU X_UU park in the (unused) upper blocks (0, 1) and (2, 3) of sm.a
    const int u0 = 32 * wave, v0 = u0 + kSB;
    if (wave < 2) {
        acc_t y = {0, 0, 0, 0};
        blk_mma<T>(&sm.a[v0 * kDLD + u0], kDLD, 1, &sm.x[u0 * kDLD + u0], kDLD, 1, kSB, y, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.a[(u0 + Mfma<T>::row(lane, v)) * kDLD + v0 + fr] = y[v];
    }
    __syncthreads();
    if (wave < 2) {
        acc_t t = {0, 0, 0, 0};
        blk_mma<T>(&sm.x[v0 * kDLD + v0], kDLD, 1, &sm.a[u0 * kDLD + v0], kDLD, 1, kSB, t, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.x[(v0 + Mfma<T>::row(lane, v)) * kDLD + u0 + fr] = -t[v];
    }
    __syncthreads();
    // over 32-blocks: X_VU = -X_VV (L_VU X_UU), U = 0..31, V = 32..63; wave = output block (bi, bj);
    // L_VU X_UU parks in the upper 32 x 32 block of sm.a
    const int bi = wave >> 1, bj = wave & 1;
    {
        acc_t y = {0, 0, 0, 0};
        const int k0 = kSB * bj;   // X_UU is lower: rows below 16 bj only
        blk_mma<T>(&sm.a[(32 + kSB * bi) * kDLD + k0], kDLD, 1, &sm.x[k0 * kDLD + kSB * bj], kDLD, 1, 32 - k0, y, lane);
        __syncthreads();
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.a[(kSB * bi + Mfma<T>::row(lane, v)) * kDLD + 32 + kSB * bj + fr] = y[v];
    }
    __syncthreads();
    {
        acc_t t = {0, 0, 0, 0};
        const int kend = kSB * (bi + 1);   // X_VV is lower
        blk_mma<T>(&sm.x[(32 + kSB * bi) * kDLD + 32], kDLD, 1, &sm.a[32 + kSB * bj], kDLD, 1, kend, t, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.x[(32 + kSB * bi + Mfma<T>::row(lane, v)) * kDLD + kSB * bj + fr] = -t[v];
    }
    __syncthreads();
    return true;
}

// Diagonal block jblk of matrix bz: read from p.S, factor and invert (chol_inv64), write L to
// p.L and the inverse to p.Td, and track the diagonal ratio.  Returns false (fail bit set) on
// a non-positive or non-finite pivot; the decision is the same in every thread.
template <typename T>
__device__ bool diag_factor(const PotrfArgs& p, int bz, DiagSmem<T>& sm);

template <typename T>
__device__ bool diag_block(const PotrfArgs& p, int bz, DiagSmem<T>& sm) {
    const int tid = threadIdx.x, nbj = p.nbj;
    const T* S = (const T*)p.S + bz * p.sL + (int64_t)p.j0 * p.ldl + p.j0;
    {   // all sixteen loads of a thread in flight at once (addresses clamped, values selected)
        T v[kNB * kNB / 256];
        const int64_t o0 = (int64_t)(tid >> 6) * p.ldl + (tid & 63), step = 4 * p.ldl;   // row tid / 64 + 4 q
#pragma unroll
        for (int q = 0; q < kNB * kNB / 256; ++q) {
            const int idx = tid + 256 * q, i = idx >> 6, j = idx & 63;
            v[q] = S[(i < nbj && j <= i) ? o0 + q * step : 0];
        }
#pragma unroll
        for (int q = 0; q < kNB * kNB / 256; ++q) {
            const int idx = tid + 256 * q, i = idx >> 6, j = idx & 63;
            sm.a[i * kDLD + j] = (i < nbj && j <= i) ? v[q] : (i == j ? T(1) : T(0));
        }
    }
    __syncthreads();
    return diag_factor<T>(p, bz, sm);
}

// The rest of diag_block for a block already in sm.a (lower part; the identity elsewhere):
// factor and invert it, track the diagonal ratio, write L and the inverse.
template <typename T>
__device__ bool diag_factor(const PotrfArgs& p, int bz, DiagSmem<T>& sm) {
    const int tid = threadIdx.x, nbj = p.nbj;
    T* L = (T*)p.L + bz * p.sL + (int64_t)p.j0 * p.ldl + p.j0;
    if (!chol_inv64<T>(sm)) {
        if (tid == 0) p.st[bz] |= p.fail_bit;
        return false;
    }
    if (tid < 64) {   // min and max of diag(L) over the block: a wave reduction
        const double d0 = (double)sm.dg[0];
        double mn = tid < nbj ? (double)sm.dg[tid] : d0, mx = mn;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const double on = __shfl_xor(mn, off), ox = __shfl_xor(mx, off);
            mn = on < mn ? on : mn;
            mx = ox > mx ? ox : mx;
        }
        if (tid == 0) {
            double* kp = p.kap + 2 * bz;
            if (!p.first) { mn = kp[0] < mn ? kp[0] : mn; mx = kp[1] > mx ? kp[1] : mx; }
            kp[0] = mn; kp[1] = mx;
            if (p.last && p.tau > 0.0 && mx > p.tau * mn) p.st[bz] |= p.tau_bit;
        }
    }
    T* Td = (T*)p.Td + bz * p.sTd + (int64_t)p.jblk * p.blkTd;
#pragma unroll
    for (int q = 0; q < kNB * kNB / 256; ++q) {
        const int idx = tid + 256 * q, i = idx >> 6, j = idx & 63;
        const bool in = i < nbj && j < nbj;
        if (in && j <= i) L[(int64_t)i * p.ldl + j] = sm.a[i * kDLD + j];
        if (in || p.tdfull) Td[i * p.ldTd + j] = (in && j <= i) ? sm.x[i * kDLD + j] : T(0);
    }
    if (!p.tdfull) {   // Td lies in L^-1: zero the rest of its block row, which 128-wide apply tiles read
        const int rest = (int)(p.ldTd - p.j0) - kNB;
        for (int idx = tid; idx < nbj * rest; idx += 256) Td[(int64_t)(idx / rest) * p.ldTd + kNB + idx % rest] = T(0);
    }
    return true;
}

template <typename T>
__global__ __launch_bounds__(256) void potrf_diag_kernel(PotrfArgs p) {
    const int bz = blockIdx.x;
    if ((p.st[bz] & p.st_mask) != p.st_val) return;
    __shared__ DiagSmem<T> sm;
    diag_block<T>(p, bz, sm);
}

// L = W (+ s I) when shifting: s = c_shift * lam[bz * lam_stride] (an estimate of lambda_max(W))
// if lam is set, else s = c_shift * trace(W).
template <typename T>
__global__ __launch_bounds__(256) void copy_shift_kernel(const T* W, T* L, int64_t r, const int* st, int st_mask,
                                                         int st_val, int shift, double c_shift, const double* lam,
                                                         int64_t lam_stride) {
    const int bz = blockIdx.y;
    if ((st[bz] & st_mask) != st_val) return;
    W += bz * r * r;
    L += bz * r * r;
    T sv = 0;
    if (shift && lam) {
        sv = (T)(c_shift * lam[bz * lam_stride]);
    } else if (shift) {
        __shared__ double red[256];
        double tr = 0;
        for (int64_t i = threadIdx.x; i < r; i += 256) tr += (double)W[i * r + i];
        red[threadIdx.x] = tr;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        sv = (T)(c_shift * red[0]);
    }
    const int64_t total = r * r;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        const int64_t i = idx / r, k = idx % r;
        L[idx] = W[idx] + ((i == k) ? sv : T(0));
    }
}

// ---------------------------------------------------------------------------
// column norms of R, the next Q, and rounding of the fp64 chain to fp32
// ---------------------------------------------------------------------------
// R += Rpart for the matrices with (st & mask) == val: the second K-split of the back-projection.
__global__ __launch_bounds__(256) void add_split_kernel(float* R, const float* Rpart, int64_t total, const int* st,
                                                        int st_mask, int st_val) {
    const int bz = blockIdx.y;
    if ((st[bz] & st_mask) != st_val) return;
    R += bz * total;
    Rpart += bz * total;
    for (int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); i < total; i += 4 * (int64_t)gridDim.x * 256) {
        if (i + 4 <= total && (total & 3) == 0) {
            const float4 a = *(const float4*)(R + i), b = *(const float4*)(Rpart + i);
            *(float4*)(R + i) = float4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
        } else {
            for (int64_t j = i; j < i + 4 && j < total; ++j) R[j] += Rpart[j];
        }
    }
}

__global__ __launch_bounds__(256) void colnorm_partial_kernel(const float* R32, const double* R64, double* part,
                                                              int64_t n, int64_t r, int nchunk, const int* st) {
    const int bz = blockIdx.z, chunk = blockIdx.y;
    const bool p64 = (st[bz] & ST_PATH64) != 0;
    const int64_t col = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
    const int rg = threadIdx.x >> 6;
    const int64_t row0 = (int64_t)chunk * kNormChunk, row1 = row0 + kNormChunk < n ? row0 + kNormChunk : n;
    double s = 0;
    if (col < r) {
        if (p64) {
            const double* R = R64 + bz * n * r;
            for (int64_t i = row0 + rg; i < row1; i += 4) { const double v = R[i * r + col]; s += v * v; }
        } else {
            const float* R = R32 + bz * n * r;
            for (int64_t i = row0 + rg; i < row1; i += 4) { const double v = (double)R[i * r + col]; s += v * v; }
        }
    }
    __shared__ double red[256];
    red[threadIdx.x] = s;
    __syncthreads();
    if (rg == 0 && col < r) {
        const double t = ((red[threadIdx.x] + red[threadIdx.x + 64]) + red[threadIdx.x + 128]) + red[threadIdx.x + 192];
        part[((int64_t)bz * nchunk + chunk) * r + col] = t;
    }
}

__global__ __launch_bounds__(256) void colscale_kernel(const double* part, double* cs, int64_t r, int nchunk,
                                                       double eps) {
    const int bz = blockIdx.y;
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= r) return;
    double s = 0;
    for (int c = 0; c < nchunk; ++c) s += part[((int64_t)bz * nchunk + c) * r + col];
    cs[bz * r + col] = 1.0 / (sqrt(s) + eps);
}

// Four consecutive k of one row of an r-column array (fp64 chain: rounded from R64 / P64 and
// written back to the fp32 copy; fp32 chain: read from it), zero at k >= r.  `vec`: r % 4 == 0,
// so a group lies inside the row and 32-byte aligned.
__device__ __forceinline__ void row4(const double* p64src, float* p32, int64_t o, int64_t k, int64_t r, bool p64,
                                     bool vec, double (&v)[4]) {
    if (vec && k < r) {
        if (p64) {
            const double4 d = *(const double4*)(p64src + o);
            v[0] = d.x; v[1] = d.y; v[2] = d.z; v[3] = d.w;
            *(float4*)(p32 + o) = float4{(float)d.x, (float)d.y, (float)d.z, (float)d.w};
        } else {
            const float4 f = *(const float4*)(p32 + o);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = 0.0;
        if (k + e < r) {
            if (p64) { v[e] = p64src[o + e]; p32[o + e] = (float)v[e]; }
            else v[e] = p32[o + e];
        }
    }
}

// Q <- R * c (fp32), and for fp64-chain matrices R32 <- R64 rounded (the weight pass reads the
// fp32 R); four k per thread.
__global__ __launch_bounds__(256) void next_q_kernel(const double* R64, float* R32, const double* cs, float* Q,
                                                     int64_t n, int64_t r, const int* st) {
    const int bz = blockIdx.y;
    if (st[bz] & ST_FAIL) return;   // no factor: Q stays as it was
    const bool p64 = (st[bz] & ST_PATH64) != 0, vec = (r % 4) == 0;
    const int64_t nr = n * r, gpr = (r + 3) / 4, groups = n * gpr;
    const double* c = cs + bz * r;
    for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups; gi += (int64_t)gridDim.x * 256) {
        const int64_t i = gi / gpr, k = 4 * (gi % gpr), o = bz * nr + i * r + k;
        double v[4];
        row4(R64, R32, o, k, r, p64, vec, v);
        float qv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[e] = k + e < r ? (float)(v[e] * c[k + e]) : 0.f;
        if (vec) *(float4*)(Q + o) = float4{qv[0], qv[1], qv[2], qv[3]};
        else
#pragma unroll
            for (int e = 0; e < 4; ++e) if (k + e < r) Q[o + e] = qv[e];
    }
}

// P32 <- P64 rounded, for fp64-chain matrices (the fp32 chain's P is already there).
__global__ __launch_bounds__(256) void round_p_kernel(const double* P64, float* P32, int64_t m, int64_t r,
                                                      const int* st) {
    const int bz = blockIdx.y;
    if ((st[bz] & ST_PATH64) == 0) return;
    const bool vec = (r % 4) == 0;
    const int64_t mr = m * r, gpr = (r + 3) / 4, groups = m * gpr;
    for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups; gi += (int64_t)gridDim.x * 256) {
        const int64_t i = gi / gpr, k = 4 * (gi % gpr), o = bz * mr + i * r + k;
        double v[4];
        row4(P64, P32, o, k, r, true, vec, v);
    }
}

// ---------------------------------------------------------------------------
// momentum / weight pass:  M <- (M + G) - (1 - mu) P R^T,  X <- X - lr s P Q^T
// ---------------------------------------------------------------------------
struct UpdArgs {
    const float* P; const float* R; const float* Q;   // fp32 [b][rows][r], k contiguous
    float* M; const void* G; void* X;
    const int* st;                                    // per-matrix state words
    int m, n, r, kp;                                  // kp: r rounded up to whole 32-k slabs
    bool vec;                                         // r % 4 == 0: 16-byte row loads
    float one_minus_mu, lr_s;
    // momentum-change partials (null: not requested): per matrix nmx slots of (max |M' - M|,
    // max |M|), one per tile, at tile y * tiles_x + x
    float* mx;
    int64_t nmx;
};

// Maxima of a and b over the workgroup (blockDim.x a multiple of 64, every thread calling);
// thread 0 writes them to out[0] and out[1].
__device__ void wg_max2_store(float a, float b, float* out) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a = fmaxf(a, __shfl_xor(a, o));
        b = fmaxf(b, __shfl_xor(b, o));
    }
    __shared__ float sa[16], sb[16];
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) { sa[w] = a; sb[w] = b; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < nw; ++i) { a = fmaxf(a, sa[i]); b = fmaxf(b, sb[i]); }
        out[0] = a;
        out[1] = b;
    }
}

// Slot of this workgroup's momentum-change partials (tile coordinates x, y).
__device__ __forceinline__ float* mx_slot(const UpdArgs& u, int bz, int tx, int ty, int tiles_x) {
    return u.mx + ((int64_t)bz * u.nmx + (int64_t)ty * tiles_x + tx) * 2;
}

// The tile of a matrix whose orthonormalization broke down with no fallback left (ST_FAIL):
// there is no factor to update with, so the step is the rank-0 one, M <- M + G, X untouched.
template <int BM, int BN, bool G_BF16>
__device__ void failed_tile(const UpdArgs& u, int bz, int m0, int n0) {
    const int64_t mn = (int64_t)u.m * u.n;
    float dmax = 0.f, smax = 0.f;
    for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
        const int row = m0 + idx / BN, col = n0 + idx % BN;
        if (row >= u.m || col >= u.n) continue;
        const int64_t off = bz * mn + (int64_t)row * u.n + col;
        float g;
        if constexpr (G_BF16) g = bf16_bits_to_float(((const uint16_t*)u.G)[off]);
        else g = ((const float*)u.G)[off];
        const float mo = u.M[off], mnew = mo + g;
        u.M[off] = mnew;
        dmax = fmaxf(dmax, fabsf(mnew - mo));
        smax = fmaxf(smax, fabsf(mo));
    }
    if (u.mx) wg_max2_store(dmax, smax, mx_slot(u, bz, n0 / BN, m0 / BM, (u.n + BN - 1) / BN));
}

// One BM x BN tile of M and X per workgroup of WGM x WGN waves: both rank-kp products on the
// bf16 matrix cores in the six-term split form (fp32 accuracy), sharing the P fragments, then
// one pass over the tile of M, G and X.  P, R and Q are read as fp32 and split into their
// three bf16 parts on the way into LDS; nine part tiles (P, R, Q x h, m, l) per 32-k slab,
// double-buffered.
template <int BM, int BN, int WGM, int WGN, bool G_BF16, bool X_BF16, int NP>
__global__ __launch_bounds__(WGM * WGN * 64) void update_kernel(UpdArgs u) {
    constexpr int NT = WGM * WGN * 64, BK = kSplitK;
    constexpr int FM = BM / WGM / 16, FN = BN / WGN / 16;
    static_assert(NT == 256, "the split loaders stage with 256 threads");
    static_assert(FM * WGM * 16 == BM && FN * WGN * 16 == BN, "whole MFMA blocks per wave");
    const TileId tid = xcd_tile_id();
    const int bz = tid.z, m0 = tid.y * BM, n0 = tid.x * BN;
    if (u.st[bz] & ST_FAIL) {
        failed_tile<BM, BN, G_BF16>(u, bz, m0, n0);
        return;
    }
    __shared__ __attribute__((aligned(16))) uint16_t ldsA[2][NP][BM * BK];       // P parts
    __shared__ __attribute__((aligned(16))) uint16_t ldsB[2][2 * NP][BN * BK];   // R parts | Q parts
    const int64_t pr = (int64_t)u.m * u.r, nr = (int64_t)u.n * u.r;
    const Op6 oP{u.P + bz * pr, nullptr, u.r, u.m, u.r, u.vec};
    const Op6 oR{u.R + bz * nr, nullptr, u.r, u.n, u.r, u.vec};
    const Op6 oQ{u.Q + bz * nr, nullptr, u.r, u.n, u.r, u.vec};
    const int t = threadIdx.x;
    Loader6<BM, S6_KC8, A6_NONE> lp;
    Loader6<BN, S6_KC8, A6_NONE> lr, lq;
    auto gload = [&](int k0) {
        lp.load(oP, m0, k0, t);
        lr.load(oR, n0, k0, t);
        lq.load(oQ, n0, k0, t);
    };
    auto lstore = [&](int buf) {
        lp.template split_store<NP>(&ldsA[buf][0][0], t);
        lr.template split_store<NP>(&ldsB[buf][0][0], t);
        lq.template split_store<NP>(&ldsB[buf][NP][0], t);
    };

    const int lane = t & 63, wave = t >> 6, wm = wave / WGN, wn = wave % WGN;
    const int fr = lane & 15, fc = lane >> 4;
    int ao[FM], bo[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) ao[i] = part_off(wm * FM * 16 + i * 16 + fr, fc);
#pragma unroll
    for (int j = 0; j < FN; ++j) bo[j] = part_off(wn * FN * 16 + j * 16 + fr, fc);
    f32x4 acc1[FM][FN], acc2[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) { acc1[i][j] = f32x4{0, 0, 0, 0}; acc2[i][j] = f32x4{0, 0, 0, 0}; }

    gload(0);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < u.kp; k0 += BK) {
        const bool more = k0 + BK < u.kp;
        if (more) gload(k0 + BK);
        u32x4 a[FM][NP], b[FN][NP], c[FN][NP];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int q = 0; q < NP; ++q) a[i][q] = *(const u32x4*)&ldsA[buf][q][ao[i]];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                b[j][q] = *(const u32x4*)&ldsB[buf][q][bo[j]];
                c[j][q] = *(const u32x4*)&ldsB[buf][NP + q][bo[j]];
            }
        // the part products smallest first: six for three parts, the last three of them for two
        // parts (hl, lh, hh), the single hh product for plain bf16
        constexpr int NTERM = NP == 1 ? 1 : NP == 2 ? 3 : 6;
#pragma unroll
        for (int term = 0; term < NTERM; ++term)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int ta = NP == 1 ? 0 : kTermA[6 - NTERM + term];
                    const int tb = NP == 1 ? 0 : kTermB[6 - NTERM + term];
                    acc1[i][j] = mma_bf16(a[i][ta], b[j][tb], acc1[i][j]);
                    acc2[i][j] = mma_bf16(a[i][ta], c[j][tb], acc2[i][j]);
                }
        if (more) lstore(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    // Epilogue: every load of the tile is issued before the first store (a store may alias a
    // later load, so interleaving them would serialize one memory round trip per element).
    const int64_t mn = (int64_t)u.m * u.n;
    float* Mp = u.M + bz * mn;
    float mv[FM][FN][4], gv[FM][FN][4], xv[FM][FN][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * FM * 16 + i * 16 + 4 * fc + v;
                const int col = n0 + wn * FN * 16 + j * 16 + fr;
                const int64_t l = (row < u.m && col < u.n) ? (int64_t)row * u.n + col : 0, off = bz * mn + l;
                mv[i][j][v] = Mp[l];
                if constexpr (G_BF16) gv[i][j][v] = bf16_bits_to_float(((const uint16_t*)u.G)[off]);
                else gv[i][j][v] = ((const float*)u.G)[off];
                if constexpr (X_BF16) xv[i][j][v] = bf16_bits_to_float(((const uint16_t*)u.X)[off]);
                else xv[i][j][v] = ((const float*)u.X)[off];
            }
    float dmax = 0.f, smax = 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * FM * 16 + i * 16 + 4 * fc + v;
                const int col = n0 + wn * FN * 16 + j * 16 + fr;
                if (row >= u.m || col >= u.n) continue;
                const int64_t l = (int64_t)row * u.n + col, off = bz * mn + l;
                const float mnew = (mv[i][j][v] + gv[i][j][v]) - u.one_minus_mu * acc1[i][j][v];
                Mp[l] = mnew;
                dmax = fmaxf(dmax, fabsf(mnew - mv[i][j][v]));
                smax = fmaxf(smax, fabsf(mv[i][j][v]));
                const float x = xv[i][j][v] - u.lr_s * acc2[i][j][v];
                if constexpr (X_BF16) ((uint16_t*)u.X)[off] = float_to_bf16_bits(x);
                else ((float*)u.X)[off] = x;
            }
    if (u.mx) wg_max2_store(dmax, smax, mx_slot(u, bz, tid.x, tid.y, (u.n + BN - 1) / BN));
}

// The weight pass for large stacks: 128 x 64 tiles of M and X, four waves of 64 x 32 that
// both stage (fp32 P, R and Q rows, split into bf16 parts on the way into LDS: 32 KB read per
// slab where pre-split parts would take 48 KB) and multiply, and a single-buffered 48 KB LDS
// stage (two barriers per slab).  Two workgroups fit on a CU, so one workgroup's memory-bound
// epilogue (the loads of each half-tile issued before its stores) runs while the other keeps
// the matrix cores busy.

// Streaming (non-temporal) 16- and 8-byte accesses for the weight pass's M, G and X, which are
// touched once: they then leave the L2 to the P, R and Q rows that every tile re-reads.
__device__ __forceinline__ float4 nt_ld4(const float* p) {
    const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
    return float4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void nt_st4(float* p, float4 v) { __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, (f32x4*)p); }
__device__ __forceinline__ uint2 nt_ld2(const uint16_t* p) {
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    return uint2{v[0], v[1]};
}
__device__ __forceinline__ void nt_st2(uint16_t* p, uint2 v) { __builtin_nontemporal_store(u32x2{v.x, v.y}, (u32x2*)p); }
template <bool G_BF16, bool X_BF16, bool FAST, int NP>
__global__ __launch_bounds__(256, 2) void update3_kernel(UpdArgs u) {
    constexpr int BM = 128, BN = 64, PA = BM * kSplitK, PB = BN * kSplitK, FM = 4, FN = 2;
    // the part tiles, reused by the epilogue as a 128 x (64 + 4) fp32 tile
    constexpr int LDS_PARTS = NP * PA + 2 * NP * PB, LDS_TILE = BM * (BN + 4) * 2;
    constexpr int LDS_N = LDS_PARTS > LDS_TILE ? LDS_PARTS : LDS_TILE;
    const TileId tid = xcd_tile_id();
    const int bz = tid.z, m0 = tid.y * BM, n0 = tid.x * BN;
    if (u.st[bz] & ST_FAIL) {
        failed_tile<BM, BN, G_BF16>(u, bz, m0, n0);
        return;
    }
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_N];   // P parts | R parts | Q parts
    const int64_t pr = (int64_t)u.m * u.r, nr = (int64_t)u.n * u.r;
    const Op6 oP{u.P + bz * pr, nullptr, u.r, u.m, u.r, u.vec};
    const Op6 oR{u.R + bz * nr, nullptr, u.r, u.n, u.r, u.vec};
    const Op6 oQ{u.Q + bz * nr, nullptr, u.r, u.n, u.r, u.vec};
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 15, fc = lane >> 4;
    f32x4 acc1[FM][FN], acc2[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) { acc1[i][j] = f32x4{0, 0, 0, 0}; acc2[i][j] = f32x4{0, 0, 0, 0}; }
    auto mma = [&]() {
        mma6_slab2<BM, BN, FM, FN, NP>(lds, lds + NP * PA, lds + NP * PA + NP * PB, acc1, acc2, wm * 64, wn * 32, fr,
                                       fc);
    };
    if constexpr (FAST) {
        // every tile interior and every slab whole: two register sets, so each slab's loads are
        // issued two slabs before its split (branch-free steady loop, then a drain)
        Loader6<BM, S6_KC8, A6_NONE> lp[2];
        Loader6<BN, S6_KC8, A6_NONE> lr[2], lq[2];
        auto load = [&](auto jc, int k) {
            constexpr int J = decltype(jc)::value;
            lp[J].load_fast(oP, m0, k, t);
            lr[J].load_fast(oR, n0, k, t);
            lq[J].load_fast(oQ, n0, k, t);
        };
        auto store = [&](auto jc) {
            constexpr int J = decltype(jc)::value;
            lp[J].template split_store<NP>(lds, t);
            lr[J].template split_store<NP>(lds + NP * PA, t);
            lq[J].template split_store<NP>(lds + NP * PA + NP * PB, t);
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        const int nslab = u.kp / kSplitK;   // >= 2
        load(I0{}, 0);
        load(I1{}, kSplitK);
        store(I0{});
        __syncthreads();
        int sl = 0;
        for (; sl + 3 < nslab; sl += 2) {   // LDS: slab sl; set 1: slab sl + 1
            load(I0{}, (sl + 2) * kSplitK);
            mma();
            __syncthreads();
            store(I1{});
            __syncthreads();
            load(I1{}, (sl + 3) * kSplitK);
            mma();
            __syncthreads();
            store(I0{});
            __syncthreads();
        }
        // the last two or three slabs: LDS holds slab sl, set 1 slab sl + 1 (sl + 2 < nslab: set 0
        // is loaded below)
        const bool three = sl + 2 < nslab;
        if (three) load(I0{}, (sl + 2) * kSplitK);
        mma();
        __syncthreads();
        store(I1{});
        __syncthreads();
        mma();
        if (three) {
            __syncthreads();
            store(I0{});
            __syncthreads();
            mma();
        }
        // the epilogue below reuses the part tiles' LDS: every wave must be done reading them
        __syncthreads();
    } else {
        Loader6<BM, S6_KC8, A6_NONE> lp;
        Loader6<BN, S6_KC8, A6_NONE> lr, lq;
        auto load = [&](int k) {
            lp.load(oP, m0, k, t);
            lr.load(oR, n0, k, t);
            lq.load(oQ, n0, k, t);
        };
        auto store = [&]() {
            lp.template split_store<NP>(lds, t);
            lr.template split_store<NP>(lds + NP * PA, t);
            lq.template split_store<NP>(lds + NP * PA + NP * PB, t);
        };
        load(0);
        store();
        __syncthreads();
        for (int k0 = 0; k0 < u.kp; k0 += kSplitK) {
            const bool more = k0 + kSplitK < u.kp;
            if (more) load(k0 + kSplitK);
            mma();
            __syncthreads();
            if (more) {
                store();
                __syncthreads();
            }
        }
    }
    const int64_t mn = (int64_t)u.m * u.n;
    // full tiles: each product tile goes through LDS to rows of 64 consecutive columns, so M, G
    // and X move as 16-byte (bf16: 8-byte) vectors; all loads of a pass before its stores
    float dmax = 0.f, smax = 0.f;   // momentum change and size over this tile
    if (m0 + BM <= u.m && n0 + BN <= u.n && (u.n & 3) == 0) {
        constexpr int TP = BN + 4;
        float* tl = (float*)lds;
        // every HBM load of the tile (M, G and X) is issued before the first product goes through
        // LDS, so a workgroup keeps all of its streaming bytes in flight at once
        using GRaw = std::conditional_t<G_BF16, uint2, float4>;
        using XRaw = std::conditional_t<X_BF16, uint2, float4>;
        float4 mv[8];
        GRaw gr[8];
        XRaw xr[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = 4 * (t + 256 * q), row = e >> 6, col = e & 63;
            const int64_t off = bz * mn + (int64_t)(m0 + row) * u.n + n0 + col;
            mv[q] = nt_ld4(u.M + off);
            if constexpr (G_BF16) gr[q] = nt_ld2((const uint16_t*)u.G + off);
            else gr[q] = nt_ld4((const float*)u.G + off);
            if constexpr (X_BF16) xr[q] = nt_ld2((const uint16_t*)u.X + off);
            else xr[q] = nt_ld4((const float*)u.X + off);
        }
        auto widen4 = [](auto w) -> float4 {
            if constexpr (std::is_same_v<decltype(w), uint2>)
                return float4{bf16_bits_to_float(w.x & 0xffffu), bf16_bits_to_float(w.x >> 16),
                              bf16_bits_to_float(w.y & 0xffffu), bf16_bits_to_float(w.y >> 16)};
            else return w;
        };
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        tl[(wm * 64 + 16 * i + 4 * fc + v) * TP + wn * 32 + 16 * j + fr] = pass ? acc2[i][j][v] : acc1[i][j][v];
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int e = 4 * (t + 256 * q), row = e >> 6, col = e & 63;
                const float4 av = *(const float4*)&tl[row * TP + col];
                const int64_t off = bz * mn + (int64_t)(m0 + row) * u.n + n0 + col;
                if (pass == 0) {
                    const float c = u.one_minus_mu;
                    const float4 mo = mv[q], gv = widen4(gr[q]);
                    const float4 mnew = float4{(mo.x + gv.x) - c * av.x, (mo.y + gv.y) - c * av.y,
                                               (mo.z + gv.z) - c * av.z, (mo.w + gv.w) - c * av.w};
                    nt_st4(u.M + off, mnew);
                    dmax = fmaxf(fmaxf(fmaxf(dmax, fabsf(mnew.x - mo.x)), fmaxf(fabsf(mnew.y - mo.y),
                                 fabsf(mnew.z - mo.z))), fabsf(mnew.w - mo.w));
                    smax = fmaxf(fmaxf(fmaxf(smax, fabsf(mo.x)), fmaxf(fabsf(mo.y), fabsf(mo.z))), fabsf(mo.w));
                } else {
                    const float c = u.lr_s;
                    const float4 xo = widen4(xr[q]);
                    const float4 x = float4{xo.x - c * av.x, xo.y - c * av.y, xo.z - c * av.z, xo.w - c * av.w};
                    if constexpr (X_BF16)
                        nt_st2((uint16_t*)u.X + off, uint2{pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w)});
                    else nt_st4((float*)u.X + off, x);
                }
            }
            __syncthreads();
        }
        if (u.mx) wg_max2_store(dmax, smax, mx_slot(u, bz, tid.x, tid.y, (u.n + BN - 1) / BN));
        return;
    }
    // partial tiles: in the MFMA layout, in two halves of rows, all loads of a half before its stores
    float* Mp = u.M + bz * mn;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float mv[2][FN][4], gv[2][FN][4], xv[2][FN][4];
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = 2 * h + ii;
                    const int row = m0 + wm * 64 + 16 * i + 4 * fc + v, col = n0 + wn * 32 + 16 * j + fr;
                    const int64_t l = (row < u.m && col < u.n) ? (int64_t)row * u.n + col : 0, off = bz * mn + l;
                    mv[ii][j][v] = Mp[l];
                    if constexpr (G_BF16) gv[ii][j][v] = bf16_bits_to_float(((const uint16_t*)u.G)[off]);
                    else gv[ii][j][v] = ((const float*)u.G)[off];
                    if constexpr (X_BF16) xv[ii][j][v] = bf16_bits_to_float(((const uint16_t*)u.X)[off]);
                    else xv[ii][j][v] = ((const float*)u.X)[off];
                }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = 2 * h + ii;
                    const int row = m0 + wm * 64 + 16 * i + 4 * fc + v, col = n0 + wn * 32 + 16 * j + fr;
                    if (row >= u.m || col >= u.n) continue;
                    const int64_t l = (int64_t)row * u.n + col, off = bz * mn + l;
                    const float mnew = (mv[ii][j][v] + gv[ii][j][v]) - u.one_minus_mu * acc1[i][j][v];
                    Mp[l] = mnew;
                    dmax = fmaxf(dmax, fabsf(mnew - mv[ii][j][v]));
                    smax = fmaxf(smax, fabsf(mv[ii][j][v]));
                    const float x = xv[ii][j][v] - u.lr_s * acc2[i][j][v];
                    if constexpr (X_BF16) ((uint16_t*)u.X)[off] = float_to_bf16_bits(x);
                    else ((float*)u.X)[off] = x;
                }
    }
    if (u.mx) wg_max2_store(dmax, smax, mx_slot(u, bz, tid.x, tid.y, (u.n + BN - 1) / BN));
}

// rank 0: M <- M + G (grid: blocks per matrix x matrices); with mx set, each block leaves
// the momentum change and size over its share in its slot of the matrix's partials
template <bool G_BF16>
__global__ __launch_bounds__(256) void add_grad_kernel(float* M, const void* G, int64_t mn, float* mx,
                                                       int64_t nmx) {
    const int64_t bz = blockIdx.y, base = bz * mn;
    float dmax = 0.f, smax = 0.f;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < mn; idx += (int64_t)gridDim.x * 256) {
        float g;
        if constexpr (G_BF16) g = bf16_bits_to_float(((const uint16_t*)G)[base + idx]);
        else g = ((const float*)G)[base + idx];
        const float mo = M[base + idx], mnew = mo + g;
        M[base + idx] = mnew;
        dmax = fmaxf(dmax, fabsf(mnew - mo));
        smax = fmaxf(smax, fabsf(mo));
    }
    if (mx) wg_max2_store(dmax, smax, mx + (bz * nmx + blockIdx.x) * 2);
}

// rmmc[bz] = max |M' - M| / max |M| of matrix bz from its nparts partials (0 or +inf where max
// |M| = 0: no change, or a change from zero momentum).  One workgroup per matrix.
__global__ __launch_bounds__(256) void rmmc_kernel(const float* mx, int64_t nmx, int nparts, float* rmmc) {
    const int64_t bz = blockIdx.x;
    float d = 0.f, s = 0.f;
    for (int i = threadIdx.x; i < nparts; i += 256) {
        d = fmaxf(d, mx[(bz * nmx + i) * 2]);
        s = fmaxf(s, mx[(bz * nmx + i) * 2 + 1]);
    }
    __shared__ float out[2];
    wg_max2_store(d, s, out);
    __syncthreads();
    if (threadIdx.x == 0) rmmc[bz] = out[1] > 0.f ? out[0] / out[1] : (out[0] > 0.f ? INFINITY : 0.f);
}

__global__ void zero_flags_kernel(int32_t* flags, int64_t b) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < b) flags[i] = 0;
}

__global__ void init_state_kernel(int* st, const int32_t* flags, int64_t b, int force64, int sticky) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= b) return;
    const bool f64 = force64 || (sticky && flags && (flags[i] & DION_FLAG_F64));
    st[i] = f64 ? ST_PATH64 : 0;
}

__global__ __launch_bounds__(256) void flags_out_kernel(const int* st, const double* cs, int64_t r,
                                                        int32_t* flags) {
    const int bz = blockIdx.x;
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    int mine = 0;
    for (int64_t k = threadIdx.x; k < r; k += 256) mine |= !isfinite(cs[bz * r + k]);
    if (mine) bad = 1;   // benign same-value race
    __syncthreads();
    if (threadIdx.x == 0) {
        const int s = st[bz];
        int f = 0;
        if (s & ST_PATH64) f |= DION_FLAG_F64;
        if (s & ST_SHIFT) f |= DION_FLAG_SHIFTED;
        if (s & ST_HH) f |= DION_FLAG_HOUSEHOLDER;
        if ((s & ST_FAIL) || bad) f |= DION_FLAG_NONFINITE;
        flags[bz] = f;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
#define DION_TRY(expr)                              \
    do {                                            \
        hipError_t e_ = (expr);                     \
        if (e_ != hipSuccess) return (int)e_;       \
    } while (0)
#define DION_TRY_HIP(expr)                          \
    do {                                            \
        hipError_t e_ = (expr);                     \
        if (e_ != hipSuccess) return e_;            \
    } while (0)

static bool aligned4(const void* p, int esz) { return ((uintptr_t)p % (uintptr_t)(4 * esz)) == 0; }

static unsigned grid_1d(int64_t total, int64_t cap = 2048) {
    int64_t g = (total + 255) / 256;
    if (g < 1) g = 1;
    return (unsigned)(g < cap ? g : cap);
}

template <typename T> struct SrcOf;
template <> struct SrcOf<float> { static constexpr int v = SRC_F32; };
template <> struct SrcOf<double> { static constexpr int v = SRC_F64; };

struct ChainCtx {
    const Plan* p;
    char* ws;
    int* st;
    hipStream_t s;
    hipEvent_t gate = nullptr;   // recorded once, after the chunk's first product (staggered chunks)
    bool* gated = nullptr;
    // shifted passes: s = c_shift * lam[b * lam_stride] (the multi-power-iteration estimate of
    // lambda_max(W)) when set, else s = c_shift * trace(W)
    const double* lam = nullptr;
    int64_t lam_stride = 0;
    // bf16 weights: the two big products of the fp32 chain as plain bf16 products
    bool plain = false;
    hipError_t open_gate() const {
        if (!gate || *gated) return hipSuccess;
        *gated = true;
        return hipEventRecord(gate, s);
    }
};

// CholeskyQR building blocks on P [b][m][r], for the matrices with (st & mask) == val.
// gram:    W = P^T P (lower tiles)
// factor:  L = chol(W (+ s I)) by blocks of kNB columns (right-looking), with the inverse
//          of every diagonal block written to the matching diagonal block of Tf; a failed
//          pivot sets `fail_bit`, a diagonal ratio above `tau` (tau > 0) sets `tau_bit`
// invert:  Tf = L^-1 (its lower off-diagonal blocks);   apply: Pout = Pin Tf^T
// The blocks of Tf above the diagonal are never written: every consumer skips them.
// W = sum over the K-splits of the partial Grams, in split order (lower triangle).
template <typename T>
__global__ __launch_bounds__(256) void gram_reduce_kernel(const T* part, T* W, int64_t r, int64_t splits,
                                                          const int* st, int st_mask, int st_val) {
    const int bz = blockIdx.y;
    if ((st[bz] & st_mask) != st_val) return;
    part += bz * splits * r * r;
    W += bz * r * r;
    const int64_t total = r * r;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        if (idx % r > idx / r) continue;            // the consumers read the lower triangle only
        T s = 0;
        for (int64_t q = 0; q < splits; ++q) s += part[q * total + idx];
        W[idx] = s;
    }
}

// W = P^T P; a split Gram leaves its partials in gpart and, unless `reduce` is false (the
// caller then sums them itself), adds them into W.
// fp32-chain Gram and apply on the split-bf16 kernel (defined with it below)
static int gram6(const ChainCtx& c, const float* P, int mask, int val, int64_t splits, int64_t kc);
static int apply6(const ChainCtx& c, const float* Pin, float* Pout, int mask, int val);
template <typename T>
static int64_t gram_splits(const Plan& p) { return (sizeof(T) == 4 && DION_PROD6) ? p.gsplit6 : p.gsplit; }

template <typename T>
static int gram(const ChainCtx& c, const T* P, int mask, int val, bool reduce = true) {
    const Plan& p = *c.p;
    const int64_t m = p.m, r = p.r;
    constexpr int S = SrcOf<T>::v;
    const bool vr = (r % 4) == 0;
    const int64_t splits = gram_splits<T>(p);
    int64_t kc = (m + splits - 1) / splits;
    if constexpr (sizeof(T) == 4 && DION_PROD6) {
        // whole 32-k slabs per split where that still leaves the last split some rows, so the
        // split-bf16 kernel can take its branch-free path
        const int64_t kc32 = (kc + kSplitK - 1) / kSplitK * kSplitK;
        if ((splits - 1) * kc32 < m) kc = kc32;
        int e;
        if ((e = gram6(c, P, mask, val, splits, kc))) return e;
        if (splits <= 1) return 0;
    } else {
        // whole 16-k slabs per split where that still leaves the last split some rows, so every
        // tile takes the branch-free main loop
        const int64_t kc16 = (kc + 15) / 16 * 16;
        if ((splits - 1) * kc16 < m) kc = kc16;
        GemmArgs g{};
        g.a = Operand{P, nullptr, r, (int)r, (int)m, vr};   // A(i,k) = P[k][i]
        g.b = Operand{P, nullptr, r, (int)r, (int)m, vr};   // B(k,j) = P[k][j]
        g.sa0 = g.sb0 = m * r * (int64_t)sizeof(T);
        g.M = g.N = (int)r;
        g.alpha = 1; g.beta = 0;
        g.st = c.st; g.st_mask = mask; g.st_val = val; g.lower = 1;
        if (splits <= 1) {
            g.c = c.ws + p.W; g.ldc = r; g.sc = r * r * (int64_t)sizeof(T);
            g.K = (int)m;
            DION_TRY((launch_gemm<T, 64, 64, false, S, false, S>(g, p.b, c.s)));
            return 0;
        }
        g.K = (int)kc;
        g.zdiv = (int)splits;
        g.ksplit_total = (int)m;
        g.ga0 = g.gb0 = kc * r * (int64_t)sizeof(T);
        g.c = c.ws + p.gpart; g.ldc = r;
        g.sc = splits * r * r * (int64_t)sizeof(T);
        g.gc = r * r * (int64_t)sizeof(T);
        DION_TRY((launch_gemm<T, 64, 64, false, S, false, S>(g, p.b, c.s)));
    }
    if (!reduce) return 0;
    dim3 grid(grid_1d(r * r, 512), (unsigned)p.b);
    hipLaunchKernelGGL((gram_reduce_kernel<T>), grid, dim3(256), 0, c.s, (const T*)(c.ws + p.gpart), (T*)(c.ws + p.W),
                       r, splits, c.st, mask, val);
    DION_TRY(hipGetLastError());
    return 0;
}

// arguments of chol_step_kernel (defined below, with the LDS block helpers it uses)
struct CholStepArgs {
    const void* S;       // source of the panel and trailing blocks at this step
    void* L; void* Tf;
    int64_t r;
    int nblk, jb;
    const int* st; int st_mask, st_val;
    PotrfArgs diag;      // the next diagonal block (task 0), base pointers
};

template <typename T>
__global__ __launch_bounds__(256) void chol_step_kernel(CholStepArgs a);

// Blocked right-looking Cholesky L = chol(W (+ s I)).  With `with_inverse` (ranks up to
// kFusedMaxBlocks blocks) Tf = L^-1 is built alongside, in nblk + 1 launches: the first diagonal
// block, then one chol_step_kernel launch per block step (trailing tiles with their panel blocks,
// the next diagonal block, the inverse tiles of the step's block row) and one for the last
// block row of the inverse.  A matrix that tau_bit marks at the last diagonal block skips the
// last inverse tiles (a later shifted call refactors it).  Without the inverse: a diagonal,
// panel and trailing launch per block.
template <typename T>
static int factor(const ChainCtx& c, int mask, int val, double tau, int fail_bit, int tau_bit, int shift,
                  bool with_inverse) {
    const Plan& p = *c.p;
    const int64_t m = p.m, r = p.r, b = p.b;
    T* W = (T*)(c.ws + p.W);
    T* L = (T*)(c.ws + p.L);
    T* Tf = (T*)(c.ws + p.Tf);
    double* kap = (double*)(c.ws + p.kap);
    constexpr int S = SrcOf<T>::v;
    const bool vr = (r % 4) == 0;
    const int64_t rr = r * r * (int64_t)sizeof(T);
    // Unshifted, the first block column reads W and writes L (W stays intact for a shifted
    // retry); shifted, L = W + s I is formed first.
    if (shift) {
        const double u = sizeof(T) == 8 ? 1.1102230246251565e-16 : 5.9604644775390625e-08;
        const double c_shift = 11.0 * ((double)m * r + (double)r * (r + 1)) * u;
        dim3 grid(grid_1d(r * r, 1024), (unsigned)b);
        hipLaunchKernelGGL((copy_shift_kernel<T>), grid, dim3(256), 0, c.s, W, L, r, c.st, mask, val, shift, c_shift,
                           c.lam, c.lam_stride);
        DION_TRY(hipGetLastError());
    }
    auto diag_args = [&](int64_t jb) {
        PotrfArgs pa{};
        pa.L = L; pa.ldl = r; pa.sL = r * r; pa.S = (jb == 0 && !shift) ? W : L;
        // the inverted diagonal blocks go straight into the diagonal of Tf = L^-1
        pa.Td = Tf; pa.sTd = r * r; pa.ldTd = r; pa.blkTd = kNB * (r + 1); pa.tdfull = 0;
        pa.j0 = (int)(jb * kNB); pa.nbj = (int)((r - jb * kNB) < kNB ? (r - jb * kNB) : kNB); pa.jblk = (int)jb;
        pa.st = c.st; pa.st_mask = mask; pa.st_val = val;
        pa.kap = kap; pa.first = jb == 0; pa.last = jb == p.nblk - 1;
        pa.tau = tau; pa.fail_bit = fail_bit; pa.tau_bit = tau_bit;
        return pa;
    };
    if (with_inverse) {
        hipLaunchKernelGGL((potrf_diag_kernel<T>), dim3((unsigned)b), dim3(256), 0, c.s, diag_args(0));
        DION_TRY(hipGetLastError());
        for (int64_t jb = 0; jb < p.nblk && p.nblk > 1; ++jb) {
            const int64_t n = p.nblk - 1 - jb, tasks = n * (n + 1) / 2 + jb;
            CholStepArgs sa{};
            sa.S = (jb == 0 && !shift) ? W : L; sa.L = L; sa.Tf = Tf;
            sa.r = r; sa.nblk = (int)p.nblk; sa.jb = (int)jb;
            sa.st = c.st; sa.st_mask = jb == p.nblk - 1 ? (mask | tau_bit) : mask; sa.st_val = val;
            if (n > 0) { sa.diag = diag_args(jb + 1); sa.diag.S = L; }
            hipLaunchKernelGGL((chol_step_kernel<T>), dim3((unsigned)tasks, (unsigned)b), dim3(256), 0, c.s, sa);
            DION_TRY(hipGetLastError());
        }
        return 0;
    }
    for (int64_t jb = 0; jb < p.nblk; ++jb) {
        const int j0 = (int)(jb * kNB);
        const int nbj = (int)((r - j0) < kNB ? (r - j0) : kNB);
        const int rest = (int)(r - j0 - nbj);
        const T* src = (jb == 0 && !shift) ? W : L;
        PotrfArgs pa{};
        pa.L = L; pa.ldl = r; pa.sL = r * r; pa.S = src;
        // the inverted diagonal blocks go straight into the diagonal of Tf = L^-1
        pa.Td = Tf; pa.sTd = r * r; pa.ldTd = r; pa.blkTd = kNB * (r + 1); pa.tdfull = 0;
        pa.j0 = j0; pa.nbj = nbj; pa.jblk = (int)jb;
        pa.st = c.st; pa.st_mask = mask; pa.st_val = val;
        pa.kap = kap; pa.first = jb == 0; pa.last = jb == p.nblk - 1;
        pa.tau = tau; pa.fail_bit = fail_bit; pa.tau_bit = tau_bit;
        hipLaunchKernelGGL((potrf_diag_kernel<T>), dim3((unsigned)b), dim3(256), 0, c.s, pa);
        DION_TRY(hipGetLastError());
        if (rest > 0) {
            const int64_t ob = (int64_t)(j0 + nbj) * r + j0, ot = (int64_t)(j0 + nbj) * (r + 1);
            T* below = L + ob;
            // panel: L21 <- S21 Td^T (one column tile covers all nbj columns, so in place is safe)
            GemmArgs g{};
            g.a = Operand{src + ob, nullptr, r, rest, nbj, vr};
            g.b = Operand{Tf + (int64_t)j0 * (r + 1), nullptr, r, nbj, nbj, vr};
            g.sa0 = rr;
            g.sb0 = rr;
            g.c = below; g.ldc = r; g.sc = rr;
            g.M = rest; g.N = nbj; g.K = nbj;
            g.alpha = 1; g.beta = 0;
            g.st = c.st; g.st_mask = mask; g.st_val = val;
            DION_TRY((launch_gemm<T, 64, 64, true, S, true, S>(g, b, c.s)));
            // trailing: L22 <- L22 - L21 L21^T (lower tiles only)
            GemmArgs h = g;
            h.a = Operand{below, nullptr, r, rest, nbj, vr};
            h.b = Operand{below, nullptr, r, rest, nbj, vr};
            h.sb0 = rr;
            h.c = L + ot;
            if (src != L) h.csrc = src + ot;
            h.M = rest; h.N = rest; h.K = nbj;
            h.alpha = -1; h.beta = 1; h.lower = 1;
            DION_TRY((launch_gemm<T, 64, 64, true, S, true, S>(h, b, c.s)));
        }
    }
    return 0;
}

constexpr int64_t kHouseholderMaxRank = 4096;   // the kernel keeps tau and the signs of R in LDS

// Last-resort orthonormalization of the fp64 chain: the thin-QR Q-factor of A (fp64 [m][r] per
// matrix, overwritten by the Householder vectors and R) written to Q, with a positive diagonal of
// R.  It follows the textbook Householder QR (the QR decomposition named in the rivista.ai
// paragraph "Tecnicamente"): for column j, H_j = I - tau_j v_j v_j^T maps A[j:, j] to beta_j e_1
// with v_j[0] = 1 and beta_j = -sign(A[j][j]) ||A[j:, j]||; H_j is applied to the columns to the
// right; then Q = H_0 ... H_{r-1} [I; 0] is accumulated backwards and column j is negated where
// beta_j < 0.  One workgroup per selected matrix, in global memory: this path runs only where the
// CholeskyQR passes broke down (or when requested), so it favors simplicity over speed.  Each
// selected matrix leaves ST_FAIL and gains ST_HH.
__global__ __launch_bounds__(1024) void householder_kernel(double* A, double* Q, int64_t m, int64_t r, int* st,
                                                           int st_mask, int st_val) {
    const int bz = blockIdx.x;
    if ((st[bz] & st_mask) != st_val) return;
    A += bz * m * r;
    Q += bz * m * r;
    constexpr int NT = 1024, RMAX = kHouseholderMaxRank;
    __shared__ double red[NT];
    __shared__ double tau[RMAX];
    __shared__ float sgn[RMAX];
    const int t = threadIdx.x;
    auto block_sum = [&](double v) {
        red[t] = v;
        __syncthreads();
        for (int w = NT / 2; w > 0; w >>= 1) {
            if (t < w) red[t] += red[t + w];
            __syncthreads();
        }
        const double s = red[0];
        __syncthreads();
        return s;
    };
    for (int64_t j = 0; j < r; ++j) {
        const double x0 = A[j * r + j];   // read before the barriers below, after which thread 0 overwrites it
        double ss = 0.0;
        for (int64_t i = j + 1 + t; i < m; i += NT) { const double a = A[i * r + j]; ss += a * a; }
        const double s = block_sum(ss);
        double tj = 0.0, beta = x0;
        if (s > 0.0) {
            const double alpha = sqrt(x0 * x0 + s);
            beta = x0 >= 0.0 ? -alpha : alpha;
            tj = (beta - x0) / beta;
            const double scale = 1.0 / (x0 - beta);
            for (int64_t i = j + 1 + t; i < m; i += NT) A[i * r + j] *= scale;
        }
        if (t == 0) { tau[j] = tj; sgn[j] = beta < 0.0 ? -1.0f : 1.0f; A[j * r + j] = beta; }
        __syncthreads();
        if (tj != 0.0) {   // columns c > j: w = v^T A[j:, c]; A[j:, c] -= tau w v   (v[0] = 1)
            for (int64_t c = j + 1 + t; c < r; c += NT) {
                double w = A[j * r + c];
                for (int64_t i = j + 1; i < m; ++i) w += A[i * r + j] * A[i * r + c];
                w *= tj;
                A[j * r + c] -= w;
                for (int64_t i = j + 1; i < m; ++i) A[i * r + c] -= w * A[i * r + j];
            }
        }
        __syncthreads();
    }
    // Q = H_0 ... H_{r-1} [I; 0], built backwards: after step j only columns >= j are non-trivial
    for (int64_t idx = t; idx < m * r; idx += NT) Q[idx] = (idx / r == idx % r) ? 1.0 : 0.0;
    __syncthreads();
    for (int64_t j = r - 1; j >= 0; --j) {
        const double tj = tau[j];
        if (tj != 0.0) {
            for (int64_t c = j + t; c < r; c += NT) {
                double w = Q[j * r + c];
                for (int64_t i = j + 1; i < m; ++i) w += A[i * r + j] * Q[i * r + c];
                w *= tj;
                Q[j * r + c] -= w;
                for (int64_t i = j + 1; i < m; ++i) Q[i * r + c] -= w * A[i * r + j];
            }
        }
        __syncthreads();
    }
    for (int64_t idx = t; idx < m * r; idx += NT)
        if (sgn[idx % r] < 0.0f) Q[idx] = -Q[idx];
    if (t == 0) st[bz] = (st[bz] & ~ST_FAIL) | ST_HH;
}

// Blocked form of the same Householder QR for ranks above kFusedMaxBlocks * kNB, where the
// one-workgroup column loop above would take seconds per matrix: panels of kHHB columns, each
// factored by one workgroup, the block reflector H_j0 ... H_j0+nb-1 = I - V T V^T kept in compact
// WY form (V unit lower trapezoidal, T upper triangular: T_cc = tau_c and
// T[0:c, c] = -tau_c T[0:c, 0:c] V[:, 0:c]^T v_c), and the columns to the right updated by
// A <- A - V (T^T (V^T A)) as three fp64 matrix-core products.  Q = H_0 ... H_{r-1} [I; 0] is then
// built backwards by Q <- Q - V (T (V^T Q)) over rows and columns from j0 on, and column c of Q
// takes the sign of R_cc.  The same reflectors (and tau, beta) as the column loop.
constexpr int kHHB = 32;

// Panel j0 of matrix bz (grid: matrices; 1024 threads): the reflectors of columns j0 .. j0 + nb - 1,
// applied within the panel; the panel then holds V explicitly (unit diagonal, zeros above), sgn
// the signs of R's diagonal and T (nb x nb, row-major, zeros below) goes to Tp.
__global__ __launch_bounds__(1024) void hh_panel_kernel(double* A, int64_t m, int64_t r, int64_t j0, double* Tp,
                                                        int64_t sT, double* sgn, int64_t ssg, const int* st,
                                                        int st_mask, int st_val) {
    const int bz = blockIdx.x;
    if ((st[bz] & st_mask) != st_val) return;
    A += bz * m * r;
    Tp += bz * sT;
    sgn += bz * ssg;
    constexpr int NT = 1024, NB = kHHB, NRG = NT / NB, U = 4, CH = 128;
    const int nb = (int)((r - j0) < NB ? (r - j0) : NB);
    __shared__ double red[NT / 64];
    __shared__ double tau[NB];
    __shared__ double Y[NB][NB + 1];
    __shared__ double T[NB][NB + 1];
    __shared__ double chunk[CH][NB + 1];
    __shared__ double wred[NRG][NB + 1];
    __shared__ double wv[NB];
    // thread (rg, col): rows rg, rg + 32, ... of panel column col, so that a wave reads two
    // 256-byte row pieces of the panel at a time; U rows of loads in flight per thread
    const int t = threadIdx.x, col = t % NB, rg = t / NB, lane = t & 63, wave = t >> 6;
    auto block_sum = [&](double v) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) red[wave] = v;
        __syncthreads();
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < NT / 64; ++q) s += red[q];
        __syncthreads();
        return s;
    };
    for (int c = 0; c < nb; ++c) {
        const int64_t j = j0 + c;
        const double x0 = A[j * r + j];
        double ss = 0.0;
        for (int64_t i = j + 1 + t; i < m; i += NT) { const double a = A[i * r + j]; ss += a * a; }
        const double s = block_sum(ss);
        double tj = 0.0, beta = x0;
        if (s > 0.0) {
            const double alpha = sqrt(x0 * x0 + s);
            beta = x0 >= 0.0 ? -alpha : alpha;
            tj = (beta - x0) / beta;
            const double scale = 1.0 / (x0 - beta);
            for (int64_t i = j + 1 + t; i < m; i += NT) A[i * r + j] *= scale;
        }
        if (t == 0) { tau[c] = tj; sgn[j] = beta < 0.0 ? -1.0 : 1.0; A[j * r + j] = 1.0; }
        __syncthreads();
        if (tj != 0.0 && c + 1 < nb) {   // panel columns to the right: w = tau v^T a, a -= w v
            const bool act = col > c && col < nb;
            double w = 0.0;
            if (act)
                for (int64_t ib = j + rg; ib < m; ib += U * NRG) {
                    double v[U], a[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int64_t i = ib + u * NRG;
                        v[u] = i < m ? A[i * r + j] : 0.0;
                        a[u] = i < m ? A[i * r + j0 + col] : 0.0;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) w += v[u] * a[u];
                }
            wred[rg][col] = w;
            __syncthreads();
            if (t < NB) {
                double acc = 0.0;
                for (int q = 0; q < NRG; ++q) acc += wred[q][t];
                wv[t] = tj * acc;
            }
            __syncthreads();
            if (act) {
                const double wc = wv[col];
                for (int64_t ib = j + rg; ib < m; ib += U * NRG) {
                    double v[U], a[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int64_t i = ib + u * NRG;
                        v[u] = i < m ? A[i * r + j] : 0.0;
                        a[u] = i < m ? A[i * r + j0 + col] : 0.0;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int64_t i = ib + u * NRG;
                        if (i < m) A[i * r + j0 + col] = a[u] - wc * v[u];
                    }
                }
            }
        }
        __syncthreads();
    }
    // V explicit above the diagonal of the panel's first nb rows
    for (int idx = t; idx < nb * nb; idx += NT) {
        const int rr = idx / nb, cc = idx % nb;
        if (rr < cc) A[(j0 + rr) * r + j0 + cc] = 0.0;
    }
    __syncthreads();
    // Y = V^T V by CH-row chunks through LDS: thread t owns the pair (t / NB, t % NB)
    double y = 0.0;
    const int c1 = t / NB, c2 = t % NB;
    for (int64_t i0 = j0; i0 < m; i0 += CH) {
#pragma unroll
        for (int q = 0; q < CH * NB / NT; ++q) {
            const int idx = t + NT * q, rr = idx / NB, cc = idx % NB;
            chunk[rr][cc] = (i0 + rr < m && cc < nb) ? A[(i0 + rr) * r + j0 + cc] : 0.0;
        }
        __syncthreads();
#pragma unroll 8
        for (int rr = 0; rr < CH; ++rr) y += chunk[rr][c1] * chunk[rr][c2];
        __syncthreads();
    }
    Y[c1][c2] = y;
    T[c1][c2] = 0.0;
    __syncthreads();
    for (int c = 0; c < nb; ++c) {   // column c of T from the columns before it
        if (t < c) {
            double acc = 0.0;
            for (int k = t; k < c; ++k) acc += T[t][k] * Y[k][c];
            T[t][c] = -tau[c] * acc;
        }
        if (t == c) T[c][c] = tau[c];
        __syncthreads();
    }
    Tp[c1 * NB + c2] = (c1 < nb && c2 < nb) ? T[c1][c2] : 0.0;
}

// Q = [I; 0] ([m][r]) for the selected matrices (grid: blocks x matrices).
__global__ __launch_bounds__(256) void hh_init_q_kernel(double* Q, int64_t m, int64_t r, const int* st, int st_mask,
                                                        int st_val) {
    const int bz = blockIdx.y;
    if ((st[bz] & st_mask) != st_val) return;
    Q += bz * m * r;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < m * r; idx += (int64_t)gridDim.x * 256)
        Q[idx] = (idx / r == idx % r) ? 1.0 : 0.0;
}

// Q[:, c] *= sign(R_cc), and the state bits of a finished Householder QR (grid: blocks x matrices).
__global__ __launch_bounds__(256) void hh_finish_kernel(double* Q, const double* sgn, int64_t ssg, int64_t m,
                                                        int64_t r, int* st, int st_mask, int st_val) {
    const int bz = blockIdx.y;
    if ((st[bz] & st_mask) != st_val) return;
    Q += bz * m * r;
    sgn += bz * ssg;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < m * r; idx += (int64_t)gridDim.x * 256)
        if (sgn[idx % r] < 0.0) Q[idx] = -Q[idx];
}

__global__ void hh_done_kernel(int* st, int64_t b, int st_mask, int st_val) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < b && (st[i] & st_mask) == st_val) st[i] = (st[i] & ~ST_FAIL) | ST_HH;
}

// Blocked Householder QR of the selected matrices: A ([b][m][r], overwritten by V) -> Q ([b][m][r]).
// Scratch: the Gram and factor regions hold V^T A and T^T (V^T A) ([nb][r] per matrix), the
// inverse region the panels' T, the column-scale region the signs of diag(R).  Every GEMM runs on
// a fixed, small grid per matrix (launch_gemm_rare), so that the launches cost little when no
// matrix is selected.
static int householder_blocked(const ChainCtx& c, double* A, double* Q, int mask, int val) {
    const Plan& p = *c.p;
    const int64_t m = p.m, r = p.r, b = p.b;
    double* W1 = (double*)(c.ws + p.W);
    double* W2 = (double*)(c.ws + p.L);
    double* Tall = (double*)(c.ws + p.Tf);
    double* sgn = (double*)(c.ws + p.cs);
    const int64_t rr = r * r, srr = rr * 8, smr = m * r * 8;
    const bool vr = (r % 4) == 0;
    constexpr int S = SRC_F64;
    const int64_t npanel = (r + kHHB - 1) / kHHB;
    auto args = [&]() {
        GemmArgs g{};
        g.st = c.st; g.st_mask = mask; g.st_val = val;
        return g;
    };
    // three products per panel j: W1 = V^T X, W2 = op(T) W1, X -= V W2 (X: rows j0.., columns x0..)
    auto reflect = [&](int64_t j0, int nb, const double* Tj, bool transpose_t, double* X, int64_t nx) -> int {
        GemmArgs g = args();
        g.a = Operand{A + j0 * r + j0, nullptr, r, nb, (int)(m - j0), vr};   // V^T (x-contiguous)
        g.b = Operand{X, nullptr, r, (int)nx, (int)(m - j0), vr};
        g.sa0 = smr; g.sb0 = smr;
        g.c = W1; g.ldc = r; g.sc = srr;
        g.M = nb; g.N = (int)nx; g.K = (int)(m - j0);
        g.alpha = 1; g.beta = 0;
        DION_TRY((launch_gemm_rare<double, false, S, false, S>(g, b, c.s)));
        GemmArgs h = args();
        h.a = Operand{Tj, nullptr, kHHB, nb, nb, true};
        h.b = Operand{W1, nullptr, r, (int)nx, nb, vr};
        h.sa0 = srr; h.sb0 = srr;
        h.c = W2; h.ldc = r; h.sc = srr;
        h.M = nb; h.N = (int)nx; h.K = nb;
        h.alpha = 1; h.beta = 0;
        if (transpose_t) DION_TRY((launch_gemm_rare<double, false, S, false, S>(h, b, c.s)));   // T^T: T[k][x]
        else DION_TRY((launch_gemm_rare<double, true, S, false, S>(h, b, c.s)));                // T: T[x][k]
        GemmArgs u = args();
        u.a = Operand{A + j0 * r + j0, nullptr, r, (int)(m - j0), nb, vr};   // V (k-contiguous)
        u.b = Operand{W2, nullptr, r, (int)nx, nb, vr};
        u.sa0 = smr; u.sb0 = srr;
        u.c = X; u.ldc = r; u.sc = smr;
        u.M = (int)(m - j0); u.N = (int)nx; u.K = nb;
        u.alpha = -1; u.beta = 1;
        DION_TRY((launch_gemm_rare<double, true, S, false, S>(u, b, c.s)));
        return 0;
    };
    int e;
    for (int64_t jb = 0; jb < npanel; ++jb) {
        const int64_t j0 = jb * kHHB, nb = (r - j0) < kHHB ? (r - j0) : kHHB, nc = r - j0 - nb;
        double* Tj = Tall + jb * kHHB * kHHB;
        hipLaunchKernelGGL(hh_panel_kernel, dim3((unsigned)b), dim3(1024), 0, c.s, A, m, r, j0, Tj, rr, sgn, r, c.st,
                           mask, val);
        DION_TRY(hipGetLastError());
        if (nc > 0 && (e = reflect(j0, (int)nb, Tj, true, A + j0 * r + j0 + nb, nc))) return e;
    }
    dim3 grid(grid_1d(m * r, 512), (unsigned)b);
    hipLaunchKernelGGL(hh_init_q_kernel, grid, dim3(256), 0, c.s, Q, m, r, c.st, mask, val);
    DION_TRY(hipGetLastError());
    for (int64_t jb = npanel - 1; jb >= 0; --jb) {
        const int64_t j0 = jb * kHHB, nb = (r - j0) < kHHB ? (r - j0) : kHHB;
        if ((e = reflect(j0, (int)nb, Tall + jb * kHHB * kHHB, false, Q + j0 * r + j0, r - j0))) return e;
    }
    hipLaunchKernelGGL(hh_finish_kernel, grid, dim3(256), 0, c.s, Q, (const double*)sgn, r, m, r, c.st, mask, val);
    DION_TRY(hipGetLastError());
    hipLaunchKernelGGL(hh_done_kernel, dim3(grid_1d(b)), dim3(256), 0, c.s, c.st, b, mask, val);
    return (int)hipGetLastError();
}

// st |= bits for the matrices with (st & mask) == val.
__global__ void set_bits_kernel(int* st, int64_t b, int st_mask, int st_val, int bits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < b && (st[i] & st_mask) == st_val) st[i] |= bits;
}

template <typename T>
__global__ __launch_bounds__(256) void copy_pred_kernel(const T* src, T* dst, int64_t total, const int* st,
                                                        int st_mask, int st_val) {
    const int bz = blockIdx.y;
    if ((st[bz] & st_mask) != st_val) return;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256)
        dst[bz * total + idx] = src[bz * total + idx];
}

// ---------------------------------------------------------------------------
// Factor and inverse in one launch, one workgroup per matrix (ranks up to kFusedMaxBlocks
// blocks): L = chol(W (+ s I)) by 64-column blocks (diagonal block with its inverse, panel
// L21 <- L21 Td^T, trailing L22 <- L22 - L21 L21^T, each product a 64 x 64 MFMA tile of the
// workgroup), then Tf = L^-1 by blocked forward substitution,
//   Tf_jj = Td_j,   Tf_ij = -Td_i (sum_{j <= k < i} L_ik Tf_kj).
// Same arithmetic as the multi-launch factor() + invert(), with one launch instead of about
// 3 nblk + 2 log2(nblk) + 2, which matters most on the rarely taken fallback paths (their
// launches are otherwise issued, and return at once, on every step).
// ---------------------------------------------------------------------------
constexpr int kFusedMaxBlocks = 8;
struct CholInvArgs {
    const void* W; void* L; void* Td; void* Tf; void* Y;
    int64_t r, nblk;
    int* st;
    int st_mask, st_val;
    double* kap;
    double tau;
    int fail_bit, tau_bit, shift;
    double c_shift;
    const double* lam;   // shift estimate per matrix (lam[bz * lam_stride]), or null: trace(W)
    int64_t lam_stride;
    // second-pass use: the near-identity partial sums of ||P^T P - I||_F^2 ([b][kNearIdParts],
    // nparts used); a matrix whose norm is <= ntau keeps its first-order T and returns
    const double* npart;
    int nparts;
    double ntau;
};

// C (M x N <= 64 x 64, ldc) = alpha A B + beta C0 with A(i,k) k-contiguous (AKC) or
// row-contiguous, B k-contiguous (BKC) or row-contiguous, and C0 read from Csrc (same layout as
// C) when given, else from C.  All loads of C0 happen before the stores of C, and the workgroup
// synchronizes at the end (C is read back by the next tile).  Operands and C may sit in LDS.
template <typename T, bool BKC, bool AKC = true>
__device__ void tile_gemm(const Operand& A, const Operand& B, int M, int N, int K, T* Cp, int64_t ldc, T alpha,
                          T beta, T* As, T* Bs, const T* Csrc = nullptr) {
    using C = TileCfg<T, 64, 64, sizeof(T) == 8 ? 16 : 32>;
    constexpr int S = SrcOf<T>::v;
    typename C::acc_t acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::acc_t{0, 0, 0, 0};
    mainloop<T, C, AKC, S, BKC, S>(A, B, 0, 0, 0, K, As, Bs, acc);
    const T* C0 = Csrc ? Csrc : Cp;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
    T sv[C::FM][C::FN][4];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = wm * C::WTM + i * 16 + Mfma<T>::row(lane, v), col = wn * C::WTN + j * 16 + (lane & 15);
                sv[i][j][v] = (beta != T(0) && row < M && col < N) ? C0[(int64_t)row * ldc + col] : T(0);
            }
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = wm * C::WTM + i * 16 + Mfma<T>::row(lane, v), col = wn * C::WTN + j * 16 + (lane & 15);
                if (row < M && col < N) Cp[(int64_t)row * ldc + col] = alpha * acc[i][j][v] + beta * sv[i][j][v];
            }
    __syncthreads();
}

// Step jb of the right-looking factorization with L^-1 built alongside, in one launch (grid:
// tasks x matrices), for ranks up to kFusedMaxBlocks blocks.  Tasks 0 .. ntr - 1 are the trailing
// tiles (i, k), jb < k <= i, column by column; each computes the panel blocks it needs itself,
//   L_i,jb = S_i,jb Td_jb^T,   L_k,jb = S_k,jb Td_jb^T   (S: W at the first unshifted step, else L)
//   L_ik   = S_ik - L_i,jb L_k,jb^T,
// so the panel needs no launch of its own.  The tiles of column jb + 1 keep L_i,jb, transposed,
// in the upper block (jb, i) of L, which the factorization leaves unused (writing it in place
// would race with the other tiles still reading S_i,jb).  Task 0, tile (jb + 1, jb + 1), then
// factors and inverts that diagonal block (as potrf_diag_kernel does).  The last jb tasks are the
// inverse tiles of block row jb,
//   X_jb,kb = -Td_jb (sum_{kb <= q < jb} L_jb,q X_q,kb),   kb < jb,
// which read L_jb,q from the upper blocks (q, jb) kept by earlier steps.  The step after the last
// diagonal block (jb = nblk - 1) has inverse tiles only.
// One thread's sixteen elements of a 64 x 64 block (rows < nr, columns < nc of a row-major array
// of pitch ld; zero elsewhere): the loads are issued together (addresses clamped, values selected
// afterwards) and stored to an LDS block of pitch kDLD later, transposed if asked.
template <typename T>
struct BlkRegs {
    T v[kNB * kNB / 256];
    __device__ __forceinline__ void fetch(const T* src, int64_t ld, int nr, int nc) {
        const int i0 = threadIdx.x >> 6, j = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < kNB * kNB / 256; ++q) {
            const int i = i0 + 4 * q;
            v[q] = src[(i < nr && j < nc) ? (int64_t)i * ld + j : 0];
        }
#pragma unroll
        for (int q = 0; q < kNB * kNB / 256; ++q) v[q] = (i0 + 4 * q < nr && j < nc) ? v[q] : T(0);
    }
    __device__ __forceinline__ void put(T* dst, bool trans) const {
        const int i0 = threadIdx.x >> 6, j = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < kNB * kNB / 256; ++q) dst[trans ? j * kDLD + i0 + 4 * q : (i0 + 4 * q) * kDLD + j] = v[q];
    }
};

// acc += A B^T for the calling wave's four 16 x 16 output blocks (row block `wave`, column blocks
// 0..3) of a 64 x 64 product of LDS blocks (pitch kDLD): C(i, j) = sum_k A[i][k] B[j][k], K a
// multiple of 16 (zero padded).
template <typename T>
__device__ __forceinline__ void blk_abt(const T* A, const T* B, int K, typename Mfma<T>::acc_t (&acc)[4], int wave,
                                        int lane) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) blk_mma<T>(&A[16 * wave * kDLD], kDLD, 1, &B[16 * jb * kDLD], 1, kDLD, K, acc[jb], lane);
}

template <typename T>
__global__ __launch_bounds__(256) void chol_step_kernel(CholStepArgs a) {
    const int bz = blockIdx.y, t = blockIdx.x;
    if ((a.st[bz] & a.st_mask) != a.st_val) return;
    using acc_t = typename Mfma<T>::acc_t;
    __shared__ DiagSmem<T> sm;
    __shared__ T bp[kNB * kDLD];
    __shared__ T bq[kNB * kDLD];
    const int64_t r = a.r, rr = r * r;
    const T* S = (const T*)a.S + bz * rr;
    T* L = (T*)a.L + bz * rr;
    T* Tf = (T*)a.Tf + bz * rr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, fr = lane & 15;
    auto nb = [&](int q) { return (int)((r - (int64_t)q * kNB) < kNB ? (r - (int64_t)q * kNB) : kNB); };
    const int jb = a.jb, j0 = jb * kNB, nbj = nb(jb), n = a.nblk - 1 - jb, ntr = n * (n + 1) / 2;
    const int K16 = (nbj + 15) / 16 * 16;
    const T* Td = Tf + (int64_t)j0 * (r + 1);   // X_jb,jb (lower; zero above its diagonal)
    acc_t acc[4];
    auto zero = [&]() {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = acc_t{0, 0, 0, 0};
    };
    // the calling thread's elements of the wave's output blocks: (row, col, value)
    auto each = [&](auto f) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) f(16 * wave + Mfma<T>::row(lane, v), 16 * q + fr, acc[q][v]);
    };
    if (t < ntr) {
        int k = jb + 1, rem = t;
        while (rem >= a.nblk - k) { rem -= a.nblk - k; ++k; }
        const int i = k + rem;
        const int64_t i0 = (int64_t)i * kNB, k0 = (int64_t)k * kNB;
        const int nbi = nb(i), nbk = nb(k);
        // every load of the task in flight at once: Td, S_i,jb, S_k,jb and S_ik (the last in the
        // accumulator layout of the update)
        BlkRegs<T> rt, ri, rk;
        rt.fetch(Td, r, nbj, nbj);
        ri.fetch(S + i0 * r + j0, r, nbi, nbj);
        if (k != i) rk.fetch(S + k0 * r + j0, r, nbk, nbj);
        const T* Sik = S + i0 * r + k0;
        T sv[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * wave + Mfma<T>::row(lane, v), col = 16 * q + fr;
                sv[q][v] = Sik[(row < nbi && col < nbk) ? (int64_t)row * r + col : 0];
            }
        rt.put(bq, false);
        ri.put(bp, false);
        if (k != i) rk.put(sm.x, false);
        __syncthreads();
        // L_i,jb = S_i,jb Td^T into sm.a; L_k,jb = S_k,jb Td^T into bp
        zero();
        blk_abt<T>(bp, bq, K16, acc, wave, lane);
        if (k != i) {
            acc_t ak[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) ak[q] = acc_t{0, 0, 0, 0};
            blk_abt<T>(sm.x, bq, K16, ak, wave, lane);
            __syncthreads();   // bp is free
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) bp[(16 * wave + Mfma<T>::row(lane, v)) * kDLD + 16 * q + fr] = ak[q][v];
        }
        each([&](int row, int col, T v) { sm.a[row * kDLD + col] = v; });
        const T* Lk = k != i ? bp : sm.a;
        __syncthreads();
        if (k == jb + 1)   // this tile's row block keeps L_i,jb, transposed, in the upper block (jb, i)
            for (int idx = threadIdx.x; idx < nbj * nbi; idx += 256) {
                const int u = idx / nbi, v = idx % nbi;
                L[(int64_t)(j0 + u) * r + i0 + v] = sm.a[v * kDLD + u];
            }
        // L_ik = S_ik - L_i,jb L_k,jb^T
        zero();
        blk_abt<T>(sm.a, Lk, K16, acc, wave, lane);
        if (t != 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 16 * wave + Mfma<T>::row(lane, v), col = 16 * q + fr;
                    if (row < nbi && col < nbk) L[(i0 + row) * r + k0 + col] = sv[q][v] - acc[q][v];
                }
            return;
        }
        // tile (jb + 1, jb + 1): the updated block goes straight into the diagonal factorization
        __syncthreads();   // every wave is done reading sm.a
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * wave + Mfma<T>::row(lane, v), col = 16 * q + fr;
                sm.a[row * kDLD + col] = (row < nbk && col <= row) ? sv[q][v] - acc[q][v] : (row == col ? T(1) : T(0));
            }
        __syncthreads();
        diag_factor<T>(a.diag, bz, sm);
        return;
    }
    // inverse tile X_jb,kb = -Td (sum_{kb <= q < jb} L_jb,q X_q,kb), kb = t - ntr; A = L_jb,q (kept
    // transposed in the upper block (q, jb)), B = X_q,kb^T; the next pair is fetched during a product
    const int kb = t - ntr, k0 = kb * kNB, nbk = nb(kb);
    BlkRegs<T> ra, rb, rt;
    ra.fetch(L + (int64_t)kb * kNB * r + j0, r, kNB, nbj);
    rb.fetch(Tf + (int64_t)kb * kNB * r + k0, r, kNB, nbk);
    rt.fetch(Td, r, nbj, nbj);
    zero();
    for (int q = kb; q < jb; ++q) {
        ra.put(bp, true);
        rb.put(bq, true);
        __syncthreads();
        if (q + 1 < jb) {
            ra.fetch(L + (int64_t)(q + 1) * kNB * r + j0, r, kNB, nbj);
            rb.fetch(Tf + (int64_t)(q + 1) * kNB * r + k0, r, kNB, nbk);
        }
        blk_abt<T>(bp, bq, kNB, acc, wave, lane);
        __syncthreads();
    }
    // Y^T into bp, Td into bq; X_jb,kb = -Td Y
    each([&](int row, int col, T v) { bp[col * kDLD + row] = v; });
    rt.put(bq, false);
    __syncthreads();
    zero();
    blk_abt<T>(bq, bp, K16, acc, wave, lane);
    each([&](int row, int col, T v) {
        if (row < nbj && col < nbk) Tf[(int64_t)(j0 + row) * r + k0 + col] = -v;
    });
}

template <typename T>
__global__ __launch_bounds__(256) void cholinv_kernel(CholInvArgs a) {
    const int bz = blockIdx.x;
    if ((a.st[bz] & a.st_mask) != a.st_val) return;
    using C = TileCfg<T, 64, 64, sizeof(T) == 8 ? 16 : 32>;
    __shared__ DiagSmem<T> sm;
    __shared__ T As[2 * C::A_STAGE];
    __shared__ T Bs[2 * C::B_STAGE];
    __shared__ double red[256];
    if (a.npart) {   // the regime test of the second pass, partial sums added by a fixed tree
        red[threadIdx.x] = (int)threadIdx.x < a.nparts ? a.npart[(int64_t)bz * kNearIdParts + threadIdx.x] : 0.0;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        const double e = sqrt(red[0]);
        __syncthreads();
        if (e <= a.ntau) return;   // first-order: T = I - Phi(E) is already in place (not finite: go on)
    }
    const int64_t r = a.r, rr = r * r, nblk = a.nblk;
    const T* W = (const T*)a.W + bz * rr;
    T* L = (T*)a.L + bz * rr;
    T* Tf = (T*)a.Tf + bz * rr;
    T* Y = (T*)a.Y + bz * rr;
    T* Td = (T*)a.Td + bz * nblk * kNB * kNB;
    const bool vr = (r % 4) == 0;
    // L = W (+ s I), s = c_shift lambda_hat (the estimate, when given) or c_shift trace(W)
    T sv = T(0);
    if (a.shift && a.lam) {
        sv = (T)(a.c_shift * a.lam[bz * a.lam_stride]);
    } else if (a.shift) {
        double tr = 0;
        for (int64_t i = threadIdx.x; i < r; i += 256) tr += (double)W[i * r + i];
        red[threadIdx.x] = tr;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        sv = (T)(a.c_shift * red[0]);
    }
    for (int64_t idx = threadIdx.x; idx < rr; idx += 256) {
        const int64_t i = idx / r, k = idx % r;
        L[idx] = W[idx] + ((i == k) ? sv : T(0));
    }
    __syncthreads();
    auto nb = [&](int64_t jb) { return (int)((r - jb * kNB) < kNB ? (r - jb * kNB) : kNB); };
    for (int64_t jb = 0; jb < nblk; ++jb) {
        PotrfArgs pa{};
        pa.L = a.L; pa.ldl = r; pa.sL = rr; pa.S = a.L;
        pa.Td = a.Td; pa.sTd = nblk * kNB * kNB; pa.ldTd = kNB; pa.blkTd = kNB * kNB; pa.tdfull = 1;
        pa.j0 = (int)(jb * kNB); pa.nbj = nb(jb); pa.jblk = (int)jb;
        pa.st = a.st; pa.kap = a.kap;
        pa.first = jb == 0; pa.last = jb == nblk - 1;
        pa.tau = a.tau; pa.fail_bit = a.fail_bit; pa.tau_bit = a.tau_bit;
        if (!diag_block<T>(pa, bz, sm)) return;
        __syncthreads();
        const int nbj = nb(jb);
        for (int64_t ib = jb + 1; ib < nblk; ++ib) {          // panel
            T* tile = L + ib * kNB * r + jb * kNB;
            const Operand A{tile, nullptr, r, nb(ib), nbj, vr};
            const Operand B{Td + jb * kNB * kNB, nullptr, kNB, nbj, nbj, true};
            tile_gemm<T, true>(A, B, nb(ib), nbj, nbj, tile, r, T(1), T(0), As, Bs);
        }
        for (int64_t kb = jb + 1; kb < nblk; ++kb)            // trailing, lower tiles
            for (int64_t ib = kb; ib < nblk; ++ib) {
                const Operand A{L + ib * kNB * r + jb * kNB, nullptr, r, nb(ib), nbj, vr};
                const Operand B{L + kb * kNB * r + jb * kNB, nullptr, r, nb(kb), nbj, vr};
                tile_gemm<T, true>(A, B, nb(ib), nb(kb), nbj, L + ib * kNB * r + kb * kNB, r, T(-1), T(1), As, Bs);
            }
    }
    __syncthreads();                                          // the state word written by thread 0
    if (a.tau_bit && (a.st[bz] & a.tau_bit)) return;          // refactored shifted: no inverse needed
    // Tf = L^-1: diagonal blocks from Td, zero above, then the blocks below by rows of blocks
    for (int64_t idx = threadIdx.x; idx < rr; idx += 256) {
        const int64_t i = idx / r, k = idx % r, bi = i / kNB, bk = k / kNB;
        Tf[idx] = (bi == bk) ? Td[(bi * kNB + (i % kNB)) * kNB + (k % kNB)] : T(0);
    }
    __syncthreads();
    for (int64_t ib = 1; ib < nblk; ++ib)
        for (int64_t jb = 0; jb < ib; ++jb) {
            const int K = (int)((ib - jb) * kNB);
            // Y = sum_{jb <= k < ib} L[ib][k] Tf[k][jb]   (64 x nb(jb), ld 64)
            const Operand A{L + ib * kNB * r + jb * kNB, nullptr, r, nb(ib), K, vr};
            const Operand B{Tf + jb * kNB * r + jb * kNB, nullptr, r, nb(jb), K, vr};
            tile_gemm<T, false>(A, B, nb(ib), nb(jb), K, Y, kNB, T(1), T(0), As, Bs);
            // Tf[ib][jb] = -Td_ib Y
            const Operand A2{Td + ib * kNB * kNB, nullptr, kNB, nb(ib), nb(ib), true};
            const Operand B2{Y, nullptr, kNB, nb(jb), nb(ib), (rr % 4) == 0};
            tile_gemm<T, false>(A2, B2, nb(ib), nb(jb), nb(ib), Tf + ib * kNB * r + jb * kNB, r, T(-1), T(0), As,
                                Bs);
        }
}

// factor + invert for the matrices with (st & mask) == val
template <typename T>
static int factor_invert(const ChainCtx& c, int mask, int val, double tau, int fail_bit, int tau_bit, int shift,
                         bool rare, const double* npart = nullptr, int nparts = 0, double ntau = 0.0);

// Tf = L^-1 (lower, [b][r][r]) from the factor L and the inverted diagonal blocks already in
// Tf, by recursive doubling over the blocks: for neighbouring block ranges U (above) and V
// (below) whose inverses are known, T_VU = -T_VV (L_VU T_UU).  log2(nblk) levels of two batched
// GEMMs; the product L_VU T_UU is parked in W (free once the factor is accepted).
template <typename T>
static int invert(const ChainCtx& c, int mask, int val) {
    const Plan& p = *c.p;
    const int64_t r = p.r, b = p.b;
    const T* L = (const T*)(c.ws + p.L);
    T* Tf = (T*)(c.ws + p.Tf);
    T* Y = (T*)(c.ws + p.W);
    constexpr int S = SrcOf<T>::v;
    const bool vr = (r % 4) == 0;
    const int64_t rr = r * r * (int64_t)sizeof(T);
    for (int64_t s = 1; s < p.nblk; s *= 2) {
        const int64_t span = 2 * s * kNB;               // rows/cols of one group
        const int64_t gfull = r / span;                 // groups with U and V entirely inside r
        // (U0, V0, |U|, |V|, number of groups) for the full groups and the trailing partial one
        struct Part { int64_t u0, nu, nv, ng; } parts[2];
        int np = 0;
        if (gfull > 0) parts[np++] = Part{0, s * kNB, s * kNB, gfull};
        const int64_t u0 = gfull * span;
        if (u0 + s * kNB < r) parts[np++] = Part{u0, s * kNB, r - (u0 + s * kNB), 1};
        for (int q = 0; q < np; ++q) {
            const Part& pt = parts[q];
            const int64_t v0 = pt.u0 + pt.nu;
            const int64_t gstep = span * (r + 1) * (int64_t)sizeof(T);
            // Y = L_VU T_UU   (T_UU lower: only k >= n contributes)
            GemmArgs g{};
            g.a = Operand{L + v0 * r + pt.u0, nullptr, r, (int)pt.nv, (int)pt.nu, vr};
            g.b = Operand{Tf + pt.u0 * r + pt.u0, nullptr, r, (int)pt.nu, (int)pt.nu, vr};
            g.sa0 = g.sb0 = g.sc = rr;
            g.ga0 = g.gb0 = g.gc = gstep;
            g.zdiv = (int)pt.ng;
            g.c = Y + v0 * r + pt.u0; g.ldc = r;
            g.M = (int)pt.nv; g.N = (int)pt.nu; g.K = (int)pt.nu;
            g.alpha = 1; g.beta = 0; g.kskip = 2;
            g.st = c.st; g.st_mask = mask; g.st_val = val;
            DION_TRY((launch_gemm<T, 64, 64, true, S, false, S>(g, b, c.s)));
            // T_VU = -T_VV Y   (T_VV lower: only k <= i contributes)
            GemmArgs h = g;
            h.a = Operand{Tf + v0 * r + v0, nullptr, r, (int)pt.nv, (int)pt.nv, vr};
            h.b = Operand{Y + v0 * r + pt.u0, nullptr, r, (int)pt.nu, (int)pt.nv, vr};
            h.c = Tf + v0 * r + pt.u0;
            h.K = (int)pt.nv;
            h.alpha = -1; h.kskip = 3;
            DION_TRY((launch_gemm<T, 64, 64, true, S, false, S>(h, b, c.s)));
        }
    }
    return 0;
}

// `rare`: a fallback path that usually has no matrix to work on, where one launch (instead of
// about 15 that return at once) is what counts; the common paths keep the multi-launch
// factorization, which spreads the panel and trailing products over many CUs.
template <typename T>
static int factor_invert(const ChainCtx& c, int mask, int val, double tau, int fail_bit, int tau_bit, int shift,
                         bool rare, const double* npart, int nparts, double ntau) {
    const Plan& p = *c.p;
    if (!rare || p.nblk > kFusedMaxBlocks) {
        int e;
        const bool inv = p.nblk <= kFusedMaxBlocks;   // L^-1 built alongside the factorization
        if ((e = factor<T>(c, mask, val, tau, fail_bit, tau_bit, shift, inv))) return e;
        if (inv) return 0;
        // a matrix marked by tau_bit here is refactored (shifted) by a later call, which inverts
        return invert<T>(c, tau_bit ? (mask | tau_bit) : mask, val);
    }
    CholInvArgs a{};
    a.W = c.ws + p.W; a.L = c.ws + p.L; a.Td = c.ws + p.Td; a.Tf = c.ws + p.Tf; a.Y = c.ws + p.W;
    a.r = p.r; a.nblk = p.nblk;
    a.st = c.st; a.st_mask = mask; a.st_val = val;
    a.kap = (double*)(c.ws + p.kap);
    a.tau = tau; a.fail_bit = fail_bit; a.tau_bit = tau_bit; a.shift = shift;
    const double u = sizeof(T) == 8 ? 1.1102230246251565e-16 : 5.9604644775390625e-08;
    a.c_shift = 11.0 * ((double)p.m * p.r + (double)p.r * (p.r + 1)) * u;
    a.lam = c.lam; a.lam_stride = c.lam_stride;
    a.npart = npart; a.nparts = nparts; a.ntau = ntau;
    hipLaunchKernelGGL((cholinv_kernel<T>), dim3((unsigned)p.b), dim3(256), 0, c.s, a);
    return (int)hipGetLastError();
}

// Pout = Pin Tf^T = Pin L^-T  (Tf lower: output column tile n0 needs only k < n0 + BN)
template <typename T>
static int apply(const ChainCtx& c, const T* Pin, T* Pout, int mask, int val) {
    if constexpr (sizeof(T) == 4 && DION_PROD6) return apply6(c, Pin, Pout, mask, val);
    const Plan& p = *c.p;
    const int64_t m = p.m, r = p.r;
    constexpr int S = SrcOf<T>::v;
    const bool vr = (r % 4) == 0;
    GemmArgs g{};
    g.a = Operand{Pin, nullptr, r, (int)m, (int)r, vr};                     // A(i,k) = Pin[i][k]
    g.b = Operand{c.ws + p.Tf, nullptr, r, (int)r, (int)r, vr};             // B(k,j) = Tf[j][k]
    g.sa0 = m * r * (int64_t)sizeof(T);
    g.sb0 = r * r * (int64_t)sizeof(T);
    g.c = Pout; g.ldc = r; g.sc = m * r * (int64_t)sizeof(T);
    g.M = (int)m; g.N = (int)r; g.K = (int)r;
    g.alpha = 1; g.beta = 0; g.kskip = 1;
    g.st = c.st; g.st_mask = mask; g.st_val = val;
    DION_TRY((launch_gemm<T, 64, 64, true, S, true, S>(g, p.b, c.s)));
    return 0;
}

// One CholeskyQR pass Pin -> Pout: W = Pin^T Pin, L = chol(W), Pout = Pin L^-T.
template <typename T>
static int cholqr_pass(const ChainCtx& c, const T* Pin, T* Pout, int mask, int val, double tau, int fail_bit,
                       int tau_bit) {
    int e;
    if ((e = gram<T>(c, Pin, mask, val))) return e;
    if ((e = factor_invert<T>(c, mask, val, tau, fail_bit, tau_bit, 0, false))) return e;
    return apply<T>(c, Pin, Pout, mask, val);
}

// Re-orthonormalization of a nearly orthonormal P1 (the second CholeskyQR pass) without a
// sequential factorization.  With W = P1^T P1 = I + E and chol(W) = I + F, F lower triangular,
// F + F^T + F F^T = E, so F = Phi(E) + O(eps^2), where Phi keeps the strictly lower part and half
// the diagonal and eps = ||E||_F (>= ||E||_2).  Then (I + F)^-1 = I - F + O(eps^2), and
// P = P1 (I + F)^-T = P1 (I - Phi(E))^T with error O(eps^2).  Per matrix, decided on the device:
//   eps <= tau:               T = I - Phi(E)          (error <= ~eps^2)
//   eps > tau, or not finite: T = L^-1 of the blocked Cholesky pass              [ST_CHOL2]
// and one apply P = P1 T^T serves both.
// Setup of a re-orthonormalization pass (grid: parts x matrices): W = the sum of the split-K
// Gram partials in split order (when the Gram was split; lower triangle), T = I - Phi(E) with
// E = W - I, and per workgroup the sum of squares of E over its share.  (A last-arriving
// workgroup could decide in place, but its device-scope fence writes back the L2 of every XCD;
// a separate launch is cheaper.)
template <typename T>
__global__ __launch_bounds__(256) void near_id_setup_kernel(const T* gpart, int64_t splits, T* W, T* Tm,
                                                            double* part, int64_t r, const int* st, int st_mask,
                                                            int st_val) {
    const int bz = blockIdx.y;
    if ((st[bz] & st_mask) != st_val) return;
    const int64_t total = r * r;
    W += bz * total;
    Tm += bz * total;
    if (gpart) gpart += bz * splits * total;
    double ss = 0.0;   // sum of squares of E over the full symmetric matrix
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        const int64_t i = idx / r, k = idx % r;
        T v = T(0);
        if (k <= i) {
            T w;
            if (gpart) {
                w = 0;
                for (int64_t q = 0; q < splits; ++q) w += gpart[q * total + idx];
                W[idx] = w;
            } else {
                w = W[idx];
            }
            const T e = w - (i == k ? T(1) : T(0));
            const double d = (double)e;
            ss += (i == k ? 1.0 : 2.0) * d * d;
            v = (i == k) ? T(1) - T(0.5) * e : -e;
        }
        Tm[idx] = v;
    }
    __shared__ double red[256];
    red[threadIdx.x] = ss;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[(int64_t)bz * kNearIdParts + blockIdx.x] = red[0];
}

// Regime bit of each selected matrix from ||E||_F, the partial sums added in part order.
__global__ void near_id_decide_kernel(const double* part, int nparts, int* st, int64_t b, int st_mask, int st_val,
                                      double tau) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= b || (st[i] & st_mask) != st_val) return;
    double ss = 0.0;
    for (int q = 0; q < nparts; ++q) ss += part[i * kNearIdParts + q];
    const double e = sqrt(ss);
    st[i] = (e <= tau) ? (st[i] & ~ST_CHOL2) : (st[i] | ST_CHOL2);   // not finite: Cholesky
}

template <typename T>
static int reortho_pass(const ChainCtx& c, const T* Pin, T* Pout, int mask, int val, double tau, int fail_bit) {
    const Plan& p = *c.p;
    const int64_t r = p.r, b = p.b;
    T* W = (T*)(c.ws + p.W);
    double* part = (double*)(c.ws + p.emax);
    const double tau_re = sizeof(T) == 8 ? kTauRe64 : kTauRe32;
    int e;
    if ((e = gram<T>(c, Pin, mask, val, false))) return e;
    {
        // about 2048 workgroups over the stack (the split partials are summed here), at most
        // kNearIdParts per matrix
        const int64_t per = std::min<int64_t>(kNearIdParts, std::max<int64_t>(16, (2048 + b - 1) / b));
        const unsigned nparts = grid_1d(r * r, per);
        dim3 grid(nparts, (unsigned)b);
        const int64_t splits = gram_splits<T>(p);
        const T* gp = splits > 1 ? (const T*)(c.ws + p.gpart) : nullptr;
        hipLaunchKernelGGL((near_id_setup_kernel<T>), grid, dim3(256), 0, c.s, gp, splits, W, (T*)(c.ws + p.Tf),
                           part, r, (const int*)c.st, mask, val);
        DION_TRY(hipGetLastError());
        if (p.nblk <= kFusedMaxBlocks) {
            // matrices far from orthonormal: a full Cholesky pass (W is untouched), T = L^-1, in
            // the fused factorization, which makes the regime test itself
            if ((e = factor_invert<T>(c, mask, val, tau_re, fail_bit, fail_bit, 0, true, part, (int)nparts, tau)))
                return e;
            return apply<T>(c, Pin, Pout, mask, val);
        }
        hipLaunchKernelGGL(near_id_decide_kernel, dim3(grid_1d(b)), dim3(256), 0, c.s, (const double*)part,
                           (int)nparts, c.st, b, mask, val, tau);
        DION_TRY(hipGetLastError());
    }
    const int cmask = mask | ST_CHOL2, cval = val | ST_CHOL2;
    if ((e = factor_invert<T>(c, cmask, cval, tau_re, fail_bit, fail_bit, 0, true))) return e;
    return apply<T>(c, Pin, Pout, mask, val);
}

// ---------------------------------------------------------------------------
// fp32-chain products on the bf16 matrix cores (six-term split, fp32 accuracy; bf16x6.hpp):
// C[M x N] = A B per matrix, with A and B read as split-bf16 operand tiles.  128 x 128 tiles,
// four multiplying waves of 64 x 64 (so each LDS fragment feeds four MFMA blocks) and four
// staging waves, triple-buffered part tiles in 144 KB of LDS: one workgroup per CU.
// ---------------------------------------------------------------------------
struct Prod6Args {
    Op6 a, b;
    int64_t sa0, sa1, sb0;       // batch strides in bytes of a.p0, a.p1, b.p0
    float* c;
    int64_t ldc, sc;             // sc in elements
    int M, N, K;
    const int* st;
    int st_mask, st_val;
    // split K: grid z = matrix * splits + split; split s covers k in [s kc, min(K, (s + 1) kc)),
    // its operands start ska / ska1 / skb bytes further (a.p0, a.p1, b.p0) and its output slice
    // scs elements further
    int splits;
    int64_t kc, ska, ska1, skb, scs;
    bool lower;                  // square output: tiles entirely above the diagonal are skipped
    bool tri;                    // B(k, j) = 0 for k > j: output column tile n0 stops at k = n0 + 128
};

// Staging side of prod6_kernel: three register sets of raw operand values and three LDS buffers,
// both indexed by slab % 3, so a slab's global loads are issued three slabs before it is split
// (enough bytes in flight per CU to cover the memory latency at the matrix-core rate).
template <int AK, int AADD, int BK6, int NT, int NP>
struct Stage6 {
    static constexpr int BT = 128, PT = BT * kSplitK, D = 3;
    Loader6<BT, AK, AADD, NT> la[D];
    Loader6<BT, BK6, A6_NONE, NT> lb[D];
    template <int J>
    __device__ __forceinline__ void load(const Op6& A, const Op6& B, int m0, int n0, int k, int K, int t) {
        if (k < K) { la[J].load(A, m0, k, t); lb[J].load(B, n0, k, t); }
    }
    // slab at k (held in set J) -> LDS buffer J; set J then loads the slab D slabs later
    template <int J>
    __device__ __forceinline__ void stage(const Op6& A, const Op6& B, int m0, int n0, int k, int K, uint16_t* lds,
                                          int t) {
        la[J].template split_store<NP>(lds, t);
        lb[J].template split_store<NP>(lds + NP * PT, t);
        load<J>(A, B, m0, n0, k + D * kSplitK, K, t);
    }
    // Launches whose tiles are all interior (every slab whole and inside both operands) use the
    // same steps without bounds tests, so the compiler waits only for the set a store consumes.
    template <int J>
    __device__ __forceinline__ void load_fast(const Op6& A, const Op6& B, int m0, int n0, int k, int t) {
        la[J].load_fast(A, m0, k, t);
        lb[J].load_fast(B, n0, k, t);
    }
    template <int J>
    __device__ __forceinline__ void stage_fast(const Op6& A, const Op6& B, int m0, int n0, int knext, uint16_t* lds,
                                               int t) {
        la[J].template split_store<NP>(lds, t);
        lb[J].template split_store<NP>(lds + NP * PT, t);
        load_fast<J>(A, B, m0, n0, knext, t);
    }
    template <int J>
    __device__ __forceinline__ void stage_fast_if(const Op6& A, const Op6& B, int m0, int n0, int knext, int K,
                                                  uint16_t* lds, int t) {
        la[J].template split_store<NP>(lds, t);
        lb[J].template split_store<NP>(lds + NP * PT, t);
        if (knext < K) load_fast<J>(A, B, m0, n0, knext, t);
    }
};

template <int AK, int AADD, int BK6, bool FAST, int NT, int NP>
__global__ __launch_bounds__(256 + NT) void prod6_kernel(Prod6Args g) {
    // Waves 0-3 multiply (a 64 x 64 sub-tile each); the NT / 64 waves after them stage the
    // operands (load, split into bf16 parts, write LDS).  Each SIMD holds one multiplying wave and
    // NT / 256 staging waves, so the staging work issues between the other wave's MFMAs; one
    // barrier per slab.
    using St = Stage6<AK, AADD, BK6, NT, NP>;
    constexpr int BT = St::BT, PT = St::PT;
    const TileId tid = xcd_tile_id();
    const int sp = g.splits > 1 ? g.splits : 1, bz = tid.z / sp, ks = tid.z % sp;
    if (g.st && (g.st[bz] & g.st_mask) != g.st_val) return;
    if (g.lower && tid.x > tid.y) return;
    const int m0 = tid.y * BT, n0 = tid.x * BT;
    __shared__ __attribute__((aligned(16))) uint16_t lds[3][2 * NP * PT];   // A parts | B parts
    const int wave = threadIdx.x >> 6;
    const bool stager = wave >= 4;
    const int st_t = threadIdx.x - 256;
    Op6 A = g.a, B = g.b;
    A.p0 = (const char*)A.p0 + bz * g.sa0;
    if (A.p1) A.p1 = (const char*)A.p1 + bz * g.sa1;
    B.p0 = (const char*)B.p0 + bz * g.sb0;
    int K = g.K;
    if (sp > 1) {
        A.p0 = (const char*)A.p0 + ks * g.ska;
        if (A.p1) A.p1 = (const char*)A.p1 + ks * g.ska1;
        B.p0 = (const char*)B.p0 + ks * g.skb;
        K = (int)(g.kc < (int64_t)g.K - ks * g.kc ? g.kc : (int64_t)g.K - ks * g.kc);
        A.kext = K;
        B.kext = K;
    }
    if (g.tri && n0 + BT < K) K = n0 + BT;
    // slab s is multiplied from LDS buffer s % 3 while the staging waves write slab s + 2 to
    // buffer (s + 2) % 3 and issue the loads of slab s + 5.  The two roles run separate loops
    // with the same barriers, so their registers (raw slabs, accumulators) never overlap.
    if (stager) {
        St sg;
        if constexpr (FAST) {
            // every tile interior, K a multiple of the slab and at least three slabs.  Steady
            // state: buffers 0, 1 hold slabs s, s + 1; register sets 2, 0, 1 hold s + 2 .. s + 4.
            const int nslab = K / kSplitK;
            sg.template load_fast<0>(A, B, m0, n0, 0, st_t);
            sg.template load_fast<1>(A, B, m0, n0, kSplitK, st_t);
            sg.template load_fast<2>(A, B, m0, n0, 2 * kSplitK, st_t);
            sg.template stage_fast_if<0>(A, B, m0, n0, 3 * kSplitK, K, lds[0], st_t);
            sg.template stage_fast_if<1>(A, B, m0, n0, 4 * kSplitK, K, lds[1], st_t);
            __syncthreads();
            int s = 0;
            for (; s + 8 <= nslab; s += 3) {
                sg.template stage_fast<2>(A, B, m0, n0, (s + 5) * kSplitK, lds[2], st_t);
                __syncthreads();
                sg.template stage_fast<0>(A, B, m0, n0, (s + 6) * kSplitK, lds[0], st_t);
                __syncthreads();
                sg.template stage_fast<1>(A, B, m0, n0, (s + 7) * kSplitK, lds[1], st_t);
                __syncthreads();
            }
            for (int k0 = s * kSplitK; k0 < K; k0 += 3 * kSplitK) {
                if (k0 + 2 * kSplitK < K) sg.template stage_fast_if<2>(A, B, m0, n0, k0 + 5 * kSplitK, K, lds[2], st_t);
                __syncthreads();
                if (k0 + kSplitK >= K) break;
                if (k0 + 3 * kSplitK < K) sg.template stage_fast_if<0>(A, B, m0, n0, k0 + 6 * kSplitK, K, lds[0], st_t);
                __syncthreads();
                if (k0 + 2 * kSplitK >= K) break;
                if (k0 + 4 * kSplitK < K) sg.template stage_fast_if<1>(A, B, m0, n0, k0 + 7 * kSplitK, K, lds[1], st_t);
                __syncthreads();
            }
            return;
        } else {
            sg.template load<0>(A, B, m0, n0, 0, K, st_t);
            sg.template load<1>(A, B, m0, n0, kSplitK, K, st_t);
            sg.template load<2>(A, B, m0, n0, 2 * kSplitK, K, st_t);
            sg.template stage<0>(A, B, m0, n0, 0, K, lds[0], st_t);
            if (kSplitK < K) sg.template stage<1>(A, B, m0, n0, kSplitK, K, lds[1], st_t);
            __syncthreads();
            for (int k0 = 0; k0 < K; k0 += 3 * kSplitK) {
                if (k0 + 2 * kSplitK < K) sg.template stage<2>(A, B, m0, n0, k0 + 2 * kSplitK, K, lds[2], st_t);
                __syncthreads();
                if (k0 + kSplitK >= K) break;
                if (k0 + 3 * kSplitK < K) sg.template stage<0>(A, B, m0, n0, k0 + 3 * kSplitK, K, lds[0], st_t);
                __syncthreads();
                if (k0 + 2 * kSplitK >= K) break;
                if (k0 + 4 * kSplitK < K) sg.template stage<1>(A, B, m0, n0, k0 + 4 * kSplitK, K, lds[1], st_t);
                __syncthreads();
            }
            return;
        }
    }
    const int lane = threadIdx.x & 63, wm = (wave >> 1) & 1, wn = wave & 1;
    const int fr = lane & 15, fc = lane >> 4;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < K; k0 += kSplitK) {
        mma6_slab<BT, BT, 4, 4, NP>(lds[buf], lds[buf] + NP * PT, acc, wm * 64, wn * 64, fr, fc);
        __syncthreads();
        buf = buf == 2 ? 0 : buf + 1;
    }
    float* C = g.c + bz * g.sc + ks * g.scs;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + 16 * i + 4 * fc + v, col = n0 + wn * 64 + 16 * j + fr;
                if (row < g.M && col < g.N) C[(int64_t)row * g.ldc + col] = acc[i][j][v];
            }
}

#ifndef DION_STAGE_THREADS
#define DION_STAGE_THREADS 512
#endif
constexpr int kStageThreads = DION_STAGE_THREADS;   // staging threads of the split-bf16 product kernel

// NP: bf16 parts per operand, 3 (fp32-accurate split) or 1 (plain bf16 products)
template <int AK, int AADD, int BK6, int NP = 3>
static hipError_t launch_prod6(const Prod6Args& g, int64_t batch, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
    dim3 grid((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128), (unsigned)batch);
    // every tile interior: whole 128-tiles along both output edges, whole slabs, vector-legal
    // operands (the operand extents are the output extents and K); the A operand k-contiguous
    // or staged as 16-byte x rows (the four-byte x-contiguous loader's per-row addresses for
    // three register sets overflow the register file)
    // (with a triangular B every tile's K is still a whole number of slabs, at least four; with
    // split K every split must be whole slabs, at least three)
    const bool fast = (AK == S6_KC || AK == S6_XC4) && g.a.vec && g.b.vec && g.M % 128 == 0 && g.N % 128 == 0 &&
                      g.K % kSplitK == 0 && g.K >= 3 * kSplitK && g.a.xext == g.M && g.a.kext == g.K &&
                      g.b.xext == g.N && g.b.kext == g.K &&
                      (g.splits <= 1 || (g.kc % kSplitK == 0 && g.kc >= 3 * kSplitK &&
                                         g.K - (g.splits - 1) * g.kc >= 3 * kSplitK));
    if constexpr (AK == S6_KC || AK == S6_XC4) {
        if (fast) {
            hipLaunchKernelGGL((prod6_kernel<AK, AADD, BK6, true, kStageThreads, NP>), grid,
                               dim3(256 + kStageThreads), 0, s, g);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((prod6_kernel<AK, AADD, BK6, false, kStageThreads, NP>), grid, dim3(256 + kStageThreads), 0, s,
                       g);
    return hipGetLastError();
}

// W = P^T P (lower 128 x 128 tiles) for the fp32 chain; with splits > 1 the split partials go
// to the Gram partial buffer (summed in split order by the consumer).
static int gram6(const ChainCtx& c, const float* P, int mask, int val, int64_t splits, int64_t kc) {
    const Plan& p = *c.p;
    const int64_t m = p.m, r = p.r;
    Prod6Args g{};
    g.a = Op6{P, nullptr, r, (int)r, (int)m, r % 4 == 0};   // A(i,k) = P[k][i]  (i contiguous, 16-byte rows)
    g.b = Op6{P, nullptr, r, (int)r, (int)m, r % 4 == 0};   // B(k,j) = P[k][j]  (j contiguous, 16-byte rows)
    g.sa0 = g.sb0 = m * r * 4;
    g.M = g.N = (int)r; g.K = (int)m;
    g.lower = true;
    g.st = c.st; g.st_mask = mask; g.st_val = val;
    if (splits <= 1) {
        g.c = (float*)(c.ws + p.W); g.ldc = r; g.sc = r * r;
        DION_TRY((launch_prod6<S6_XC4, A6_NONE, S6_XC4>(g, p.b, c.s)));
        return 0;
    }
    g.splits = (int)splits; g.kc = kc;
    g.ska = g.skb = kc * r * 4;
    g.c = (float*)(c.ws + p.gpart); g.ldc = r; g.sc = splits * r * r; g.scs = r * r;
    DION_TRY((launch_prod6<S6_XC4, A6_NONE, S6_XC4>(g, p.b * splits, c.s)));
    return 0;
}

// Pout = Pin Tf^T for the fp32 chain (Tf lower: column tile n0 needs k < n0 + 128 only).
static int apply6(const ChainCtx& c, const float* Pin, float* Pout, int mask, int val) {
    const Plan& p = *c.p;
    const int64_t m = p.m, r = p.r;
    const bool vr = (r % 4) == 0;
    Prod6Args g{};
    g.a = Op6{Pin, nullptr, r, (int)m, (int)r, vr};                    // A(i,k) = Pin[i][k]
    g.b = Op6{c.ws + p.Tf, nullptr, r, (int)r, (int)r, vr};            // B(k,j) = Tf[j][k]
    g.sa0 = m * r * 4; g.sb0 = r * r * 4;
    g.c = Pout; g.ldc = r; g.sc = m * r;
    g.M = (int)m; g.N = (int)r; g.K = (int)r;
    g.tri = true;
    g.st = c.st; g.st_mask = mask; g.st_val = val;
    DION_TRY((launch_prod6<S6_KC, A6_NONE, S6_KC>(g, p.b, c.s)));
    return 0;
}

// P0 = (M + G) Q  and  R = (M + G)^T P for one chain.
template <typename T, int ASRC>
static int bq_gemm(const ChainCtx& c, const float* M, const void* G, int gsz, const float* Q, T* P, int mask, int val) {
    const Plan& p = *c.p;
    const int64_t m = p.m, n = p.n, r = p.r;
    if constexpr (sizeof(T) == 4 && DION_PROD6) {
        if (c.plain && stream16_ok(n, M, G, gsz == 2, false))   // bf16 weights: B streamed once
            return stream16_product(M, G, gsz == 2, Q, (uint16_t*)(c.ws + p.t16), (float*)P, m, n, r, p.b, false,
                                    c.st, mask, val, c.s);
        const bool va = (n % 4 == 0) && aligned4(M, 4) && aligned4(G, gsz);
        Prod6Args g{};
        g.a = Op6{M, G, n, (int)m, (int)n, va};               // A(i,k) = B[i][k]  (k contiguous)
        g.b = Op6{Q, nullptr, r, (int)r, (int)n, r % 4 == 0};   // B(k,j) = Q[k][j]  (j contiguous)
        g.sa0 = m * n * 4; g.sa1 = m * n * gsz; g.sb0 = n * r * 4;
        g.c = (float*)P; g.ldc = r; g.sc = m * r;
        g.M = (int)m; g.N = (int)r; g.K = (int)n;
        g.st = c.st; g.st_mask = mask; g.st_val = val;
        hipError_t he;
        if (c.plain) he = ASRC == SRC_SUM_BF16 ? launch_prod6<S6_KC, A6_BF16, S6_XC4, 1>(g, p.b, c.s)
                                               : launch_prod6<S6_KC, A6_F32, S6_XC4, 1>(g, p.b, c.s);
        else he = ASRC == SRC_SUM_BF16 ? launch_prod6<S6_KC, A6_BF16, S6_XC4>(g, p.b, c.s)
                                       : launch_prod6<S6_KC, A6_F32, S6_XC4>(g, p.b, c.s);
        DION_TRY(he);
        return 0;
    }
    GemmArgs g{};
    const bool va = (n % 4 == 0) && aligned4(M, 4) && aligned4(G, gsz);
    g.a = Operand{M, G, n, (int)m, (int)n, va};                    // A(i,k) = B[i][k]
    g.b = Operand{Q, nullptr, r, (int)r, (int)n, (r % 4) == 0};    // B(k,j) = Q[k][j]
    g.sa0 = m * n * 4; g.sa1 = m * n * gsz; g.sb0 = n * r * 4;
    g.c = P; g.ldc = r; g.sc = m * r * (int64_t)sizeof(T);
    g.M = (int)m; g.N = (int)r; g.K = (int)n;
    g.alpha = 1; g.beta = 0;
    g.st = c.st; g.st_mask = mask; g.st_val = val;
    DION_TRY((launch_gemm<T, 64, 64, true, ASRC, false, SRC_F32>(g, p.b, c.s)));
    return 0;
}

template <typename T, int ASRC>
static int btp_gemm(const ChainCtx& c, const float* M, const void* G, int gsz, const T* P, T* R, int mask, int val) {
    const Plan& p = *c.p;
    const int64_t m = p.m, n = p.n, r = p.r;
    if constexpr (sizeof(T) == 4 && DION_PROD6) {
        if (c.plain && stream16_ok(n, M, G, gsz == 2, true))    // bf16 weights: B streamed once
            return stream16_product(M, G, gsz == 2, (const float*)P, (uint16_t*)(c.ws + p.t16), (float*)R, m, n, r,
                                    p.b, true, c.st, mask, val, c.s);
        const bool va = (n % 4 == 0) && aligned4(M, 4) && aligned4(G, gsz);
        Prod6Args g{};
        g.a = Op6{M, G, n, (int)n, (int)m, va};               // A(i,k) = B[k][i]  (i contiguous)
        g.b = Op6{P, nullptr, r, (int)r, (int)m, r % 4 == 0};   // B(k,j) = P[k][j]  (j contiguous)
        g.sa0 = m * n * 4; g.sa1 = m * n * gsz; g.sb0 = m * r * 4;
        g.c = (float*)R; g.ldc = r; g.sc = n * r;
        g.M = (int)n; g.N = (int)r; g.K = (int)m;
        g.st = c.st; g.st_mask = mask; g.st_val = val;
        // K split in two (second half into the unused fp64 R region, added back in split order)
        // when that turns a final partial round of tiles (one workgroup per CU) into whole rounds
        const int64_t tiles = ((n + 127) / 128) * ((r + 127) / 128) * p.b, slots = 256;
        const double rounds1 = (double)((tiles + slots - 1) / slots), rounds2 = (double)((2 * tiles + slots - 1) / slots) / 2;
        if (m % 64 == 0 && m / 2 >= 3 * kSplitK && rounds2 < rounds1 - 0.2) {
            g.splits = 2; g.kc = m / 2;
            g.ska = g.kc * n * 4; g.ska1 = g.kc * n * gsz; g.skb = g.kc * r * 4;
            g.scs = (int64_t)(p.R64 - p.R32) / 4;
            hipError_t he;
            if (c.plain) he = ASRC == SRC_SUM_BF16 ? launch_prod6<S6_XC4, A6_BF16, S6_XC4, 1>(g, p.b * 2, c.s)
                                                   : launch_prod6<S6_XC4, A6_F32, S6_XC4, 1>(g, p.b * 2, c.s);
            else he = ASRC == SRC_SUM_BF16 ? launch_prod6<S6_XC4, A6_BF16, S6_XC4>(g, p.b * 2, c.s)
                                           : launch_prod6<S6_XC4, A6_F32, S6_XC4>(g, p.b * 2, c.s);
            DION_TRY(he);
            dim3 grid(grid_1d(n * r / 4, 1024), (unsigned)p.b);
            hipLaunchKernelGGL(add_split_kernel, grid, dim3(256), 0, c.s, (float*)R, (const float*)(c.ws + p.R64), n * r,
                               (const int*)c.st, mask, val);
            DION_TRY(hipGetLastError());
            return 0;
        }
        hipError_t he;
        if (c.plain) he = ASRC == SRC_SUM_BF16 ? launch_prod6<S6_XC4, A6_BF16, S6_XC4, 1>(g, p.b, c.s)
                                               : launch_prod6<S6_XC4, A6_F32, S6_XC4, 1>(g, p.b, c.s);
        else he = ASRC == SRC_SUM_BF16 ? launch_prod6<S6_XC4, A6_BF16, S6_XC4>(g, p.b, c.s)
                                       : launch_prod6<S6_XC4, A6_F32, S6_XC4>(g, p.b, c.s);
        DION_TRY(he);
        return 0;
    }
    GemmArgs g{};
    const bool va = (n % 4 == 0) && aligned4(M, 4) && aligned4(G, gsz);
    g.a = Operand{M, G, n, (int)n, (int)m, va};                    // A(i,k) = B[k][i]
    g.b = Operand{P, nullptr, r, (int)r, (int)m, (r % 4) == 0};    // B(k,j) = P[k][j]
    g.sa0 = m * n * 4; g.sa1 = m * n * gsz; g.sb0 = m * r * (int64_t)sizeof(T);
    g.c = R; g.ldc = r; g.sc = n * r * (int64_t)sizeof(T);
    g.M = (int)n; g.N = (int)r; g.K = (int)m;
    g.alpha = 1; g.beta = 0;
    g.st = c.st; g.st_mask = mask; g.st_val = val;
    DION_TRY((launch_gemm<T, 64, 64, false, ASRC, false, SrcOf<T>::v>(g, p.b, c.s)));
    return 0;
}

template <typename T>
static int run_chain(const ChainCtx& c, const float* M, const void* G, bool g_bf16, const float* Q,
                     bool force32, void* const* ev, bool householder = false, bool spectral = false) {
    // ev: events marking the starts of the chain's three phases (product, QR, back-projection)
    auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord((hipEvent_t)ev[i], c.s) : hipSuccess; };
    const Plan& p = *c.p;
    const bool is64 = sizeof(T) == 8;
    T* P = (T*)(c.ws + (is64 ? p.P64 : p.P32));
    T* R = (T*)(c.ws + (is64 ? p.R64 : p.R32));
    const int gsz = g_bf16 ? 2 : 4;
    int e;
    if (!is64) {
        // fp32 chain: matrices not (yet) owned by the fp64 chain; P32 -> tmp -> P32
        T* tmp = (T*)(c.ws + p.P64b);
        const int mask = ST_PATH64 | ST_FAIL, val = 0;
        const int fail = force32 ? ST_FAIL : ST_PATH64;
        DION_TRY(mark(0));
        if ((e = g_bf16 ? bq_gemm<T, SRC_SUM_BF16>(c, M, G, gsz, Q, P, mask, val)
                        : bq_gemm<T, SRC_SUM_F32>(c, M, G, gsz, Q, P, mask, val))) return e;
        DION_TRY(c.open_gate());
        DION_TRY(mark(1));
        if ((e = cholqr_pass<T>(c, P, tmp, mask, val, force32 ? 0.0 : kTau32, fail, ST_PATH64))) return e;
        if ((e = reortho_pass<T>(c, tmp, P, mask, val, kNearId32, fail))) return e;
        DION_TRY(mark(2));
        return g_bf16 ? btp_gemm<T, SRC_SUM_BF16>(c, M, G, gsz, P, R, mask, val)
                      : btp_gemm<T, SRC_SUM_F32>(c, M, G, gsz, P, R, mask, val);
    }
    // fp64 chain: P64 -> P64b -> P64 (-> P64b -> P64 after a shifted first pass)
    T* Pb = (T*)(c.ws + p.P64b);
    const int A64 = ST_PATH64, SH = ST_SHIFT, F = ST_FAIL;
    DION_TRY(mark(0));
    if ((e = g_bf16 ? bq_gemm<T, SRC_SUM_BF16>(c, M, G, gsz, Q, P, A64, A64)
                    : bq_gemm<T, SRC_SUM_F32>(c, M, G, gsz, Q, P, A64, A64))) return e;
    DION_TRY(c.open_gate());
    DION_TRY(mark(1));
    if (householder) {   // requested: every fp64-chain matrix goes to the Householder QR below
        hipLaunchKernelGGL(set_bits_kernel, dim3(grid_1d(p.b)), dim3(256), 0, c.s, c.st, p.b, A64, A64, F);
        DION_TRY(hipGetLastError());
    }
    // pass 1: unshifted attempt; a failed pivot or a large diagonal ratio marks SHIFT,
    // and the marked matrices factor W + s I instead (W is kept by the factorization)
    if ((e = gram<T>(c, P, A64 | F, A64))) return e;
    if ((e = factor_invert<T>(c, A64 | SH | F, A64, kTau64, SH, SH, 0, false))) return e;
    ChainCtx cs = c;
    if (spectral) {   // the shift from a multi-power-iteration estimate of lambda_max(W), not trace(W)
        double* pw = (double*)(c.ws + p.pw);
        const int64_t stride = (int64_t)(p.spw / sizeof(double));
        MpiArgs ma{};
        ma.W = (const double*)(c.ws + p.W); ma.r = p.r; ma.k = kShiftPool; ma.V0 = nullptr; ma.first = p.c0;
        ma.ws = pw; ma.ws_stride = stride;
        ma.lam = pw + 2 * p.r * kShiftPool + 1; ma.lam_stride = stride;
        ma.st = c.st; ma.st_mask = A64 | SH | F; ma.st_val = A64 | SH;
        if ((e = run_lambda_max(ma, p.b, kShiftIters, c.s))) return e;
        cs.lam = ma.lam; cs.lam_stride = stride;
    }
    if ((e = factor_invert<T>(cs, A64 | SH | F, A64 | SH, 0.0, F, 0, 1, true))) return e;
    if ((e = apply<T>(c, P, Pb, A64 | F, A64))) return e;
    // pass 2
    if ((e = reortho_pass<T>(c, Pb, P, A64 | F, A64, kNearId64, F))) return e;
    // pass 3, only after a shifted first pass
    if ((e = reortho_pass<T>(c, P, Pb, A64 | SH | F, A64 | SH, kNearId64, F))) return e;
    {
        // rare copies (failed or shifted matrices only): few workgroups per matrix, so that the
        // launch costs little when no matrix needs it
        dim3 grid(grid_1d(p.m * p.r, 128), (unsigned)p.b);
        // Where a pass broke down, P still holds P0 times an upper-triangular matrix (the passes
        // before the failing one), whose Q-factor is that of P0: Householder QR of a copy in Pb,
        // the Q-factor written back to P
        if constexpr (sizeof(T) == 8) if (p.r <= kHouseholderMaxRank) {
            hipLaunchKernelGGL((copy_pred_kernel<T>), grid, dim3(256), 0, c.s, (const T*)P, Pb, p.m * p.r, c.st,
                               A64 | F, A64 | F);
            DION_TRY(hipGetLastError());
            if (p.nblk > kFusedMaxBlocks) {   // large ranks: the blocked form on the matrix cores
                if ((e = householder_blocked(c, (double*)Pb, (double*)P, A64 | F, A64 | F))) return e;
            } else {
                hipLaunchKernelGGL(householder_kernel, dim3((unsigned)p.b), dim3(1024), 0, c.s, (double*)Pb,
                                   (double*)P, p.m, p.r, c.st, A64 | F, A64 | F);
                DION_TRY(hipGetLastError());
            }
        }
        hipLaunchKernelGGL((copy_pred_kernel<T>), grid, dim3(256), 0, c.s, Pb, P, p.m * p.r, c.st,
                           A64 | SH | F | ST_HH, A64 | SH);
        DION_TRY(hipGetLastError());
    }
    DION_TRY(mark(2));
    return g_bf16 ? btp_gemm<T, SRC_SUM_BF16>(c, M, G, gsz, P, R, A64, A64)
                  : btp_gemm<T, SRC_SUM_F32>(c, M, G, gsz, P, R, A64, A64);
}

// nparts: set to the number of momentum-change partials per matrix (tiles of the launch)
template <bool GB, bool XB, int NP>
static hipError_t launch_update(const Plan& p, const char* ws, const float* Q, float* M, const void* G, void* X,
                                float mu, float lr, hipStream_t s, float* mx, int* nparts) {
    UpdArgs u{};
    u.P = (const float*)(ws + p.P32);
    u.R = (const float*)(ws + p.R32);
    u.Q = Q;
    u.M = M; u.G = G; u.X = X;
    u.st = (const int*)(ws + p.st);
    u.mx = mx;
    u.nmx = p.nmx;
    u.m = (int)p.m; u.n = (int)p.n; u.r = (int)p.r; u.kp = (int)p.kp;
    u.vec = (p.r % 4) == 0;
    u.one_minus_mu = 1.0f - mu;
    u.lr_s = (float)((double)lr * sqrt((double)p.m / (double)p.n));
    // 128 x 64 tiles while they still fill the chip, else 64 x 64
    const int64_t big = ((p.n + 63) / 64) * ((p.m + 127) / 128) * p.b;
    if (big >= kUpdBigMinTiles) {
        dim3 grid((unsigned)((p.n + 63) / 64), (unsigned)((p.m + 127) / 128), (unsigned)p.b);
        *nparts = (int)(grid.x * grid.y);
        // all tiles interior, whole slabs, vector-legal rows: the two-set branch-free loop
        const bool fast = p.m % 128 == 0 && p.n % 64 == 0 && p.r % kSplitK == 0 && p.r >= 2 * kSplitK && u.vec;
        if (fast) hipLaunchKernelGGL((update3_kernel<GB, XB, true, NP>), grid, dim3(256), 0, s, u);
        else hipLaunchKernelGGL((update3_kernel<GB, XB, false, NP>), grid, dim3(256), 0, s, u);
    } else {
        dim3 grid((unsigned)((p.n + 63) / 64), (unsigned)((p.m + 63) / 64), (unsigned)p.b);
        *nparts = (int)(grid.x * grid.y);
        hipLaunchKernelGGL((update_kernel<64, 64, 2, 2, GB, XB, NP>), grid, dim3(256), 0, s, u);
    }
    return hipGetLastError();
}

// The whole step for the matrices of one chunk, on stream s.
static int run_chunk(const Plan& p, void* X, const void* G, float* M, float* Q, float mu, float lr, float eps,
                     int x_bf16, int g_bf16, char* ws, int32_t* flags, uint32_t options, hipStream_t s,
                     void* const* ev, hipEvent_t gate = nullptr, float* rmmc = nullptr) {
    float* mx = rmmc ? (float*)(ws + p.mx) : nullptr;
    auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess; };
    if (p.b == 0) return 0;
    const int64_t mn = p.m * p.n;
    if (p.r == 0) {
        for (int i = 0; i < DION_NUM_PHASES; ++i) DION_TRY(mark(i));
        const int64_t per = std::min<int64_t>(p.nmx, std::max<int64_t>(1, 8192 / p.b));
        dim3 grid(grid_1d(mn, per), (unsigned)p.b);
        if (g_bf16) hipLaunchKernelGGL((add_grad_kernel<true>), grid, dim3(256), 0, s, M, G, mn, mx, p.nmx);
        else hipLaunchKernelGGL((add_grad_kernel<false>), grid, dim3(256), 0, s, M, G, mn, mx, p.nmx);
        DION_TRY(hipGetLastError());
        if (rmmc) {
            hipLaunchKernelGGL(rmmc_kernel, dim3((unsigned)p.b), dim3(256), 0, s, (const float*)mx, p.nmx,
                               (int)grid.x, rmmc);
            DION_TRY(hipGetLastError());
        }
        if (flags) {  // a fill kernel rather than a memset node, so callers may capture the step in a graph
            hipLaunchKernelGGL(zero_flags_kernel, dim3(grid_1d(p.b)), dim3(256), 0, s, flags, p.b);
            DION_TRY(hipGetLastError());
        }
        if (gate) DION_TRY(hipEventRecord(gate, s));
        DION_TRY(mark(DION_NUM_PHASES));
        return 0;
    }
    const bool force64 = options & DION_OPT_FORCE_F64;
    const bool force32 = options & DION_OPT_FORCE_F32;
    const bool sticky = options & DION_OPT_STICKY_F64;
    bool gated = false;
    ChainCtx c{&p, ws, (int*)(ws + p.st), s, gate, &gated};
    c.plain = x_bf16 && !(options & DION_OPT_EXACT_PRODUCTS);
    DION_TRY(mark(DION_PHASE_INIT));
    hipLaunchKernelGGL(init_state_kernel, dim3(grid_1d(p.b)), dim3(256), 0, s, c.st, (const int32_t*)flags, p.b,
                       (int)force64, (int)sticky);
    DION_TRY(hipGetLastError());
    int e;
    if (!force64 && (e = run_chain<float>(c, M, G, g_bf16, Q, force32, ev ? ev + DION_PHASE_F32_PRODUCT : nullptr)))
        return e;
    if (force64 && ev)
        for (int i = DION_PHASE_F32_PRODUCT; i <= DION_PHASE_F32_BACKPROJECT; ++i) DION_TRY(mark(i));
    if (!force32 && (e = run_chain<double>(c, M, G, g_bf16, Q, force32, ev ? ev + DION_PHASE_F64_PRODUCT : nullptr,
                                           (options & DION_OPT_HOUSEHOLDER) != 0,
                                           (options & DION_OPT_SPECTRAL_SHIFT) != 0)))
        return e;
    if (force32 && ev)
        for (int i = DION_PHASE_F64_PRODUCT; i <= DION_PHASE_F64_BACKPROJECT; ++i) DION_TRY(mark(i));
    DION_TRY(c.open_gate());
    DION_TRY(mark(DION_PHASE_NORMS));

    // column norms -> c = 1 / (||r_j|| + eps); Q <- R c; fp64-chain P, R rounded to fp32
    {
        dim3 grid((unsigned)((p.r + 63) / 64), (unsigned)p.nchunk, (unsigned)p.b);
        hipLaunchKernelGGL(colnorm_partial_kernel, grid, dim3(256), 0, s, (const float*)(ws + p.R32),
                           (const double*)(ws + p.R64), (double*)(ws + p.part), p.n, p.r, (int)p.nchunk, c.st);
        DION_TRY(hipGetLastError());
        dim3 g2((unsigned)((p.r + 255) / 256), (unsigned)p.b);
        hipLaunchKernelGGL(colscale_kernel, g2, dim3(256), 0, s, (const double*)(ws + p.part), (double*)(ws + p.cs),
                           p.r, (int)p.nchunk, (double)eps);
        DION_TRY(hipGetLastError());
        dim3 g3(grid_1d(p.n * ((p.r + 3) / 4), 1024), (unsigned)p.b);
        hipLaunchKernelGGL(next_q_kernel, g3, dim3(256), 0, s, (const double*)(ws + p.R64), (float*)(ws + p.R32),
                           (const double*)(ws + p.cs), Q, p.n, p.r, c.st);
        DION_TRY(hipGetLastError());
        dim3 g4(grid_1d(p.m * ((p.r + 3) / 4), 1024), (unsigned)p.b);
        hipLaunchKernelGGL(round_p_kernel, g4, dim3(256), 0, s, (const double*)(ws + p.P64), (float*)(ws + p.P32),
                           p.m, p.r, c.st);
        DION_TRY(hipGetLastError());
    }
    DION_TRY(mark(DION_PHASE_UPDATE));
    hipError_t he;
    int nparts = 0;
    // the weight pass's products: plain bf16 for bf16 weights, two-part split (three part
    // products) for fp32 weights, the fp32-accurate three-part split (six) on request
    const bool exact = options & DION_OPT_EXACT_PRODUCTS;
    if (c.plain) he = g_bf16 ? launch_update<true, true, 1>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts)
                             : launch_update<false, true, 1>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts);
    else if (x_bf16) he = g_bf16 ? launch_update<true, true, 3>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts)
                                 : launch_update<false, true, 3>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts);
    else if (exact) he = g_bf16 ? launch_update<true, false, 3>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts)
                                : launch_update<false, false, 3>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts);
    else he = g_bf16 ? launch_update<true, false, 2>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts)
                     : launch_update<false, false, 2>(p, ws, Q, M, G, X, mu, lr, s, mx, &nparts);
    DION_TRY(he);
    if (rmmc) {
        hipLaunchKernelGGL(rmmc_kernel, dim3((unsigned)p.b), dim3(256), 0, s, (const float*)mx, p.nmx, nparts, rmmc);
        DION_TRY(hipGetLastError());
    }
    DION_TRY(mark(DION_PHASE_FLAGS));
    if (flags) {
        hipLaunchKernelGGL(flags_out_kernel, dim3((unsigned)p.b), dim3(256), 0, s, c.st,
                           (const double*)(ws + p.cs), p.r, flags);
        DION_TRY(hipGetLastError());
    }
    DION_TRY(mark(DION_NUM_PHASES));
    return 0;
}

// Streams and events of the internal fork/join, one set per device, created on first use
// (default priority).  A step can be split into chunks of whole matrices, each run on its own
// stream.  The chunks are staggered: chunk c + 1 starts once chunk c has issued its first
// product, so that chunk c's latency-bound CholeskyQR (few workgroups, many dependent
// launches) runs beside chunk c + 1's compute-bound products, and chunk c's back-projection
// and weight pass beside chunk c + 1's CholeskyQR.
constexpr int kMaxChunks = 8;
struct StreamSet {
    bool ready = false;
    hipStream_t s[kMaxChunks];
    hipEvent_t fork, join[kMaxChunks], gate[kMaxChunks];
};
static std::mutex g_stream_mu;
static StreamSet g_streams[64];

static hipError_t stream_set(StreamSet** out) {
    int dev = 0;
    DION_TRY_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    StreamSet& ss = g_streams[dev];
    if (!ss.ready) {
        for (int i = 0; i < kMaxChunks; ++i) {
            DION_TRY_HIP(hipStreamCreateWithFlags(&ss.s[i], hipStreamNonBlocking));
            DION_TRY_HIP(hipEventCreateWithFlags(&ss.join[i], hipEventDisableTiming));
            DION_TRY_HIP(hipEventCreateWithFlags(&ss.gate[i], hipEventDisableTiming));
        }
        DION_TRY_HIP(hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming));
        ss.ready = true;
    }
    *out = &ss;
    return hipSuccess;
}

static int auto_chunks(const Plan&) {
    // Concurrent chunks start in lockstep, so their latency-bound phases overlap each other
    // rather than the GEMMs; measured no gain on the 24 x 1024^2 stack.  Off by default.
    return 1;
}

int run_step(const Plan& p, void* X, const void* G, float* M, float* Q, float mu, float lr, float eps, int x_bf16,
             int g_bf16, char* ws, int32_t* flags, uint32_t options, void* stream, void* const* ev, float* rmmc) {
    hipStream_t s = (hipStream_t)stream;
    if (p.b == 0) return 0;
    int nc = (int)((options >> DION_OPT_CHUNKS_SHIFT) & 15u);
    if (nc == 0) nc = auto_chunks(p);
    if (nc > kMaxChunks) nc = kMaxChunks;
    if (nc > p.b) nc = (int)p.b;
    if (nc <= 1)
        return run_chunk(p, X, G, M, Q, mu, lr, eps, x_bf16, g_bf16, ws, flags, options, s, ev, nullptr, rmmc);
    std::lock_guard<std::mutex> lock(g_stream_mu);
    StreamSet* ss = nullptr;
    DION_TRY(stream_set(&ss));
    DION_TRY(hipEventRecord(ss->fork, s));
    const int64_t mn = p.m * p.n, xs = x_bf16 ? 2 : 4, gs = g_bf16 ? 2 : 4;
    for (int c = 0; c < nc; ++c) {
        const int64_t c0 = p.b * c / nc, c1 = p.b * (c + 1) / nc;
        const Plan q = chunk_plan(p, c0, c1 - c0);
        DION_TRY(hipStreamWaitEvent(ss->s[c], ss->fork, 0));
        if (c > 0) DION_TRY(hipStreamWaitEvent(ss->s[c], ss->gate[c - 1], 0));
        int e = run_chunk(q, (char*)X + c0 * mn * xs, (const char*)G + c0 * mn * gs, M + c0 * mn,
                          Q ? Q + c0 * p.n * p.r : nullptr, mu, lr, eps, x_bf16, g_bf16, ws, flags ? flags + c0 : nullptr,
                          options, ss->s[c], c == 0 ? ev : nullptr, ss->gate[c], rmmc ? rmmc + c0 : nullptr);
        if (e) return e;
        DION_TRY(hipEventRecord(ss->join[c], ss->s[c]));
        DION_TRY(hipStreamWaitEvent(s, ss->join[c], 0));
    }
    return 0;
}

}  // namespace dion
