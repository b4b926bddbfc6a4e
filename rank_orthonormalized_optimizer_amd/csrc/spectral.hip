// Multi-power-iteration estimate of the largest eigenvalue of symmetric positive semi-definite
// matrices (the Gram matrices W = P0^T P0 of the Dion step).
//
// The DASH summary (gist.science, "Methodologie", 2. "Efficiënte Inverse-Root Solvers", the item
// on multi-power-iteration scaling): the spectral radius is estimated by power iteration run in
// parallel from a pool of up to 32 start vectors, and replaces the Frobenius norm as the scale of
// a matrix.  Here the estimate is the largest Rayleigh quotient of the pool after t normalized
// products.  The shifted CholeskyQR of the fallback chain can take its shift from it instead of
// from trace(W) = ||P0||_F^2, which exceeds ||P0||_2^2 by up to the rank.
//
// Layout: W is [b][r][r] fp64 row-major and only its lower triangle is read (the Gram kernels
// write lower tiles only).  The pool lives in a per-matrix scratch slice of `ws_stride` doubles:
// two r x k buffers (row-major, k vectors side by side) and trace(W) behind them.  Instead of
// normalizing every product, each product divides by trace(W) >= lambda_max, so the iterates
// shrink by at most the rank per product and stay far from fp64 underflow for the <= 64 products
// allowed; the Rayleigh quotient is scale-free, so the estimate is the same.
//
// Kernels: one init launch (the pool, from the caller's vectors or a SplitMix64 counter stream,
// and the trace), t + 1 product launches over 64-row blocks (W tiles mirrored from the lower
// triangle through LDS, fp64 matrix-core products with the pool), one finish launch per
// matrix (fixed-order dot products and the pool's maximum).  Every launch returns at once for a
// matrix whose state word does not match, so the Dion step can run it for the shifted matrices
// only.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dion_plan.h"
#include "gemm_mfma.hpp"

namespace dion {

namespace {

constexpr int kRows = 64;   // rows of W and of the pool per product workgroup

// The n-th output (n >= 1) of SplitMix64 seeded with 0 (Steele, Lea and Flood, "Fast Splittable
// Pseudorandom Number Generators", 2014): the state advances by the golden-ratio increment and
// each output is the state passed through the variant-13 finalizer.
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t n) {
    uint64_t z = n * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ bool owned(const MpiArgs& a, int bz) {
    return !a.st || (a.st[bz] & a.st_mask) == a.st_val;
}

// The pool V_0 (caller's vectors, or 2u - 1 with u the top 53 bits of SplitMix64 output
// (first + bz)*r*k + i*k + j + 1) and trace(W), fixed-order.
__global__ __launch_bounds__(256) void mpi_init_kernel(MpiArgs a) {
    const int bz = blockIdx.y;
    if (!owned(a, bz)) return;
    const int64_t rk = a.r * a.k;
    double* V = a.ws + bz * a.ws_stride;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < rk; idx += (int64_t)gridDim.x * 256) {
        double v;
        if (a.V0) {
            v = a.V0[bz * rk + idx];
        } else {
            const uint64_t z = splitmix64_at((uint64_t)((a.first + bz) * rk + idx) + 1);
            v = (double)(z >> 11) * 0x1.0p-53 * 2.0 - 1.0;
        }
        V[idx] = v;
    }
    if (blockIdx.x == 0) {
        __shared__ double red[256];
        const double* W = a.W + bz * a.r * a.r;
        const int64_t r = a.r;
        double tr = 0;
        // eight diagonal loads in flight per thread (clamped addresses, zero outside)
        for (int64_t i0 = threadIdx.x; i0 < r; i0 += 256 * 8) {
            double d[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t i = i0 + 256 * q;
                const double x = W[(i < r ? i : 0) * (r + 1)];
                d[q] = i < r ? x : 0.0;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) tr += d[q];
        }
        red[threadIdx.x] = tr;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        if (threadIdx.x == 0) V[2 * rk] = red[0];
    }
}

// V_out[rows of this block] = W V_in / trace(W), for the 64 rows R0.. of W; the pool buffer
// `src` is read and the other one written.  Each wave multiplies 16 rows by the 32 pool columns
// on the fp64 matrix cores (two 16 x 16 blocks, v_mfma_f64_16x16x4, k = 4 s + lane / 16 at
// step s).  The next column tile of W and of the pool is loaded into registers while the
// current one is multiplied from LDS (loads branch-free: addresses clamped into the matrix,
// values selected to zero outside it), so each tile's HBM latency overlaps the previous tile's
// matrix-core work.  LDS pitches 66 (W) and 48 (pool) doubles put each half-wave's fragment
// reads in distinct banks.  (Loading each wave's W fragments straight into registers, without
// LDS, measured 13% slower: below the diagonal a fragment load then touches 16 rows of W.)
__global__ __launch_bounds__(256) void mpi_product_kernel(MpiArgs a, int src) {
    const int bz = blockIdx.y;
    if (!owned(a, bz)) return;
    const int64_t r = a.r, rk = r * a.k;
    const int k = a.k;
    const double* W = a.W + bz * r * r;
    double* base = a.ws + bz * a.ws_stride;
    const double* Vin = base + (src ? rk : 0);
    double* Vout = base + (src ? 0 : rk);
    const double tau = base[2 * rk];
    const double scale = tau > 0.0 ? 1.0 / tau : 0.0;
    constexpr int kWPitch = kRows + 2, kVPitch = kMpiMaxPool + 16;
    __shared__ double Wt[kRows][kWPitch];
    __shared__ double Vt[kRows][kVPitch];
    constexpr int kWPer = kRows * kRows / 256, kVPer = kRows * kMpiMaxPool / 256;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const int64_t R0 = (int64_t)blockIdx.x * kRows;
    const int64_t ntile = (r + kRows - 1) / kRows;
    double wr[kWPer], vr[kVPer];
    // element (gi, gc) of the symmetric W from the lower triangle: W[gi][gc] if gc <= gi, else
    // W[gc][gi]; threads run along the stored rows so the loads coalesce either way
    auto load_tile = [&](int64_t cb) {
        const int64_t C0 = cb * kRows;
        const bool lower = C0 <= R0;
#pragma unroll
        for (int q = 0; q < kWPer; ++q) {
            const int e = tid + 256 * q;
            const int i = lower ? (e >> 6) : (e & (kRows - 1));
            const int c = lower ? (e & (kRows - 1)) : (e >> 6);
            const int64_t gi = R0 + i, gc = C0 + c;
            const bool ok = gi < r && gc < r;
            const int64_t hi = ok ? (gc <= gi ? gi : gc) : 0, lo = ok ? (gc <= gi ? gc : gi) : 0;
            const double w = W[hi * r + lo];
            wr[q] = ok ? w : 0.0;
        }
#pragma unroll
        for (int q = 0; q < kVPer; ++q) {
            const int e = tid + 256 * q;
            const int c = e / kMpiMaxPool, j = e % kMpiMaxPool;
            const int64_t gc = C0 + c;
            const bool ok = gc < r && j < k;
            const double v = Vin[ok ? gc * k + j : 0];
            vr[q] = ok ? v : 0.0;
        }
    };
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
    load_tile(0);
    for (int64_t cb = 0; cb < ntile; ++cb) {
        const bool lower = cb * kRows <= R0;
        __syncthreads();   // the previous tile's products are done with the LDS tiles
#pragma unroll
        for (int q = 0; q < kWPer; ++q) {
            const int e = tid + 256 * q;
            const int i = lower ? (e >> 6) : (e & (kRows - 1));
            const int c = lower ? (e & (kRows - 1)) : (e >> 6);
            Wt[i][c] = wr[q];
        }
#pragma unroll
        for (int q = 0; q < kVPer; ++q) {
            const int e = tid + 256 * q;
            Vt[e / kMpiMaxPool][e % kMpiMaxPool] = vr[q];
        }
        __syncthreads();
        load_tile(cb + 1 < ntile ? cb + 1 : cb);   // the last tile reloads itself: no branch on the loads
#pragma unroll
        for (int st = 0; st < kRows / 4; ++st) {
            const int kk = 4 * st + lk;
            const double af = Wt[16 * wave + lr][kk];
            acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(af, Vt[kk][lr], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(af, Vt[kk][16 + lr], acc1, 0, 0, 0);
        }
    }
    // D[row][col] of a 16 x 16 block: lane l, element v holds row l / 16 + 4 v, column l % 16
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t gi = R0 + 16 * wave + lk + 4 * v;
        if (gi < r) {
            if (lr < k) Vout[gi * k + lr] = acc0[v] * scale;
            if (16 + lr < k) Vout[gi * k + 16 + lr] = acc1[v] * scale;
        }
    }
}

// lambda_hat = max_j trace(W) (V_t . V_t+1)_j / (V_t . V_t)_j over the pool (0 for a zero
// vector); `last` is the buffer the last product wrote (V_t+1).  1024 threads: column j = tid % 32,
// row group g = tid / 32 takes rows g, g + 32, ... four at a time; the 32 groups' partial sums are
// added in group order.
__global__ __launch_bounds__(1024) void mpi_finish_kernel(MpiArgs a, int last) {
    const int bz = blockIdx.x;
    if (!owned(a, bz)) return;
    const int64_t r = a.r, rk = r * a.k;
    const int k = a.k;
    const double* base = a.ws + bz * a.ws_stride;
    const double* V1 = base + (last ? rk : 0);
    const double* V0 = base + (last ? 0 : rk);
    const double tau = base[2 * rk];
    __shared__ double sn[1024], sd[1024];
    const int j = threadIdx.x & 31, g = threadIdx.x >> 5;
    double num = 0.0, den = 0.0;
    if (j < k)
        for (int64_t i0 = g; i0 < r; i0 += 32 * 4) {
            double x[4], y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = i0 + 32 * q;
                const int64_t o = (i < r ? i : 0) * k + j;
                x[q] = i < r ? V0[o] : 0.0;
                y[q] = i < r ? V1[o] : 0.0;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                num = fma(x[q], y[q], num);
                den = fma(x[q], x[q], den);
            }
        }
    sn[threadIdx.x] = num;
    sd[threadIdx.x] = den;
    __syncthreads();
    if (threadIdx.x < 32) {
        double n = 0.0, d = 0.0;
        for (int q = 0; q < 32; ++q) {
            n += sn[q * 32 + j];
            d += sd[q * 32 + j];
        }
        double lam = j < k ? (d > 0.0 ? tau * (n / d) : 0.0) : -INFINITY;
        for (int off = 16; off > 0; off >>= 1) lam = fmax(lam, __shfl_xor(lam, off, 32));
        if (threadIdx.x == 0) a.lam[bz * a.lam_stride] = lam;
    }
}

}  // namespace

int run_lambda_max(const MpiArgs& a, int64_t b, int iters, void* stream) {
    const hipStream_t s = (hipStream_t)stream;
    if (b == 0) return 0;
    const int64_t rk = a.r * a.k;
    int64_t gx = (rk + 255) / 256;
    if (gx > 1024) gx = 1024;
    hipLaunchKernelGGL(mpi_init_kernel, dim3((unsigned)gx, (unsigned)b), dim3(256), 0, s, a);
    for (int i = 1; i <= iters + 1; ++i)
        hipLaunchKernelGGL(mpi_product_kernel, dim3((unsigned)((a.r + kRows - 1) / kRows), (unsigned)b), dim3(256), 0,
                           s, a, (i - 1) & 1);
    hipLaunchKernelGGL(mpi_finish_kernel, dim3((unsigned)b), dim3(1024), 0, s, a, (iters + 1) & 1);
    return (int)hipGetLastError();
}

}  // namespace dion
