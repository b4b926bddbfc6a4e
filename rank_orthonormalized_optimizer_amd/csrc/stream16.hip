// Plain bf16 products that stream B = M + G once from HBM, for stacks whose weights are bf16
// (operands rounded once to bf16, fp32 accumulation on the bf16 matrix cores):
//
//   P0 = (M + G) Q      (p16_kernel, the power-iteration step)
//   R  = (M + G)^T P    (r16_kernel, the back-projection)
//
// Both are HBM-bound: 6 bytes of M and G per element of B (4 with bf16 G... plus the fp32 M)
// against 2 r flops.  A workgroup owns a panel of B and all r <= 256 columns of the output, so
// B is read exactly once; the small operand (Q or P) is first written transposed in bf16
// (t16_kernel), so that its MFMA fragments are 16-byte rows, and is shared by the workgroup's
// waves through LDS.  Global loads run kStreamD slabs ahead in register sets; the slab loop is
// branch-free (the last slabs re-read the final slab's addresses, their values unused or zero),
// so the compiler only waits for the set a slab consumes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dion.h"
#include "dion_plan.h"
#include "gemm_mfma.hpp"
#include "bf16x6.hpp"

namespace dion {

constexpr int kStreamD = 4;   // slabs of global loads in flight per register set rotation

// The transposed bf16 copy of an fp32 [rows][cols] array in 32-row slabs: element (i, c) goes to
// out[bz][i / 32][c][i % 32], zero for rows <= i < pitch (pitch a multiple of 32).  A slab of the
// transposed operand (all cols x 32) is then one contiguous block, read with whole cache lines.
// 64 x 64 tiles through LDS; grid (ceil(cols / 64), ceil(pitch / 64), batch).
__global__ __launch_bounds__(256) void t16_kernel(const float* in, uint16_t* out, int64_t rows, int64_t cols,
                                                  int64_t pitch, const int* st, int st_mask, int st_val) {
    const int bz = blockIdx.z;
    if (st && (st[bz] & st_mask) != st_val) return;
    __shared__ float tile[64][65];
    const int64_t i0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    in += bz * rows * cols;
    out += bz * cols * pitch;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int64_t i = i0 + ty + 4 * q, c = c0 + tx;
        tile[ty + 4 * q][tx] = (i < rows && c < cols) ? in[i * cols + c] : 0.f;
    }
    __syncthreads();
    // eight consecutive rows of one column per thread, one 16-byte store; four threads fill the
    // 64 bytes of a (slab, column) row, so a wave writes 1 KB of consecutive memory
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = threadIdx.x + 256 * q, i8 = idx & 3, cl = (idx >> 2) & 63, il = 32 * (idx >> 8) + 8 * i8;
        const int64_t c = c0 + cl, i = i0 + il;
        if (c < cols && i < pitch) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(tile[il + 2 * e][cl], tile[il + 2 * e + 1][cl]);
            *(uint4*)&out[((i >> 5) * cols + c) * kSplitK + (i & 31)] = uint4{w[0], w[1], w[2], w[3]};
        }
    }
}

// LDS tile of the transposed small operand: 256 rows (output columns) by one 32-k slab, bf16,
// swizzled as part_off (16-byte chunks XORed with bits 2..3 of the row).
constexpr int kT16Rows = 256;

// Each of 512 threads stages one row half (16 k) of the 256 x 32 slab: two 16-byte chunks.
// Values outside the operand are loaded from a valid address and zeroed only when stored: a
// register still waiting for its load must not be written, or the compiler waits for every load
// in flight first.
struct SmallSlab {
    uint4 v[2];
    bool ok;
    __device__ __forceinline__ void load(const uint16_t* p, bool in) {
        v[0] = *(const uint4*)p;
        v[1] = *(const uint4*)(p + 8);
        ok = in;
    }
    __device__ __forceinline__ void store(uint16_t* lds, int j, int half) const {
        const uint32_t k = ok ? 0xffffffffu : 0u;   // a bit mask, not a select of aggregates
        *(uint4*)&lds[part_off(j, 2 * half)] = uint4{v[0].x & k, v[0].y & k, v[0].z & k, v[0].w & k};
        *(uint4*)&lds[part_off(j, 2 * half + 1)] = uint4{v[1].x & k, v[1].y & k, v[1].z & k, v[1].w & k};
    }
};

struct Stream16Args {
    const float* M;
    const void* G;
    const uint16_t* T;   // transposed bf16 small operand [b][pitch / 32][r][32] (t16_kernel)
    float* C;            // output [b][rows][r] (P0: rows = m; R: rows = n)
    int64_t m, n, r, pitch;
    const int* st;
    int st_mask, st_val;
};

// P0 = (M + G) Q.  Workgroup: 128 rows of one matrix by output columns [256 y, 256 y + 256).
// Eight waves of 16 rows: lane (fr, fg) owns row 16 w + fr and, in each 32-k step, k = 8 fg ..
// 8 fg + 7, i.e. exactly its MFMA A fragment, loaded from M and G straight into registers.  Loads
// come in super-slabs of KS k-steps, so that one visit reads 128 KS contiguous bytes of each row
// of M (the four lanes of a row side by side), D super-slabs ahead.  The Q^T slabs (256 x 32 bf16
// per k-step) go through double-buffered LDS; sixteen 16 x 16 column blocks per wave.
template <bool G_BF16, int KS, int D>
__global__ __launch_bounds__(512) void p16_kernel(Stream16Args a) {
    const TileId tid = xcd_tile_id();
    const int bz = tid.z;
    if (a.st && (a.st[bz] & a.st_mask) != a.st_val) return;
    const int64_t row0 = (int64_t)tid.x * 128, col0 = (int64_t)tid.y * kT16Rows;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, fr = lane & 15, fg = lane >> 4;
    const int64_t row = row0 + 16 * w + fr;
    const bool rok = row < a.m;
    const int64_t mn = a.m * a.n;
    const int64_t rbase = bz * mn + (rok ? row : 0) * a.n;   // this lane's row (row 0 when outside)
    const int jb = t >> 1, half = t & 1;
    const bool jok = col0 + jb < a.r;
    const uint16_t* Tr = a.T + (int64_t)bz * a.r * a.pitch + (int64_t)(jok ? col0 + jb : 0) * kSplitK + 16 * half;
    const int64_t slab = a.r * kSplitK;   // elements per 32-k slab of the small operand
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][KS][kT16Rows * kSplitK];

    const int nstep = (int)((a.n + kSplitK - 1) / kSplitK);     // 32-k steps
    const int nsup = (nstep + KS - 1) / KS;                       // super-slabs
    const int npad = (nsup + D - 1) / D * D;
    float4 am[D][KS][2];
    uint4 ag[D][KS][G_BF16 ? 1 : 2];
    bool aok[D][KS];
    SmallSlab sb[D][KS];
    auto load = [&](int d, int u) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int st = u * KS + kk;
            const int sc = st < nstep ? st : nstep - 1;          // past the end: re-read the last step
            const int64_t k = (int64_t)sc * kSplitK;
            // n % 8 == 0: the lane's eight k are all inside the row or all outside (then columns 0..7)
            const bool kin = st < nstep && k + 8 * fg < a.n;
            const int64_t o = rbase + (kin ? k + 8 * fg : 0);
            am[d][kk][0] = *(const float4*)(a.M + o);
            am[d][kk][1] = *(const float4*)(a.M + o + 4);
            if constexpr (G_BF16) {
                ag[d][kk][0] = *(const uint4*)((const uint16_t*)a.G + o);
            } else {
                ag[d][kk][0] = *(const uint4*)((const float*)a.G + o);
                ag[d][kk][1] = *(const uint4*)((const float*)a.G + o + 4);
            }
            aok[d][kk] = kin && rok;                              // zeroed in frag(), once loaded
            sb[d][kk].load(Tr + sc * slab, st < nstep && jok);
        }
    };
    auto frag = [&](int d, int kk) -> u32x4 {
        float g[8];
        if constexpr (G_BF16) {
            const uint4 q = ag[d][kk][0];
            const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                g[2 * e] = bf16_bits_to_float(wv[e] & 0xffffu);
                g[2 * e + 1] = bf16_bits_to_float(wv[e] >> 16);
            }
        } else {
            const float4 g0 = *(const float4*)&ag[d][kk][0], g1 = *(const float4*)&ag[d][kk][1];
            g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
        }
        const float4 m0 = am[d][kk][0], m1 = am[d][kk][1];
        const u32x4 f{pack_bf16x2(m0.x + g[0], m0.y + g[1]), pack_bf16x2(m0.z + g[2], m0.w + g[3]),
                      pack_bf16x2(m1.x + g[4], m1.y + g[5]), pack_bf16x2(m1.z + g[6], m1.w + g[7])};
        const uint32_t k = aok[d][kk] ? 0xffffffffu : 0u;
        return u32x4{f[0] & k, f[1] & k, f[2] & k, f[3] & k};
    };
    f32x4 acc[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(d, d);
        __builtin_amdgcn_sched_barrier(0);   // the sets issued in order: set 0's loads complete first
    }
    for (int u0 = 0; u0 < npad; u0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            // keep each stage's conversions after its own loads' wait: hoisting a later set's
            // would make the compiler wait for every load in flight
            __builtin_amdgcn_sched_barrier(0);
            const int u = u0 + d;
            u32x4 af[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                af[kk] = frag(d, kk);
                sb[d][kk].store(lds[u & 1][kk], jb, half);
            }
            load(d, u + D);
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int cb = 0; cb < 16; ++cb) {
                    const u32x4 bf = *(const u32x4*)&lds[u & 1][kk][part_off(16 * cb + fr, fg)];
                    acc[cb] = mma_bf16(af[kk], bf, acc[cb]);
                }
        }
    }
    float* C = a.C + bz * a.m * a.r;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t rr = row0 + 16 * w + 4 * fg + v, cc = col0 + 16 * cb + fr;
            if (rr < a.m && cc < a.r) C[rr * a.r + cc] = acc[cb][v];
        }
}

#ifndef DION_P16_KS
#define DION_P16_KS 1
#endif
#ifndef DION_P16_D
#define DION_P16_D 4
#endif
constexpr int kP16KS = DION_P16_KS, kP16D = DION_P16_D;   // k-steps per super-slab, super-slabs in flight

// R = (M + G)^T P.  Workgroup: 128 columns j of one matrix (rows of R) by output columns
// [256 y, 256 y + 256); the contraction runs over the m rows of B in 32-row slabs.  Each thread
// loads two consecutive rows (pair p) by four columns (group c) of M and G (16- and 8-byte
// vectors), forms bf16 B and writes it transposed into LDS ([j][i], 16-byte chunks of eight i per
// MFMA fragment); P^T's slab goes through LDS as in p16_kernel.  Waves 2 x 4, each 64 j by 64
// output columns.  A wave stages four pairs by sixteen groups (16 lanes read 256 contiguous bytes
// of a row of M), and the chunk of row j sits at chunk ^ ((j >> 4) & 3): the transposed 4-byte
// writes of a wave then fall in 64 distinct banks, and a fragment read (16 consecutive rows, one
// chunk) in distinct 16-byte slots.
constexpr int kR16Pitch = 40;   // bf16 per LDS row of the transposed B slab (32 + 8: rows 16-byte aligned)
__device__ __forceinline__ int r16_off(int j, int i) {   // bf16 offset of (j, i), i even
    return j * kR16Pitch + 8 * (((i >> 3) ^ (j >> 4)) & 3) + (i & 7);
}

template <bool G_BF16>
__global__ __launch_bounds__(512) void r16_kernel(Stream16Args a) {
    constexpr int D = kStreamD;
    const TileId tid = xcd_tile_id();
    const int bz = tid.z;
    if (a.st && (a.st[bz] & a.st_mask) != a.st_val) return;
    const int64_t j0 = (int64_t)tid.x * 128, col0 = (int64_t)tid.y * kT16Rows;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, fr = lane & 15, fg = lane >> 4;
    const int wm = w >> 2, wn = w & 3;
    // staging share of the B slab: rows 2 p, 2 p + 1 and columns 4 c .. 4 c + 3 (see above)
    const int p = 4 * (w & 3) + (lane >> 4), c4 = 4 * (16 * (w >> 2) + (lane & 15));
    const bool cok = j0 + c4 < a.n;          // n % 4 == 0: a group of four is all in or all out
    const int64_t mn = a.m * a.n;
    const int64_t cofs = bz * mn + (cok ? j0 + c4 : 0);
    const int jb = t >> 1, half = t & 1;
    const bool tok = col0 + jb < a.r;
    const uint16_t* Tr = a.T + (int64_t)bz * a.r * a.pitch + (int64_t)(tok ? col0 + jb : 0) * kSplitK + 16 * half;
    const int64_t slab = a.r * kSplitK;
    __shared__ __attribute__((aligned(16))) uint16_t la[2][128 * kR16Pitch];
    __shared__ __attribute__((aligned(16))) uint16_t lb[2][kT16Rows * kSplitK];

    const int nslab = (int)((a.m + kSplitK - 1) / kSplitK);
    const int npad = (nslab + D - 1) / D * D;
    float4 am[D][2];
    uint2 ag[D][G_BF16 ? 2 : 4];
    bool ok0[D], ok1[D];
    SmallSlab sb[D];
    auto load = [&](int d, int s) {
        const int sc = s < nslab ? s : nslab - 1;
        const int64_t i = (int64_t)sc * kSplitK + 2 * p;
        const bool i0ok = s < nslab && i < a.m, i1ok = s < nslab && i + 1 < a.m;
        const int64_t o0 = cofs + (i0ok ? i : 0) * a.n, o1 = cofs + (i1ok ? i + 1 : 0) * a.n;
        am[d][0] = *(const float4*)(a.M + o0);
        am[d][1] = *(const float4*)(a.M + o1);
        if constexpr (G_BF16) {
            ag[d][0] = *(const uint2*)((const uint16_t*)a.G + o0);
            ag[d][1] = *(const uint2*)((const uint16_t*)a.G + o1);
        } else {
            const uint4 g0 = *(const uint4*)((const float*)a.G + o0), g1 = *(const uint4*)((const float*)a.G + o1);
            ag[d][0] = uint2{g0.x, g0.y}; ag[d][1] = uint2{g0.z, g0.w};
            ag[d][2] = uint2{g1.x, g1.y}; ag[d][3] = uint2{g1.z, g1.w};
        }
        ok0[d] = i0ok && cok;                                    // zeroed in stage(), once loaded
        ok1[d] = i1ok && cok;
        sb[d].load(Tr + sc * slab, s < nslab && tok);
    };
    // B values of the two rows, summed in fp32 and rounded to bf16, written at [c4 + e][2 p]
    auto stage = [&](int d, uint16_t* l) {
        float g0[4], g1[4];
        if constexpr (G_BF16) {
            const uint2 a0 = ag[d][0], a1 = ag[d][1];
            g0[0] = bf16_bits_to_float(a0.x & 0xffffu); g0[1] = bf16_bits_to_float(a0.x >> 16);
            g0[2] = bf16_bits_to_float(a0.y & 0xffffu); g0[3] = bf16_bits_to_float(a0.y >> 16);
            g1[0] = bf16_bits_to_float(a1.x & 0xffffu); g1[1] = bf16_bits_to_float(a1.x >> 16);
            g1[2] = bf16_bits_to_float(a1.y & 0xffffu); g1[3] = bf16_bits_to_float(a1.y >> 16);
        } else {
            g0[0] = __uint_as_float(ag[d][0].x); g0[1] = __uint_as_float(ag[d][0].y);
            g0[2] = __uint_as_float(ag[d][1].x); g0[3] = __uint_as_float(ag[d][1].y);
            g1[0] = __uint_as_float(ag[d][2].x); g1[1] = __uint_as_float(ag[d][2].y);
            g1[2] = __uint_as_float(ag[d][3].x); g1[3] = __uint_as_float(ag[d][3].y);
        }
        const float4 m0 = am[d][0], m1 = am[d][1];
        const bool v0 = ok0[d], v1 = ok1[d];
        const float r0[4] = {v0 ? m0.x + g0[0] : 0.f, v0 ? m0.y + g0[1] : 0.f, v0 ? m0.z + g0[2] : 0.f,
                             v0 ? m0.w + g0[3] : 0.f};
        const float r1[4] = {v1 ? m1.x + g1[0] : 0.f, v1 ? m1.y + g1[1] : 0.f, v1 ? m1.z + g1[2] : 0.f,
                             v1 ? m1.w + g1[3] : 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) *(uint32_t*)&l[r16_off(c4 + e, 2 * p)] = pack_bf16x2(r0[e], r1[e]);
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int s0 = 0; s0 < npad; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            __builtin_amdgcn_sched_barrier(0);   // as in p16_kernel: one stage's work per wait
            const int s = s0 + d;
            uint16_t* ba = la[s & 1];
            uint16_t* bb = lb[s & 1];
            stage(d, ba);
            sb[d].store(bb, jb, half);
            load(d, s + D);
            __syncthreads();
            u32x4 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *(const u32x4*)&ba[r16_off(wm * 64 + 16 * i + fr, 8 * fg)];
#pragma unroll
            for (int j = 0; j < 4; ++j) bf[j] = *(const u32x4*)&bb[part_off(wn * 64 + 16 * j + fr, fg)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mma_bf16(af[i], bf[j], acc[i][j]);
        }
    }
    float* C = a.C + bz * a.n * a.r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t rr = j0 + wm * 64 + 16 * i + 4 * fg + v, cc = col0 + wn * 64 + 16 * j + fr;
                if (rr < a.n && cc < a.r) C[rr * a.r + cc] = acc[i][j][v];
            }
}

// Host side: a transposed bf16 copy of the small operand (Q for the product, P for the
// back-projection) into tbuf ([b][stream16_pitch(rows) / 32][r][32] bf16), then the product.  Returns a
// hipError_t value.  The caller has checked stream16_ok().
bool stream16_ok(int64_t n, const void* M, const void* G, int g_bf16, bool backproject) {
    const int64_t need = backproject ? 4 : 8;
    const uintptr_t ga = (uintptr_t)G, ma = (uintptr_t)M;
    return n % need == 0 && (ma & 15u) == 0 && (ga & (g_bf16 ? 7u : 15u)) == 0;
}

int stream16_product(const float* M, const void* G, int g_bf16, const float* small, uint16_t* tbuf, float* C,
                     int64_t m, int64_t n, int64_t r, int64_t b, bool backproject, const int* st, int st_mask,
                     int st_val, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (b <= 0 || r <= 0) return 0;
    // the small operand: Q [n][r] for the product, P [m][r] for the back-projection
    const int64_t rows = backproject ? m : n;
    const int64_t pitch = stream16_pitch(rows);
    dim3 tg((unsigned)((r + 63) / 64), (unsigned)((pitch + 63) / 64), (unsigned)b);
    hipLaunchKernelGGL(t16_kernel, tg, dim3(256), 0, s, small, tbuf, rows, r, pitch, st, st_mask, st_val);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    Stream16Args a{};
    a.M = M; a.G = G; a.T = tbuf; a.C = C;
    a.m = m; a.n = n; a.r = r; a.pitch = pitch;
    a.st = st; a.st_mask = st_mask; a.st_val = st_val;
    const unsigned cy = (unsigned)((r + kT16Rows - 1) / kT16Rows);
    if (!backproject) {
        dim3 grid((unsigned)((m + 127) / 128), cy, (unsigned)b);
        if (g_bf16) hipLaunchKernelGGL((p16_kernel<true, kP16KS, kP16D>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((p16_kernel<false, kP16KS, kP16D>), grid, dim3(512), 0, s, a);
    } else {
        dim3 grid((unsigned)((n + 127) / 128), cy, (unsigned)b);
        if (g_bf16) hipLaunchKernelGGL((r16_kernel<true>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((r16_kernel<false>), grid, dim3(512), 0, s, a);
    }
    return (int)hipGetLastError();
}

}  // namespace dion
