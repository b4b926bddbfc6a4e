// Workspace planner and internal launch interface of the Dion step.
// Pure host code: the sizes and offsets below are computed without any HIP call.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace dion {

// Block size of the blocked Cholesky / triangular solves (rank is cut into
// column blocks of this width; the last one may be narrower).
constexpr int kNB = 64;
// Row chunk of the column-norm partial sums.
constexpr int kNormChunk = 64;

// Per-matrix state word kept in the workspace during a call.
enum : int {
    ST_PATH64 = 1,   // the fp64 chain owns this matrix
    ST_SHIFT = 2,    // the fp64 chain needs the shifted first pass (and a third pass)
    ST_FAIL = 4,     // a factorization broke down with no further fallback
    ST_CHOL2 = 8,    // this re-orthonormalization pass uses the Cholesky path (P^T P far from I)
    ST_HH = 16,      // P came from the fp64 Householder QR
};

// Partial sums of squares per matrix written by the near-identity test (fixed-order reduction).
constexpr int kNearIdParts = 256;

// Multi-power-iteration estimate of the largest eigenvalue: pool size limit, and the pool size and
// iteration count the step uses for the shift of its shifted CholeskyQR pass.
constexpr int kMpiMaxPool = 32;
constexpr int kMpiMaxIters = 64;
constexpr int kShiftPool = 32;
constexpr int kShiftIters = 10;

// Row pitch (elements) of the transposed bf16 copy of Q or P used by the plain bf16 products:
// rows padded with zeros to whole 32-wide slabs.
inline int64_t stream16_pitch(int64_t rows) { return (rows + 31) / 32 * 32; }

struct Plan {
    int64_t m, n, b, r;
    int64_t nblk;      // number of rank column blocks
    int64_t nchunk;    // row chunks of the column-norm reduction
    int64_t gsplit;    // K-splits of the fp64 Gram products (partials reduced in fixed order)
    int64_t gsplit6;   // K-splits of the fp32 Gram products (split-bf16 kernel, 128 x 128 tiles)
    int64_t kp;        // rank padded to a multiple of 32 (k-slabs of the split-bf16 weight pass)
    int64_t c0;        // index of the first matrix (0, or a chunk's offset in the whole stack)
    // byte offsets into the workspace (all 256-byte aligned)
    size_t P32, R32, cs, st, kap, emax, W, L, Td, Tf, P64, P64b, R64, part, gpart, pw, mx, t16;
    size_t total;
    // bytes per matrix of each region (a region is [batch][...] and contiguous)
    size_t sP32, sR32, scs, sst, skap, semax, sW, sL, sTd, sTf, sP64, sP64b, sR64, spart, sgpart, spw, smx, st16;
    int64_t nmx;       // momentum-change partials per matrix (one per 64 x 64 block of M)
};

// The sub-plan of matrices [c0, c0 + cb): same sizes, region offsets advanced to matrix c0.
inline Plan chunk_plan(const Plan& p, int64_t c0, int64_t cb) {
    Plan q = p;
    q.b = cb;
    q.c0 = p.c0 + c0;
    const size_t c = (size_t)c0;
    q.P32 += c * p.sP32; q.R32 += c * p.sR32; q.cs += c * p.scs; q.st += c * p.sst; q.kap += c * p.skap; q.emax += c * p.semax;
    q.W += c * p.sW; q.L += c * p.sL; q.Td += c * p.sTd; q.Tf += c * p.sTf; q.P64 += c * p.sP64;
    q.P64b += c * p.sP64b; q.R64 += c * p.sR64; q.part += c * p.spart; q.gpart += c * p.sgpart;
    q.pw += c * p.spw; q.mx += c * p.smx; q.t16 += c * p.st16;
    return q;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Returns false when the sizes overflow or are invalid.
inline bool make_plan(int64_t m, int64_t n, int64_t b, int64_t r, Plan* p) {
    if (m < 1 || n < 1 || b < 0 || r < 0 || r > (m < n ? m : n)) return false;
    const int64_t lim = (int64_t)1 << 40;
    if (m > lim || n > lim || b > lim || (double)m * (double)n * (double)(b ? b : 1) > 9.0e15) return false;
    Plan q{};
    q.m = m; q.n = n; q.b = b; q.r = r;
    q.nblk = (r + kNB - 1) / kNB;
    q.nchunk = (n + kNormChunk - 1) / kNormChunk;
    q.kp = (r + 31) / 32 * 32;
    {   // split the Gram's long K (= m) over the grid: the fewest splits that give the launch at
        // least 1.5 64 x 64 workgroups per CU (measured on 24 x 1024 x 256: two splits, about 1.9
        // workgroups per CU, beat one split (0.9, too few waves to hide latency) and four (3.75,
        // twice the partials and each workgroup's fill and drain over a quarter of the K range)),
        // keeping >= 128 rows per split and the partials within 512 MB
        const int64_t nt = (r + 63) / 64;
        const int64_t tiles = nt * (nt + 1) / 2 * (b > 0 ? b : 1);
        int64_t best = 1;
        for (int64_t s = 2; s <= 16 && best * tiles < 384; ++s) {
            if (s > m / 128 || (double)(b > 0 ? b : 1) * s * r * r * 8 > 512.0 * (1 << 20)) break;
            best = s;
        }
        q.gsplit = tiles > 0 ? best : 1;
    }
    {   // the same model for the fp32 Gram on the split-bf16 kernel: one 128 x 128 workgroup per
        // CU, 32-k slabs, >= 256 rows per split
        const int64_t nt = (r + 127) / 128;
        const int64_t tiles = nt * (nt + 1) / 2 * (b > 0 ? b : 1);
        const int64_t slots = 256, slabs = (m + 31) / 32;
        int64_t best = 1;
        double best_cost = 0.0;
        for (int64_t s = 1; s <= 16; ++s) {
            if (s > 1 && (s > m / 256 || (double)(b > 0 ? b : 1) * s * r * r * 4 > 512.0 * (1 << 20))) break;
            const double rounds = (double)((s * tiles + slots - 1) / slots);
            const double cost = rounds * (double)((slabs + s - 1) / s + 3);
            if (s == 1 || cost < best_cost) { best = s; best_cost = cost; }
        }
        q.gsplit6 = tiles > 0 ? best : 1;
    }
    size_t off = 0;
    auto take = [&](double bytes) { size_t o = off; off = align256(off + (size_t)bytes); return o; };
    const double B = (double)b;
    q.P32 = take(B * m * r * 4);           // fp32 P (fp32 chain works in place here; weight pass)
    q.R32 = take(B * n * r * 4);           // fp32 R (weight pass)
    q.cs = take(B * r * 8);                // 1 / (||r_j|| + eps), fp64
    q.st = take(B * 4);                    // state words
    q.kap = take(B * 2 * 8);               // running min / max Cholesky diagonal
    q.emax = take(B * kNearIdParts * 8);   // partial sums of |P^T P - I|^2 of a re-orthonormalization pass
    q.W = take(B * r * r * 8);             // Gram matrix (fp32 or fp64)
    q.L = take(B * r * r * 8);             // Cholesky factor, in place
    q.Td = take(B * q.nblk * kNB * kNB * 8);   // inverses of the diagonal blocks
    q.Tf = take(B * r * r * 8);            // full inverse L^-1 (lower)
    q.P64 = take(B * m * r * 8);           // fp64 chain P
    q.P64b = take(B * m * r * 8);          // second P buffer (fp64 chain; fp32 chain's scratch)
    q.R64 = take(B * n * r * 8);           // fp64 chain R
    q.part = take(B * q.nchunk * r * 8);   // column-norm partial sums (fp64)
    const double gp64 = q.gsplit > 1 ? (double)q.gsplit * r * r * 8 : 0.0;
    const double gp32 = q.gsplit6 > 1 ? (double)q.gsplit6 * r * r * 4 : 0.0;
    const double gpm = gp64 > gp32 ? gp64 : gp32;
    q.gpart = take(B * gpm);               // Gram partials (either chain)
    const double pw = (2.0 * r * kShiftPool + 2) * 8;
    q.pw = take(B * pw);                   // spectral-shift pool: two r x 32 fp64 buffers, trace, estimate
    q.t16 = take(B * r * stream16_pitch(m > n ? m : n) * 2);   // transposed bf16 Q or P (plain bf16 products)
    q.nmx = ((m + 63) / 64) * ((n + 63) / 64);
    q.mx = take(B * q.nmx * 2 * 4);        // per block of M: max |M' - M| and max |M| (fp32)
    q.total = off;
    if (q.total > ((size_t)1 << 46)) return false;
    q.sP32 = (size_t)(m * r * 4); q.sR32 = (size_t)(n * r * 4); q.scs = (size_t)(r * 8); q.sst = 4; q.skap = 16; q.semax = kNearIdParts * 8;
    q.sW = q.sL = q.sTf = (size_t)(r * r * 8); q.sTd = (size_t)(q.nblk * kNB * kNB * 8);
    q.sP64 = q.sP64b = (size_t)(m * r * 8); q.sR64 = (size_t)(n * r * 8); q.spart = (size_t)(q.nchunk * r * 8);
    q.sgpart = (size_t)gpm;
    q.spw = (size_t)pw;
    q.smx = (size_t)(q.nmx * 2 * 4);
    q.st16 = (size_t)(r * stream16_pitch(m > n ? m : n) * 2);
    *p = q;
    return true;
}

// Host-side validation of a dion_step_batched call, before anything touches the GPU (DION_*
// status codes).  check_step_args: sizes, hyper-parameters, dtypes and options, and the
// workspace plan.  check_step_buffers: null pointers, alignment, workspace size, overlaps.
int check_step_args(int64_t m, int64_t n, int64_t batch, int64_t rank, float mu, float lr, float eps, int x_dtype,
                    int g_dtype, uint32_t options, Plan* p);
int check_step_buffers(const Plan& p, const void* X, const void* G, const float* M, const float* Q, int x_dtype,
                       int g_dtype, const void* workspace, size_t workspace_bytes, const int32_t* flags);

// Run the step (arguments already validated).  Returns a hipError_t value.
// rmmc: null, or device fp32 [b] for the relative maximum momentum change of each matrix.
int run_step(const Plan& p, void* X, const void* G, float* M, float* Q,
             float mu, float lr, float eps, int x_bf16, int g_bf16,
             char* ws, int32_t* flags, uint32_t options, void* stream, void* const* events,
             float* rmmc = nullptr);

// Multi-power-iteration estimate of lambda_max for a stack of symmetric PSD matrices (only the
// lower triangle of W is read).  Per matrix bz: pool and trace in ws + bz * ws_stride (doubles:
// two r x k buffers, then the trace), the estimate written to lam[bz * lam_stride].  V0 is
// [b][r][k] or null (SplitMix64 start vectors, counted from matrix index first + bz, so that a
// matrix gets the same vectors whichever chunk it runs in); st null runs every matrix, else only
// those with (st[bz] & st_mask) == st_val.
struct MpiArgs {
    const double* W;
    int64_t r;
    int k;
    const double* V0;
    int64_t first;
    double* ws;
    int64_t ws_stride;
    double* lam;
    int64_t lam_stride;
    const int* st;
    int st_mask, st_val;
};
// Enqueues 1 + (iters + 1) + 1 launches; returns a hipError_t value.
int run_lambda_max(const MpiArgs& a, int64_t b, int iters, void* stream);

// Plain bf16 products streaming B = M + G once (stream16.hip).  stream16_ok: the shapes and
// alignments their vector loads need (n % 8 == 0 for the product, n % 4 == 0 for the
// back-projection; M 16-byte and G 8- or 16-byte aligned).  stream16_product: P0 = (M + G) Q
// (backproject false, small = Q) or R = (M + G)^T P (true, small = P) into C, for the matrices
// with (st & mask) == val, using tbuf (>= b r stream16_pitch(rows) bf16) for the transposed
// small operand, stored in contiguous 32-row slabs; returns a hipError_t value.
bool stream16_ok(int64_t n, const void* M, const void* G, int g_bf16, bool backproject);
int stream16_product(const float* M, const void* G, int g_bf16, const float* small, uint16_t* tbuf, float* C,
                     int64_t m, int64_t n, int64_t r, int64_t b, bool backproject, const int* st, int st_mask,
                     int st_val, void* stream);

// Element-wise optimizers (arguments already validated).  Return a hipError_t value.
int run_adamw(void* p, const void* g, float* m, float* v, int64_t n, int64_t t, float lr, float b1, float b2,
              float eps, float wd, int p_bf16, int g_bf16, void* stream);
int run_lion(void* p, const void* g, float* m, int64_t n, float lr, float b1, float b2, float wd, int p_bf16,
             int g_bf16, void* stream);

}  // namespace dion
