// extern "C" entry points of the Dion step library: argument validation (pure
// host code, no HIP call before every check has passed), workspace sizing,
// status strings.  The launch sequence itself lives in dion_step.hip.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "dion.h"
#include "dion_plan.h"

namespace {

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

bool overlap(const Range& a, const Range& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

Range span(const void* p, double bytes) {
    const uintptr_t lo = (uintptr_t)p;
    return Range{lo, lo + (uintptr_t)bytes};
}

}  // namespace

namespace dion {

int check_step_args(int64_t m, int64_t n, int64_t batch, int64_t rank, float mu, float lr, float eps, int x_dtype,
                    int g_dtype, uint32_t options, Plan* p) {
    if (m < 1 || n < 1 || batch < 0) return DION_ERR_SHAPE;
    if (rank < 0 || rank > (m < n ? m : n)) return DION_ERR_RANK;
    if (!(mu >= 0.0f && mu < 1.0f) || !isfinite(lr) || !isfinite(eps) || !(eps >= 0.0f)) return DION_ERR_HYPER;
    if ((x_dtype != DION_F32 && x_dtype != DION_BF16) || (g_dtype != DION_F32 && g_dtype != DION_BF16))
        return DION_ERR_DTYPE;
    const uint32_t known = DION_OPT_STICKY_F64 | DION_OPT_FORCE_F64 | DION_OPT_FORCE_F32 | DION_OPT_HOUSEHOLDER |
                           DION_OPT_SPECTRAL_SHIFT | DION_OPT_EXACT_PRODUCTS | (15u << DION_OPT_CHUNKS_SHIFT);
    if ((options & ~known) || ((options & DION_OPT_FORCE_F64) && (options & DION_OPT_FORCE_F32)) ||
        ((options & DION_OPT_HOUSEHOLDER) && ((options & DION_OPT_FORCE_F32) || rank > 4096)) ||
        ((options & DION_OPT_SPECTRAL_SHIFT) && (options & DION_OPT_FORCE_F32)))
        return DION_ERR_OPTION;
    if (!make_plan(m, n, batch, rank, p)) return DION_ERR_SHAPE;
    return DION_OK;
}

int check_step_buffers(const Plan& p, const void* X, const void* G, const float* M, const float* Q, int x_dtype,
                       int g_dtype, const void* workspace, size_t workspace_bytes, const int32_t* flags) {
    if (!X || !G || !M || (p.r > 0 && !Q) || !workspace) return DION_ERR_NULL;
    if (((uintptr_t)X | (uintptr_t)G | (uintptr_t)M | (uintptr_t)Q | (uintptr_t)flags) & 15u) return DION_ERR_ALIGN;
    if ((uintptr_t)workspace & 255u) return DION_ERR_ALIGN;
    if (workspace_bytes < p.total) return DION_ERR_WORKSPACE;
    const double mn = (double)p.b * (double)p.m * (double)p.n;
    const Range rs[6] = {
        span(X, mn * (x_dtype == DION_BF16 ? 2 : 4)),
        span(G, mn * (g_dtype == DION_BF16 ? 2 : 4)),
        span(M, mn * 4),
        span(Q, p.r > 0 ? (double)p.b * (double)p.n * (double)p.r * 4 : 0.0),
        span(workspace, (double)p.total),
        span(flags, flags ? (double)p.b * 4 : 0.0),
    };
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (overlap(rs[i], rs[j])) return DION_ERR_OVERLAP;
    return DION_OK;
}

}  // namespace dion

extern "C" {

size_t dion_workspace_size(int64_t m, int64_t n, int64_t batch, int64_t rank) {
    dion::Plan p;
    if (!dion::make_plan(m, n, batch, rank, &p)) return 0;
    return p.total;
}

int dion_step_batched_ex(void* X, const void* G, float* M, float* Q, int64_t m, int64_t n, int64_t batch,
                         int64_t rank, float mu, float lr, float eps, int x_dtype, int g_dtype, void* workspace,
                         size_t workspace_bytes, int32_t* flags, uint32_t options, void* stream,
                         const dion_step_outputs* out) {
    dion::Plan p;
    int st = dion::check_step_args(m, n, batch, rank, mu, lr, eps, x_dtype, g_dtype, options, &p);
    if (st != DION_OK || batch == 0) return st;
    st = dion::check_step_buffers(p, X, G, M, Q, x_dtype, g_dtype, workspace, workspace_bytes, flags);
    if (st != DION_OK) return st;
    float* rmmc = out ? out->rmmc : nullptr;
    if (rmmc) {
        if ((uintptr_t)rmmc & 3u) return DION_ERR_ALIGN;
        const double mn = (double)batch * (double)m * (double)n;
        const Range r = span(rmmc, (double)batch * 4);
        const Range others[6] = {span(X, mn * (x_dtype == DION_BF16 ? 2 : 4)), span(G, mn * (g_dtype == DION_BF16 ? 2 : 4)),
                                 span(M, mn * 4), span(Q, rank > 0 ? (double)batch * (double)n * (double)rank * 4 : 0.0),
                                 span(workspace, (double)p.total), span(flags, flags ? (double)batch * 4 : 0.0)};
        for (const Range& o : others)
            if (overlap(r, o)) return DION_ERR_OVERLAP;
    }
    const int e = dion::run_step(p, X, G, M, Q, mu, lr, eps, x_dtype == DION_BF16, g_dtype == DION_BF16,
                                 (char*)workspace, flags, options, stream, out ? out->events : nullptr, rmmc);
    return e ? DION_ERR_HIP - e : DION_OK;
}

int dion_step_batched_profiled(void* X, const void* G, float* M, float* Q, int64_t m, int64_t n, int64_t batch,
                               int64_t rank, float mu, float lr, float eps, int x_dtype, int g_dtype,
                               void* workspace, size_t workspace_bytes, int32_t* flags, uint32_t options,
                               void* stream, void* const* events) {
    const dion_step_outputs out{events, nullptr};
    return dion_step_batched_ex(X, G, M, Q, m, n, batch, rank, mu, lr, eps, x_dtype, g_dtype, workspace,
                                workspace_bytes, flags, options, stream, &out);
}

int dion_step_batched(void* X, const void* G, float* M, float* Q, int64_t m, int64_t n, int64_t batch, int64_t rank,
                      float mu, float lr, float eps, int x_dtype, int g_dtype, void* workspace,
                      size_t workspace_bytes, int32_t* flags, uint32_t options, void* stream) {
    return dion_step_batched_profiled(X, G, M, Q, m, n, batch, rank, mu, lr, eps, x_dtype, g_dtype, workspace,
                                      workspace_bytes, flags, options, stream, nullptr);
}

int dion_adamw_step(void* param, const void* grad, float* exp_avg, float* exp_avg_sq, int64_t n, int64_t t,
                    float lr, float beta1, float beta2, float eps, float weight_decay, int p_dtype, int g_dtype,
                    void* stream) {
    if (n < 0 || n > ((int64_t)1 << 46)) return DION_ERR_SHAPE;
    if (t < 1 || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !isfinite(lr) ||
        !isfinite(weight_decay) || !isfinite(eps) || !(eps >= 0.0f))
        return DION_ERR_HYPER;
    if ((p_dtype != DION_F32 && p_dtype != DION_BF16) || (g_dtype != DION_F32 && g_dtype != DION_BF16))
        return DION_ERR_DTYPE;
    if (n == 0) return DION_OK;
    if (!param || !grad || !exp_avg || !exp_avg_sq) return DION_ERR_NULL;
    if (((uintptr_t)param | (uintptr_t)grad | (uintptr_t)exp_avg | (uintptr_t)exp_avg_sq) & 15u) return DION_ERR_ALIGN;
    const double dn = (double)n;
    const Range rs[4] = {span(param, dn * (p_dtype == DION_BF16 ? 2 : 4)), span(grad, dn * (g_dtype == DION_BF16 ? 2 : 4)),
                         span(exp_avg, dn * 4), span(exp_avg_sq, dn * 4)};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(rs[i], rs[j])) return DION_ERR_OVERLAP;
    const int e = dion::run_adamw(param, grad, exp_avg, exp_avg_sq, n, t, lr, beta1, beta2, eps, weight_decay,
                                  p_dtype == DION_BF16, g_dtype == DION_BF16, stream);
    return e ? DION_ERR_HIP - e : DION_OK;
}

int dion_lion_step(void* param, const void* grad, float* exp_avg, int64_t n, float lr, float beta1, float beta2,
                   float weight_decay, int p_dtype, int g_dtype, void* stream) {
    if (n < 0 || n > ((int64_t)1 << 46)) return DION_ERR_SHAPE;
    if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !isfinite(lr) ||
        !isfinite(weight_decay))
        return DION_ERR_HYPER;
    if ((p_dtype != DION_F32 && p_dtype != DION_BF16) || (g_dtype != DION_F32 && g_dtype != DION_BF16))
        return DION_ERR_DTYPE;
    if (n == 0) return DION_OK;
    if (!param || !grad || !exp_avg) return DION_ERR_NULL;
    if (((uintptr_t)param | (uintptr_t)grad | (uintptr_t)exp_avg) & 15u) return DION_ERR_ALIGN;
    const double dn = (double)n;
    const Range rs[3] = {span(param, dn * (p_dtype == DION_BF16 ? 2 : 4)), span(grad, dn * (g_dtype == DION_BF16 ? 2 : 4)),
                         span(exp_avg, dn * 4)};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlap(rs[i], rs[j])) return DION_ERR_OVERLAP;
    const int e = dion::run_lion(param, grad, exp_avg, n, lr, beta1, beta2, weight_decay, p_dtype == DION_BF16,
                                 g_dtype == DION_BF16, stream);
    return e ? DION_ERR_HIP - e : DION_OK;
}

size_t dion_lambda_max_workspace_size(int64_t r, int64_t batch, int32_t k) {
    if (r < 1 || r > ((int64_t)1 << 24) || batch < 0 || batch > 65535 || k < 1 || k > dion::kMpiMaxPool) return 0;
    return (size_t)batch * (size_t)(2 * r * k + 2) * sizeof(double);
}

int dion_lambda_max_batched(const double* W, int64_t r, int64_t batch, const double* V0, int32_t k, int32_t iters,
                            double* lambda, void* workspace, size_t workspace_bytes, void* stream) {
    if (r < 1 || r > ((int64_t)1 << 24) || batch < 0 || batch > 65535 || k < 1 || k > dion::kMpiMaxPool ||
        (double)r * (double)r * (double)batch > 1.0e15)
        return DION_ERR_SHAPE;
    if (iters < 0 || iters > dion::kMpiMaxIters) return DION_ERR_HYPER;
    if (batch == 0) return DION_OK;
    if (!W || !lambda || !workspace) return DION_ERR_NULL;
    if ((((uintptr_t)W | (uintptr_t)V0 | (uintptr_t)lambda) & 7u) || ((uintptr_t)workspace & 255u)) return DION_ERR_ALIGN;
    const size_t need = dion_lambda_max_workspace_size(r, batch, k);
    if (workspace_bytes < need) return DION_ERR_WORKSPACE;
    const double b = (double)batch;
    const Range rs[4] = {span(lambda, b * 8), span(workspace, (double)need), span(W, b * r * r * 8),
                         span(V0, V0 ? b * r * k * 8 : 0.0)};
    for (int i = 0; i < 2; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(rs[i], rs[j])) return DION_ERR_OVERLAP;
    dion::MpiArgs a{};
    a.W = W; a.r = r; a.k = k; a.V0 = V0; a.first = 0;
    a.ws = (double*)workspace; a.ws_stride = 2 * r * k + 2;
    a.lam = lambda; a.lam_stride = 1;
    a.st = nullptr;
    const int e = dion::run_lambda_max(a, batch, iters, stream);
    return e ? DION_ERR_HIP - e : DION_OK;
}

const char* dion_strerror(int status) {
    switch (status) {
        case DION_OK: return "success";
        case DION_ERR_NULL: return "a required pointer is NULL";
        case DION_ERR_SHAPE: return "invalid shape (m, n >= 1, batch >= 0) or size overflow";
        case DION_ERR_RANK: return "rank outside [0, min(m, n)]";
        case DION_ERR_HYPER: return "invalid hyper-parameter (mu, betas in [0,1), finite lr and decay, finite eps >= 0, step >= 1, iterations 0..64)";
        case DION_ERR_ALIGN: return "misaligned pointer (16 bytes, 8 for fp64 arrays; workspace 256 bytes)";
        case DION_ERR_OVERLAP: return "overlapping buffers";
        case DION_ERR_WORKSPACE: return "workspace smaller than dion_workspace_size()";
        case DION_ERR_DTYPE: return "unsupported dtype (DION_F32 or DION_BF16)";
        case DION_ERR_OPTION: return "unknown or contradictory option bits";
        case DION_ERR_SCRATCH: return "stack too large for the built-in scratch of dion_step_batched_noalloc "
                                      "(DION_NOALLOC_SCRATCH_BYTES); call dion_step_batched with a workspace";
        default: break;
    }
    if (status <= DION_ERR_HIP) return "HIP runtime error (status = -100 - hipError_t)";
    return "unknown status";
}

int dion_version(void) { return 100; }

}  // extern "C"
