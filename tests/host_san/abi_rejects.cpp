// Drives the C ABI's host validation through its rejection cases with fake device addresses
// (never dereferenced: every case must be decided on the host), plus the size queries and a
// few accepted calls that reach the device stubs.  Built with the sanitizers by
// tests/test_host_sanitizers.py; exits nonzero on the first unexpected status.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dion.h"

extern int g_stub_calls;

static int failures = 0;
static void expect(const char* what, long got, long want) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: got %ld, want %ld\n", what, got, want);
        ++failures;
    }
}

static const uintptr_t BASE = (uintptr_t)1 << 40, MB = (uintptr_t)1 << 20;
static void* P(uintptr_t a) { return (void*)a; }

struct StepArgs {
    uintptr_t X = BASE, G = BASE + 64 * MB, M = BASE + 128 * MB, Q = BASE + 192 * MB;
    int64_t m = 64, n = 96, batch = 2, rank = 8;
    float mu = 0.95f, lr = 0.01f, eps = 1e-8f;
    int x_dtype = 0, g_dtype = 0;
    uintptr_t ws = BASE + 256 * MB;
    size_t ws_bytes = (size_t)1 << 30;
    uintptr_t flags = 0;
    uint32_t options = 0;
    uintptr_t rmmc = 0;
};

static int step(const StepArgs& a) {
    dion_step_outputs out;
    out.events = nullptr;
    out.rmmc = (float*)P(a.rmmc);
    return dion_step_batched_ex(P(a.X), P(a.G), (float*)P(a.M), (float*)P(a.Q), a.m, a.n, a.batch, a.rank, a.mu,
                                a.lr, a.eps, a.x_dtype, a.g_dtype, P(a.ws), a.ws_bytes, (int32_t*)P(a.flags),
                                a.options, nullptr, &out);
}

int main() {
    const float nan = NAN, inf = INFINITY;
    // dion_step_batched: one field changed from a valid call per case
    struct Case { const char* name; void (*edit)(StepArgs&); int want; };
    const Case cases[] = {
        {"m=0", [](StepArgs& a) { a.m = 0; }, DION_ERR_SHAPE},
        {"n<0", [](StepArgs& a) { a.n = -3; }, DION_ERR_SHAPE},
        {"batch<0", [](StepArgs& a) { a.batch = -1; }, DION_ERR_SHAPE},
        {"huge m*n", [](StepArgs& a) { a.m = (int64_t)1 << 40; a.n = (int64_t)1 << 40; }, DION_ERR_SHAPE},
        {"rank>min", [](StepArgs& a) { a.rank = 65; }, DION_ERR_RANK},
        {"rank<0", [](StepArgs& a) { a.rank = -1; }, DION_ERR_RANK},
        {"mu=1", [](StepArgs& a) { a.mu = 1.0f; }, DION_ERR_HYPER},
        {"mu<0", [](StepArgs& a) { a.mu = -0.1f; }, DION_ERR_HYPER},
        {"lr nan", [](StepArgs& a) { a.lr = NAN; }, DION_ERR_HYPER},
        {"eps<0", [](StepArgs& a) { a.eps = -1e-8f; }, DION_ERR_HYPER},
        {"eps inf", [](StepArgs& a) { a.eps = INFINITY; }, DION_ERR_HYPER},
        {"x_dtype", [](StepArgs& a) { a.x_dtype = 2; }, DION_ERR_DTYPE},
        {"g_dtype", [](StepArgs& a) { a.g_dtype = -1; }, DION_ERR_DTYPE},
        {"option 8", [](StepArgs& a) { a.options = 8; }, DION_ERR_OPTION},
        {"f32+f64", [](StepArgs& a) { a.options = DION_OPT_FORCE_F32 | DION_OPT_FORCE_F64; }, DION_ERR_OPTION},
        {"hh+f32", [](StepArgs& a) { a.options = DION_OPT_HOUSEHOLDER | DION_OPT_FORCE_F32; }, DION_ERR_OPTION},
        {"hh rank", [](StepArgs& a) { a.options = DION_OPT_HOUSEHOLDER; a.m = a.n = a.rank = 4097; a.batch = 1; },
         DION_ERR_OPTION},
        {"option 128", [](StepArgs& a) { a.options = 128; }, DION_ERR_OPTION},
        {"spectral+f32", [](StepArgs& a) { a.options = DION_OPT_SPECTRAL_SHIFT | DION_OPT_FORCE_F32; },
         DION_ERR_OPTION},
        {"X null", [](StepArgs& a) { a.X = 0; }, DION_ERR_NULL},
        {"Q null", [](StepArgs& a) { a.Q = 0; }, DION_ERR_NULL},
        {"ws null", [](StepArgs& a) { a.ws = 0; }, DION_ERR_NULL},
        {"M align", [](StepArgs& a) { a.M += 4; }, DION_ERR_ALIGN},
        {"flags align", [](StepArgs& a) { a.flags = BASE + 300 * MB + 8; }, DION_ERR_ALIGN},
        {"ws align", [](StepArgs& a) { a.ws += 16; }, DION_ERR_ALIGN},
        {"rmmc align", [](StepArgs& a) { a.rmmc = BASE + 400 * MB + 2; }, DION_ERR_ALIGN},
        {"ws small", [](StepArgs& a) { a.ws_bytes = 1024; }, DION_ERR_WORKSPACE},
        {"G overlaps X", [](StepArgs& a) { a.G = BASE + 1024; }, DION_ERR_OVERLAP},
        {"Q overlaps M", [](StepArgs& a) { a.Q = BASE + 128 * MB + 4096; }, DION_ERR_OVERLAP},
        {"flags in ws", [](StepArgs& a) { a.flags = BASE + 256 * MB + 512; }, DION_ERR_OVERLAP},
        {"rmmc in X", [](StepArgs& a) { a.rmmc = BASE + 64; }, DION_ERR_OVERLAP},
    };
    for (const Case& c : cases) {
        StepArgs a;
        c.edit(a);
        expect(c.name, step(a), c.want);
    }
    expect("no device call for a rejected step", g_stub_calls, 0);
    {   // empty batch: nothing to do, nothing checked beyond the sizes
        StepArgs a;
        a.batch = 0; a.X = a.G = a.M = a.Q = a.ws = 0;
        expect("empty batch", step(a), DION_OK);
    }
    {   // accepted: reaches the device and passes its status on
        StepArgs a;
        expect("accepted step", step(a), -100 - 7);
        expect("one device call", g_stub_calls, 1);
        a.rank = 0; a.Q = 0;
        expect("rank 0, no Q", step(a), -100 - 7);
    }
    // the size queries (overflowing sizes give 0, not a wrapped size)
    expect("ws size batch 0", (long)dion_workspace_size(64, 96, 0, 8), 0);
    expect("ws size bad rank", (long)dion_workspace_size(64, 96, 2, 65), 0);
    expect("ws size overflow", (long)dion_workspace_size((int64_t)1 << 40, (int64_t)1 << 40, 1 << 20, 1 << 20), 0);
    if (dion_workspace_size(64, 96, 2, 8) == 0) { fprintf(stderr, "FAIL ws size of a valid call\n"); ++failures; }
    expect("lambda ws size", (long)dion_lambda_max_workspace_size(256, 4, 32), 4L * (2 * 256 * 32 + 2) * 8);
    expect("lambda ws k=33", (long)dion_lambda_max_workspace_size(256, 4, 33), 0);
    for (int st = -120; st <= 10; ++st)
        if (!dion_strerror(st) || !dion_strerror(st)[0]) { fprintf(stderr, "FAIL strerror %d\n", st); ++failures; }
    if (dion_version() <= 0) { fprintf(stderr, "FAIL version\n"); ++failures; }

    // element-wise optimizers
    const int calls0 = g_stub_calls;
    auto adamw = [&](uintptr_t p, uintptr_t g, uintptr_t m, uintptr_t v, int64_t n, int64_t t, float lr, float b1,
                     float b2, float eps, float wd, int pd) {
        return dion_adamw_step(P(p), P(g), (float*)P(m), (float*)P(v), n, t, lr, b1, b2, eps, wd, pd, 0, nullptr);
    };
    const uintptr_t p0 = BASE, g0 = BASE + 64 * MB, m0 = BASE + 128 * MB, v0 = BASE + 192 * MB;
    expect("adamw n<0", adamw(p0, g0, m0, v0, -1, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0), DION_ERR_SHAPE);
    expect("adamw t=0", adamw(p0, g0, m0, v0, 1000, 0, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0), DION_ERR_HYPER);
    expect("adamw b1=1", adamw(p0, g0, m0, v0, 1000, 1, 1e-3f, 1.0f, 0.999f, 1e-8f, 0.f, 0), DION_ERR_HYPER);
    expect("adamw lr inf", adamw(p0, g0, m0, v0, 1000, 1, inf, 0.9f, 0.999f, 1e-8f, 0.f, 0), DION_ERR_HYPER);
    expect("adamw wd nan", adamw(p0, g0, m0, v0, 1000, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, nan, 0), DION_ERR_HYPER);
    expect("adamw dtype", adamw(p0, g0, m0, v0, 1000, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 3), DION_ERR_DTYPE);
    expect("adamw null", adamw(0, g0, m0, v0, 1000, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0), DION_ERR_NULL);
    expect("adamw align", adamw(p0, g0 + 8, m0, v0, 1000, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0), DION_ERR_ALIGN);
    expect("adamw overlap", adamw(p0, BASE + 2048, m0, v0, 1000, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0),
           DION_ERR_OVERLAP);
    expect("adamw empty", adamw(0, 0, 0, 0, 0, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.f, 0), DION_OK);
    auto lion = [&](uintptr_t p, uintptr_t g, uintptr_t m, int64_t n, float lr, float b1, float b2, int gd) {
        return dion_lion_step(P(p), P(g), (float*)P(m), n, lr, b1, b2, 0.f, 0, gd, nullptr);
    };
    expect("lion n<0", lion(p0, g0, m0, -1, 1e-4f, 0.9f, 0.99f, 0), DION_ERR_SHAPE);
    expect("lion b2=1", lion(p0, g0, m0, 1000, 1e-4f, 0.9f, 1.0f, 0), DION_ERR_HYPER);
    expect("lion lr nan", lion(p0, g0, m0, 1000, nan, 0.9f, 0.99f, 0), DION_ERR_HYPER);
    expect("lion dtype", lion(p0, g0, m0, 1000, 1e-4f, 0.9f, 0.99f, 7), DION_ERR_DTYPE);
    expect("lion null", lion(p0, g0, 0, 1000, 1e-4f, 0.9f, 0.99f, 0), DION_ERR_NULL);
    expect("lion align", lion(p0 + 4, g0, m0, 1000, 1e-4f, 0.9f, 0.99f, 0), DION_ERR_ALIGN);
    expect("lion overlap", lion(p0, g0, BASE + 1024, 1000, 1e-4f, 0.9f, 0.99f, 0), DION_ERR_OVERLAP);
    expect("no device call for a rejected element-wise step", g_stub_calls, calls0);

    // lambda_max estimate
    auto lam = [&](uintptr_t W, int64_t r, int64_t b, uintptr_t V0, int k, int it, uintptr_t l, uintptr_t ws,
                   size_t wsb) {
        return dion_lambda_max_batched((const double*)P(W), r, b, (const double*)P(V0), k, it, (double*)P(l), P(ws),
                                       wsb, nullptr);
    };
    const size_t lws = dion_lambda_max_workspace_size(256, 4, 32);
    const uintptr_t L = BASE + 64 * MB, WS = BASE + 128 * MB;
    expect("lam r=0", lam(BASE, 0, 4, 0, 32, 10, L, WS, lws), DION_ERR_SHAPE);
    expect("lam batch", lam(BASE, 256, 65536, 0, 32, 10, L, WS, lws), DION_ERR_SHAPE);
    expect("lam k=33", lam(BASE, 256, 4, 0, 33, 10, L, WS, lws), DION_ERR_SHAPE);
    expect("lam iters", lam(BASE, 256, 4, 0, 32, 65, L, WS, lws), DION_ERR_HYPER);
    expect("lam W null", lam(0, 256, 4, 0, 32, 10, L, WS, lws), DION_ERR_NULL);
    expect("lam V0 align", lam(BASE, 256, 4, BASE + 32 * MB + 12, 32, 10, L, WS, lws), DION_ERR_ALIGN);
    expect("lam ws small", lam(BASE, 256, 4, 0, 32, 10, L, WS, 1000), DION_ERR_WORKSPACE);
    expect("lam in W", lam(BASE, 256, 4, 0, 32, 10, BASE + 8, WS, lws), DION_ERR_OVERLAP);
    expect("lam V0 in ws", lam(BASE, 256, 4, WS, 32, 10, L, WS, lws), DION_ERR_OVERLAP);
    expect("lam empty", lam(0, 256, 0, 0, 32, 10, 0, 0, 0), DION_OK);
    expect("no device call for a rejected estimate", g_stub_calls, calls0);
    expect("accepted estimate", lam(BASE, 256, 4, 0, 32, 10, L, WS, lws), -100 - 7);

    if (failures) return 1;
    printf("host ABI validation: all cases as expected\n");
    return 0;
}
