// Test-only stand-ins for the library's device-side entry points, so that the host validation of
// the C ABI (csrc/dion_api.cpp) builds and runs without a GPU, under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Each counts that it was reached and returns a fixed nonzero
// hipError_t-like value, which the API must pass on as -100 - value.
#include "dion_plan.h"

int g_stub_calls = 0;
constexpr int kStubError = 7;

namespace dion {
int run_step(const Plan&, void*, const void*, float*, float*, float, float, float, int, int, char*, int32_t*,
             uint32_t, void*, void* const*, float*) {
    ++g_stub_calls;
    return kStubError;
}
int run_lambda_max(const MpiArgs&, int64_t, int, void*) {
    ++g_stub_calls;
    return kStubError;
}
int run_adamw(void*, const void*, float*, float*, int64_t, int64_t, float, float, float, float, float, int, int,
              void*) {
    ++g_stub_calls;
    return kStubError;
}
int run_lion(void*, const void*, float*, int64_t, float, float, float, float, int, int, void*) {
    ++g_stub_calls;
    return kStubError;
}
}  // namespace dion
