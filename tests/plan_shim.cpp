// Host build of the planner's constexpr helpers for the CPU tests: the
// matrix-core kernel calls gemvplan::mfma_step_range on the device; the tests
// call the same function here, compiled by the host compiler.
#include "../memory_bound_gemv_f32_amd/csrc/gemv_plan.hpp"

extern "C" {

void shim_mfma_step_range(int K, int waves, int wave, int* first, int* end) {
    const gemvplan::StepRange r = gemvplan::mfma_step_range(K, waves, wave);
    *first = r.first;
    *end = r.end;
}

int shim_compensated_roundings(long long n) { return gemvplan::compensated_roundings(n); }

}  // extern "C"
