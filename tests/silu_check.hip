// GPU check of the GEMM epilogues' SiLU over every fp32 input (test
// infrastructure, built by build() into tests/_build/libsilu_check.so and
// called by tests/test_gpu_exp.py).  For each of the 2^32 fp32 bit patterns g
// it compares the library's device function w8a8::silu_f32(g) with
// g / (1 + exp_f32_rn(-g)), the same fp32 add and divide on the correctly
// rounded exponential; the two can differ only through the exponential.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "exp_f32_rn.h"
#include "internal.h"

namespace {

__global__ void silu_sweep(unsigned long long* count, uint32_t* examples, int max_examples) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < (1ull << 32); u += stride) {
        const float g = __uint_as_float((uint32_t)u);
        const float got = w8a8::silu_f32(g);
        const float want = g / (1.0f + w8a8_test::exp_f32_rn(-g));
        const bool same = __float_as_uint(got) == __float_as_uint(want) || (got != got && want != want);
        if (!same) {
            const unsigned long long i = atomicAdd(count, 1ull);
            if (i < (unsigned long long)max_examples) examples[i] = (uint32_t)u;
        }
    }
}

}  // namespace

// Runs the sweep on the current device; writes the number of differing inputs
// and up to max_examples of them (bit patterns, in no particular order).
// Returns 0, or the HIP error code.
extern "C" __attribute__((visibility("default"))) int silu_check_all(unsigned long long* mismatches,
                                                                    uint32_t* examples, int max_examples) {
    if (max_examples < 0 || max_examples > 1024) return (int)hipErrorInvalidValue;
    unsigned long long* d_count = nullptr;
    uint32_t* d_ex = nullptr;
    hipError_t e = hipMalloc(&d_count, sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMalloc(&d_ex, 1024 * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(d_count, 0, sizeof(unsigned long long));
    if (e == hipSuccess) {
        silu_sweep<<<4096, 256>>>(d_count, d_ex, max_examples);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(mismatches, d_count, sizeof(unsigned long long), hipMemcpyDeviceToHost);
    if (e == hipSuccess && max_examples > 0)
        e = hipMemcpy(examples, d_ex, (size_t)max_examples * sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (d_count) (void)hipFree(d_count);
    if (d_ex) (void)hipFree(d_ex);
    return (int)e;
}
