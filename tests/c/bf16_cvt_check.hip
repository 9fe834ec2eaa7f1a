// The target's float -> bfloat16 conversion (v_cvt_pk_bf16_f32, which the
// library's bf16 kernels use) against the bit-level definition of round to
// nearest even, on every one of the 2^32 binary32 inputs, compiled with the
// library's floating-point flags (denormals kept).  Definition: add 0x7fff
// plus the lowest kept bit to the binary32 pattern and keep the upper 16
// bits; a NaN keeps its sign and upper payload bits with the quiet bit set.
// Prints the mismatch count and up to 8 examples; exit status 0 when none.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ uint32_t rne_bits(uint32_t u)
{
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

constexpr uint32_t kPerThread = 4096;
constexpr uint32_t kThreads = 1u << 20;  // kThreads * kPerThread = 2^32
constexpr uint32_t kBlock = 256;

__global__ __launch_bounds__(kBlock) void check(uint32_t* mismatches, uint32_t* example)
{
    const uint32_t t = blockIdx.x * kBlock + threadIdx.x;  // grid kThreads / kBlock: t < kThreads
    const uint32_t base = t * kPerThread;
    uint32_t count = 0, first = 0;
    for (uint32_t j = 0; j < kPerThread; j += 2) {
        const uint32_t u0 = base + j, u1 = base + j + 1;
        const f32x2 v = {__uint_as_float(u0), __uint_as_float(u1)};
        const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        const uint32_t lo_ok = (hw & 0xffffu) == rne_bits(u0), hi_ok = (hw >> 16) == rne_bits(u1);
        if (!lo_ok && count++ == 0) first = u0;
        if (!hi_ok && count++ == 0) first = u1;
    }
    mismatches[t] = count;
    example[t] = first;
}

int main()
{
    uint32_t *d_count = nullptr, *d_example = nullptr;
    if (hipMalloc(&d_count, kThreads * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&d_example, kThreads * sizeof(uint32_t)) != hipSuccess) {
        printf("hipMalloc failed\n");
        return 2;
    }
    hipLaunchKernelGGL(check, dim3(kThreads / kBlock), dim3(kBlock), 0, 0, d_count, d_example);
    if (hipDeviceSynchronize() != hipSuccess) {
        printf("kernel failed\n");
        return 2;
    }
    std::vector<uint32_t> count(kThreads), example(kThreads);
    if (hipMemcpy(count.data(), d_count, kThreads * sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(example.data(), d_example, kThreads * sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) {
        printf("copy failed\n");
        return 2;
    }
    uint64_t total = 0;
    int shown = 0;
    for (uint32_t t = 0; t < kThreads; t++) {
        total += count[t];
        if (count[t] && shown < 8) {
            float x;
            memcpy(&x, &example[t], sizeof x);
            printf("mismatch at input 0x%08x (%g)\n", example[t], x);
            shown++;
        }
    }
    printf("mismatches %llu of 4294967296\n", (unsigned long long)total);
    (void)hipFree(d_count);
    (void)hipFree(d_example);
    return total == 0 ? 0 : 1;
}
