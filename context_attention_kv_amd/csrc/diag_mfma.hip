// diag_mfma.hip -- sustained bf16 matrix-core rate of the whole chip.
//
// Every wave keeps its SIMD's matrix core busy with independent
// 32x32x16 bf16 products whose operands come from registers only, so the
// launch's rate is set by the matrix cores and by the clock the chip holds
// while they run; with random operands that clock sits below the one reached
// with zeros because the products' power draw depends on the operand bits.
#include <hip/hip_runtime.h>

#include "cakv_diag.h"

namespace cakv {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// integer hash (xorshift-multiply) mapped to [-1, 1)
__device__ __forceinline__ float hash_unit(unsigned x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return (float)(x & 0xFFFFu) * (1.f / 32768.f) - 1.f;
}

__global__ void __launch_bounds__(256) mfma_burn_kernel(int zero, int iters, float* sink) {
    const unsigned gid = blockIdx.x * 256u + threadIdx.x;
    bf16x8 A[8], B[4];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int i = 0; i < 8; ++i) A[f][i] = (__bf16)(zero ? 0.f : hash_unit(gid * 131u + f * 17u + i));
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int i = 0; i < 8; ++i) B[f][i] = (__bf16)(zero ? 0.f : hash_unit(gid * 977u + f * 29u + i + 7u));
    f32x16 acc[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i & 7], B[(i >> 1) & 3], acc[i & 3], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    if (s == 1234.5f) sink[0] = s;
}

}  // namespace

int launch_mfma_burn(int zero, int iters, float* sink, void* stream) {
    hipLaunchKernelGGL(mfma_burn_kernel, dim3(CAKV_DIAG_MFMA_WG), dim3(256), 0,
                       static_cast<hipStream_t>(stream), zero, iters, sink);
    return (int)hipGetLastError();
}

}  // namespace cakv
