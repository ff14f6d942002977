// state_ops.hip -- bandwidth-bound kernels on the running softmax state.
//
//   state_init : m = -inf, l = 0, o = 0 (the empty state before any block).
//   finalize   : out = o / l, lse = m + ln l; rows with l = 0 give (0, -inf).
//   lse_merge  : (o_a, lse_a) + (o_b, lse_b) over disjoint key sets.
//
// Web page "Sequence parallelism -- splitting the token dimension across
// GPUs": the state is the running max, normaliser and value accumulator of
// section "But softmax seems to require all attention scores at once"; the
// merge combines partial results over key portions as section "Training and
// inference stress this dimension differently" describes, using that
// section's rescale rule for normalised pairs.
//
// Each thread owns 4 consecutive elements of one row of o ([B, Tq, Hq, D],
// 16-byte accesses, fully coalesced); the per-row scalars live in
// [B, Hq, Tq] arrays. All threads of a row sit in the same wave (D/4 <= 64
// threads, row-aligned), so a row's scalar is read by every lane before any
// lane writes it: outputs may alias inputs.
#include <hip/hip_runtime.h>

#include "fwd_args.h"

namespace cakv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
init_kernel(float* __restrict__ m, float* __restrict__ l, float* __restrict__ o, long long rows,
            int D) {
    const long long n4 = rows * (D / 4);
    for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n4;
         i += (long long)gridDim.x * kThreads) {
        reinterpret_cast<f32x4*>(o)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < rows) {
            m[i] = -INFINITY;
            l[i] = 0.f;
        }
    }
}

// Adds `value` to one tile counter: the tiles of a block that the schedule
// skips as a whole (nothing else is launched for it).
__global__ void counter_add_kernel(unsigned long long* counter, unsigned long long value) {
    if (threadIdx.x == 0) atomicAdd(counter, value);
}

template <int D>
__global__ void __launch_bounds__(kThreads)
finalize_kernel(const float* m, const float* l, const float* o, void* out, int out_bf16,
                float* lse, int Hq, int Tq, long long rows) {
    // D / 8 threads per row, each with two 16-byte vectors of it (the first
    // and the second half of the row) in flight: 709-716 against 761-775 us
    // at 4.19 M rows for one vector per thread (four per thread: 744-749)
    constexpr int TPR = D / 8;
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = i / TPR;
    const int c = (int)(i % TPR);
    if (row >= rows) return;
    const int h = (int)(row % Hq);
    const long long bt = row / Hq;
    const int t = (int)(bt % Tq);
    const long long b = bt / Tq;
    const long long si = (b * Hq + h) * Tq + t;
    const long long v0 = row * (D / 4) + c, v1 = v0 + TPR;   // 16-byte vectors of o / out
    const f32x4 x0 = reinterpret_cast<const f32x4*>(o)[v0];
    const f32x4 x1 = reinterpret_cast<const f32x4*>(o)[v1];
    const float lv = l[si];
    const float mv = m[si];
    const float inv = lv > 0.f ? 1.f / lv : 0.f;
    const f32x4 y0 = x0 * inv, y1 = x1 * inv;
    if (out_bf16) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        reinterpret_cast<bf16x4*>(out)[v0] = __builtin_convertvector(y0, bf16x4);
        reinterpret_cast<bf16x4*>(out)[v1] = __builtin_convertvector(y1, bf16x4);
    } else {
        reinterpret_cast<f32x4*>(out)[v0] = y0;
        reinterpret_cast<f32x4*>(out)[v1] = y1;
    }
    if (c == 0 && lse) lse[si] = lv > 0.f ? mv + logf(lv) : -INFINITY;
}

template <int D>
__global__ void __launch_bounds__(kThreads)
merge_kernel(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
             float* o_out, float* lse_out, int Hq, int Tq, long long rows) {
    constexpr int TPR = D / 4;
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long row = i / TPR;
    const int c = (int)(i % TPR);
    if (row >= rows) return;
    const int h = (int)(row % Hq);
    const long long bt = row / Hq;
    const int t = (int)(bt % Tq);
    const long long b = bt / Tq;
    const long long si = (b * Hq + h) * Tq + t;
    const float la = lse_a[si], lb = lse_b[si];
    // o rows are read and written once: non-temporal loads and store (+7 %
    // against plain ones; the same for finalize is 3-5 % slower; two vectors
    // per thread, as finalize has, 3.5 % slower here)
    const f32x4 xa = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o_a) + i);
    const f32x4 xb = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o_b) + i);
    const float M = fmaxf(la, lb);
    f32x4 r;
    float lo;
    if (M == -INFINITY) {
        r = f32x4{0.f, 0.f, 0.f, 0.f};
        lo = -INFINITY;
    } else {
        const float ea = expf(la - M), eb = expf(lb - M);
        const float z = ea + eb;
        lo = M + logf(z);
        const float wa = ea / z, wb = eb / z;
        r = wa * xa + wb * xb;
    }
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(o_out) + i);
    if (c == 0) lse_out[si] = lo;
}

int grid_for(long long threads) { return (int)((threads + kThreads - 1) / kThreads); }

}  // namespace

int launch_state_init(float* m, float* l, float* o, long long rows, int D, void* stream) {
    const long long n4 = rows * (D / 4);
    long long blocks = (n4 + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(init_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), m, l, o, rows, D);
    return (int)hipGetLastError();
}

int launch_counter_add(unsigned long long* counter, unsigned long long value, void* stream) {
    hipLaunchKernelGGL(counter_add_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       counter, value);
    return (int)hipGetLastError();
}

int launch_finalize(const float* m, const float* l, const float* o, void* out, int out_bf16,
                    float* lse, int B, int Hq, int Tq, int D, void* stream) {
    const long long rows = (long long)B * Hq * Tq;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (D == 128)
        hipLaunchKernelGGL(finalize_kernel<128>, dim3(grid_for(rows * 16)), dim3(kThreads), 0, st,
                           m, l, o, out, out_bf16, lse, Hq, Tq, rows);
    else if (D == 64)
        hipLaunchKernelGGL(finalize_kernel<64>, dim3(grid_for(rows * 8)), dim3(kThreads), 0, st,
                           m, l, o, out, out_bf16, lse, Hq, Tq, rows);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

int launch_lse_merge(const float* o_a, const float* lse_a, const float* o_b,
                     const float* lse_b, float* o_out, float* lse_out, int B, int Hq, int Tq,
                     int D, void* stream) {
    const long long rows = (long long)B * Hq * Tq;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (D == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3(grid_for(rows * 32)), dim3(kThreads), 0, st,
                           o_a, lse_a, o_b, lse_b, o_out, lse_out, Hq, Tq, rows);
    else if (D == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3(grid_for(rows * 16)), dim3(kThreads), 0, st,
                           o_a, lse_a, o_b, lse_b, o_out, lse_out, Hq, Tq, rows);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace cakv
