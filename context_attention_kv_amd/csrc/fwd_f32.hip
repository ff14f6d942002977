// fwd_f32.hip -- ring-step attention forward for fp32 inputs (fp32 vector ALU).
//
// Same fold as the bf16 kernel (web page "Sequence parallelism -- splitting the
// token dimension across GPUs", sections "But softmax seems to require all
// attention scores at once" and "Causal attention gives us another
// optimization"), kept in full fp32: one lane owns one query row, its query
// and accumulator live in registers, and every 64-key tile of K and V is
// staged in LDS and read by all lanes at the same address (a broadcast).
// This path serves fp32 inputs, where a bf16 product would not meet fp32
// accuracy; it is not the throughput path.
#include <hip/hip_runtime.h>

#include "fwd_args.h"

namespace cakv {
namespace {

constexpr int kRows = 64;  // rows (lanes) per workgroup: two 32-row slabs
constexpr int kBK = 64;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ int keys_needed(const FwdArgs& a, int t, long long last_q_pos) {
    const int len = a.kv_len[t];
    if (!a.causal) return len;
    const long long n = last_q_pos - a.kv_off[t] + 1;
    return n <= 0 ? 0 : (n < len ? (int)n : len);
}

template <int D>
__global__ void __launch_bounds__(kRows) fwd_f32_kernel(const FwdArgs a) {
    __shared__ float4 ks[kBK * D / 4];
    __shared__ float4 vs[kBK * D / 4];
    const int lane = threadIdx.x;
    const int nqt = (a.Tq + kRows - 1) / kRows;
    const int qt = nqt - 1 - (int)(blockIdx.x % nqt);
    const int bh = blockIdx.x / nqt;
    const int b = bh / a.Hq, h = bh % a.Hq;
    const int g = h / (a.Hq / a.Hkv);
    const int row0 = qt * kRows;
    const int row = row0 + lane;
    const bool valid = row < a.Tq;
    const int wg_rows = min(kRows, a.Tq - row0);
    const long long first_pos = a.q_off + row0;
    const long long last_pos = a.q_off + row0 + wg_rows - 1;
    const long long qpos = a.q_off + row;
    const long long kv_rs = (long long)a.Hkv * D;

    float q[D], o[D];
    const float* qrow = static_cast<const float*>(a.q) + (((long long)b * a.Tq + row) * a.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
        const float4 x = valid ? *reinterpret_cast<const float4*>(qrow + c) : float4{0, 0, 0, 0};
        q[c] = x.x; q[c + 1] = x.y; q[c + 2] = x.z; q[c + 3] = x.w;
    }
    float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = 0.f;
    const long long si = ((long long)b * a.Hq + h) * a.Tq + row;
    const long long oi = (((long long)b * a.Tq + row) * a.Hq + h) * D;
    if (a.load_state && valid) {
        m_run = a.m[si] * 1.44269504088896341f;
        l_run = a.l[si];
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = a.o[oi + c];
    }

    unsigned long long n_full = 0, n_masked = 0;
    for (int t = 0; t < a.n_blocks; ++t) {
        const int need = keys_needed(a, t, last_pos);
        const int len = a.kv_len[t];
        const long long base = ((long long)b * len) * kv_rs + (long long)g * D;
        const float* kb = static_cast<const float*>(a.k[t]) + base;
        const float* vb = static_cast<const float*>(a.v[t]) + base;
        for (int key0 = 0; key0 < need; key0 += kBK) {
            __syncthreads();
            for (int c = lane; c < kBK * D / 4; c += kRows) {
                const int key = c / (D / 4), col = c % (D / 4);
                const bool ok = key0 + key < len;
                ks[c] = ok ? *reinterpret_cast<const float4*>(kb + (long long)(key0 + key) * kv_rs + 4 * col)
                           : float4{0, 0, 0, 0};
                vs[c] = ok ? *reinterpret_cast<const float4*>(vb + (long long)(key0 + key) * kv_rs + 4 * col)
                           : float4{0, 0, 0, 0};
            }
            __syncthreads();
            const int tile_keys = min(kBK, len - key0);
            const long long kpos0 = a.kv_off[t] + key0;
            const long long kpos_last = kpos0 + tile_keys - 1;
            if (a.causal && kpos0 > last_pos) continue;
            if (lane == 0) {
                for (int sl = 0; sl < 2; ++sl) {
                    const int r0 = row0 + 32 * sl;
                    if (r0 >= a.Tq) continue;
                    const long long p0 = a.q_off + r0, p1 = a.q_off + min(r0 + 32, a.Tq) - 1;
                    if (!a.causal || kpos_last <= p0) ++n_full;
                    else if (kpos0 <= p1) ++n_masked;
                }
            }
            const bool need_mask = (a.causal && kpos_last > first_pos) || tile_keys < kBK;
            const float* kl = reinterpret_cast<const float*>(ks);
            const float* vl = reinterpret_cast<const float*>(vs);
            // 16-key steps of the running update (each step is one "block" of
            // the online rule; the result does not depend on the cut).
#pragma unroll 1
            for (int j0 = 0; j0 < tile_keys; j0 += 16) {
                float s[16];
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < D; ++c) acc = __builtin_fmaf(q[c], kl[(j0 + j) * D + c], acc);
                    if (need_mask && (j0 + j >= tile_keys || (a.causal && kpos0 + j0 + j > qpos)))
                        acc = -INFINITY;
                    s[j] = acc;
                    mx = fmaxf(mx, acc);
                }
                const float m_new = fmaxf(m_run, mx * a.scale_log2);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
                float rs = 0.f;
#pragma unroll
                for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], a.scale_log2, -m_use));
                    rs += p;
#pragma unroll
                    for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, vl[(j0 + j) * D + c], o[c]);
                }
                l_run = l_run * alpha + rs;
                m_run = m_new;
            }
        }
    }

    if (valid) {
        if (a.store_state) {
            a.m[si] = m_run * kLn2;
            a.l[si] = l_run;
#pragma unroll
            for (int c = 0; c < D; ++c) a.o[oi + c] = o[c];
        } else {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
            if (a.lse) a.lse[si] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
            if (a.out_bf16) {
                __bf16* out = static_cast<__bf16*>(a.out) + oi;
#pragma unroll
                for (int c = 0; c < D; ++c) out[c] = (__bf16)(o[c] * inv);
            } else {
                float* out = static_cast<float*>(a.out) + oi;
#pragma unroll
                for (int c = 0; c < D; ++c) out[c] = o[c] * inv;
            }
        }
    }
    if (a.counters && lane == 0 && (n_full | n_masked)) {
        atomicAdd(a.counters + 0, n_full);
        atomicAdd(a.counters + 1, n_masked);
    }
}

}  // namespace

int fwd_f32_wg_rows() { return kRows; }

int launch_fwd_f32(const FwdArgs& a, int D, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (D == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(a.n_wg), dim3(kRows), 0, st, a);
    else if (D == 64)
        hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(a.n_wg), dim3(kRows), 0, st, a);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace cakv
