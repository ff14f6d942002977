// fwd_f32.hip -- ring-step attention forward for fp32 inputs (fp32 vector ALU).
//
// Same fold as the bf16 kernel (web page "Sequence parallelism -- splitting the
// token dimension across GPUs", sections "But softmax seems to require all
// attention scores at once" and "Causal attention gives us another
// optimization"), kept in full fp32: one lane owns one query row, its query
// and accumulator live in registers, and every key tile of K and V is staged
// in LDS and read by all lanes at the same address (a broadcast). The four
// waves of a workgroup share its 64 rows and take every fourth key tile each,
// with running states of their own; at the end the four states of a row are
// combined by the same rescale rule (the result does not depend on how the
// keys are cut). This path serves fp32 inputs, where a bf16 product would not
// meet fp32 accuracy; it is not the throughput path.
#include <hip/hip_runtime.h>

#include "fwd_args.h"

namespace cakv {
namespace {

constexpr int kRows = 64;   // rows (lanes) per workgroup: two 32-row slabs
constexpr int kWaves = 4;   // waves per workgroup, each on every fourth key tile
constexpr int kCountKeys = CAKV_TILE_K;   // keys per tile of the tile counters
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ int keys_needed(const FwdArgs& a, int t, long long last_q_pos) {
    const int len = a.kv_len[t];
    if (!a.causal) return len;
    const long long n = last_q_pos - a.kv_off[t] + 1;
    return n <= 0 ? 0 : (n < len ? (int)n : len);
}

template <int D>
struct F32Cfg {
    static constexpr int BK = 2048 / D;                    // keys per tile: 16 KB of K and V
    static constexpr int STAGE = BK * D;                   // floats per K (or V) tile
    static constexpr int MERGE = kWaves * kRows * (D + 2); // floats of the four states
    static constexpr int SMEM = (kWaves * 2 * STAGE > MERGE ? kWaves * 2 * STAGE : MERGE);
};

template <int D>
__global__ void __launch_bounds__(kRows * kWaves) fwd_f32_kernel(const FwdArgs a) {
    using C = F32Cfg<D>;
    constexpr int kBK = C::BK;
    __shared__ float4 smem4[C::SMEM / 4];
    float* smem = reinterpret_cast<float*>(smem4);
    const int tid = threadIdx.x;
    const int lane = tid & (kRows - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kRows);
    const int nqt = (a.Tq + kRows - 1) / kRows;
    const int wid = wg_permute((int)blockIdx.x, a.n_wg, a.wg_mul, a.wg_add);
    const int qt = nqt - 1 - wid % nqt;
    const int bh = wid / nqt;
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
    if (a.load_state && valid && wave == 0) {   // one wave carries the incoming state
        m_run = a.m[si] * 1.44269504088896341f;
        l_run = a.l[si];
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = a.o[oi + c];
    }
    unsigned long long n_full = 0, n_masked = 0, n_skip = 0;
    float* ks = smem + wave * 2 * C::STAGE;   // this wave's K and V tile
    float* vs = ks + C::STAGE;

    // tiles in block order, kBK keys at a time; step r gives tile 4r + w to wave w
    int t = 0, key0 = 0, need = 0;
    auto settle = [&]() {   // move (t, key0) to the next tile that exists
        while (t < a.n_blocks && key0 >= need) {
            ++t;
            key0 = 0;
            if (t < a.n_blocks) need = keys_needed(a, t, last_pos);
        }
    };
    if (a.n_blocks > 0) need = keys_needed(a, 0, last_pos);
    settle();
    while (t < a.n_blocks) {
        // this wave's tile of the current group of kWaves tiles: skip `wave` tiles ahead
        int mt = t, mk = key0, mneed = need;
        for (int s = 0; s < wave && mt < a.n_blocks; ++s) {
            mk += kBK;
            while (mt < a.n_blocks && mk >= mneed) {
                ++mt;
                mk = 0;
                if (mt < a.n_blocks) mneed = keys_needed(a, mt, last_pos);
            }
        }
        const bool have = mt < a.n_blocks;
        __syncthreads();   // every wave is done with its previous tile
        if (have) {
            const int len = a.kv_len[mt];
            const long long base = ((long long)b * len) * kv_rs + (long long)g * D;
            const float* kb = static_cast<const float*>(a.k[mt]) + base;
            const float* vb = static_cast<const float*>(a.v[mt]) + base;
            for (int c = lane; c < kBK * D / 4; c += kRows) {
                const int key = c / (D / 4), col = c % (D / 4);
                const bool ok = mk + key < len;
                reinterpret_cast<float4*>(ks)[c] =
                    ok ? *reinterpret_cast<const float4*>(kb + (long long)(mk + key) * kv_rs + 4 * col)
                       : float4{0, 0, 0, 0};
                reinterpret_cast<float4*>(vs)[c] =
                    ok ? *reinterpret_cast<const float4*>(vb + (long long)(mk + key) * kv_rs + 4 * col)
                       : float4{0, 0, 0, 0};
            }
        }
        __syncthreads();
        if (have) {
            const int len = a.kv_len[mt];
            const int tile_keys = min(kBK, len - mk);
            const long long kpos0 = a.kv_off[mt] + mk;
            const long long kpos_last = kpos0 + tile_keys - 1;
            // tile counters are kept per 32-row slab and 64-key tile: the wave
            // whose key tile starts a 64-key tile classifies all of it
            if (lane == 0 && mk % kCountKeys == 0) {
                const long long c_last = kpos0 + min(kCountKeys, len - mk) - 1;
                for (int sl = 0; sl < 2; ++sl) {
                    const int r0 = row0 + 32 * sl;
                    if (r0 >= a.Tq) continue;
                    const long long p0 = a.q_off + r0, p1 = a.q_off + min(r0 + 32, a.Tq) - 1;
                    if (!a.causal || c_last <= p0) ++n_full;
                    else if (kpos0 <= p1) ++n_masked;
                    else ++n_skip;
                }
            }
            const bool need_mask = (a.causal && kpos_last > first_pos) || tile_keys < kBK;
            // 16-key steps of the running update (each step is one "block" of
            // the online rule; the result does not depend on the cut).
#pragma unroll 1
            for (int j0 = 0; j0 < tile_keys; j0 += 16) {
                float sc[16];
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < D; ++c) acc = __builtin_fmaf(q[c], ks[(j0 + j) * D + c], acc);
                    if (need_mask && (j0 + j >= tile_keys || (a.causal && kpos0 + j0 + j > qpos)))
                        acc = -INFINITY;
                    sc[j] = acc;
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
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j], a.scale_log2, -m_use));
                    rs += p;
#pragma unroll
                    for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, vs[(j0 + j) * D + c], o[c]);
                }
                l_run = l_run * alpha + rs;
                m_run = m_new;
            }
        }
        // next step: four tiles on
        for (int s = 0; s < kWaves && t < a.n_blocks; ++s) {
            key0 += kBK;
            settle();
        }
    }

    // ---- combine the four waves' states of each row (rescale rule) ----
    __syncthreads();   // the tile buffers become the merge area
    float* ms = smem;                       // [kWaves][kRows]
    float* ls = ms + kWaves * kRows;        // [kWaves][kRows]
    float* os = ls + kWaves * kRows;        // [kWaves][kRows][D]
    ms[wave * kRows + lane] = m_run;
    ls[wave * kRows + lane] = l_run;
#pragma unroll
    for (int c = 0; c < D; ++c) os[(wave * kRows + lane) * D + c] = o[c];
    __syncthreads();
    if (wave == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ms[w * kRows + lane]);
        const float m_use = M == -INFINITY ? 0.f : M;
        float wt[kWaves];
        l_run = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            wt[w] = __builtin_amdgcn_exp2f(ms[w * kRows + lane] - m_use);
            l_run += wt[w] * ls[w * kRows + lane];
        }
#pragma unroll
        for (int c = 0; c < D; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) acc = __builtin_fmaf(wt[w], os[(w * kRows + lane) * D + c], acc);
            o[c] = acc;
        }
        m_run = M;
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
    }
    if (a.counters && lane == 0 && wave == 0) {
        // counted tiles of blocks (or block tails) past the workgroup's last
        // query, which no wave visits, and of blocks the host's schedule left
        // out of the list: skipped for each of its slabs
        long long unvisited = a.skip_tiles;
        for (int t = 0; t < a.n_blocks; ++t)
            unvisited += (a.kv_len[t] + kCountKeys - 1) / kCountKeys -
                         (keys_needed(a, t, last_pos) + kCountKeys - 1) / kCountKeys;
        n_skip += (unsigned long long)unvisited * (unsigned long long)((wg_rows + 31) / 32);
    }
    if (a.counters && lane == 0 && (n_full | n_masked | n_skip)) {
        atomicAdd(a.counters + 0, n_full);
        atomicAdd(a.counters + 1, n_masked);
        atomicAdd(a.counters + 2, n_skip);
    }
}

}  // namespace

int fwd_f32_wg_rows() { return kRows; }

int launch_fwd_f32(const FwdArgs& args, int D, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    FwdArgs a = args;
    const WgPerm pm = wg_perm(a.wg_order, a.n_wg);
    a.wg_mul = pm.mul;
    a.wg_add = pm.add;
    if (D == 128)
        hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(a.n_wg), dim3(kRows * kWaves), 0, st, a);
    else if (D == 64)
        hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(a.n_wg), dim3(kRows * kWaves), 0, st, a);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace cakv
