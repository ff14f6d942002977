// fwd_bf16.hip -- ring-step attention forward on gfx950 bf16 matrix cores.
//
// Computes, for every local query row, the online-softmax fold of a list of
// key/value blocks (web page "Sequence parallelism -- splitting the token
// dimension across GPUs", section "But softmax seems to require all attention
// scores at once": running max m, normaliser l, accumulator o, rescaled by
// e^{m - m_new} whenever the maximum grows), with the causal rule of section
// "Causal attention gives us another optimization" applied from global
// positions only where a tile straddles the diagonal.
//
// Work decomposition (MI355X: 256 CUs in 8 XCDs, 64-wide waves):
//   * a workgroup is 4 waves and serves one (batch, kv head); each wave owns
//     RW = 32*QS query rows of one query head. With grouped heads the waves
//     of a workgroup take different query heads of the same positions, so a
//     key/value tile staged once in LDS feeds all heads that read it.
//   * per 64-key tile: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as
//     the A operand, Q^T held in registers as the B operand), so a lane owns
//     one query column and its scores sit in its own registers: row max and
//     row sum need one cross-half exchange, the rescale of O is per lane.
//     Rows of the K operand are permuted so that each half-wave holds 16
//     consecutive keys; P^T then feeds O^T += V^T P^T directly as the B
//     operand, with V^T read from a transposed LDS copy.
//   * LDS layouts are XOR-swizzled so that the 16-byte operand reads and the
//     staging writes are free of bank conflicts; the next tile is prefetched
//     into registers while the current one is multiplied.
//   * workgroup ids are remapped so that each XCD works through a contiguous
//     range of (batch, kv head) pairs (their K/V stream then hits that XCD's
//     L2), heaviest query tiles first.
#include <hip/hip_runtime.h>

#include "fwd_args.h"

namespace cakv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;  // keys per tile
constexpr float kLn2 = 0.69314718055994531f;

// A-operand row i of a 32x32 product lands in output row i, which the
// 32x32 layout gives to half-wave (i/4)%2 at register 4*(i/8) + i%4. Loading
// key 16*((i/4)%2) + 4*(i/8) + i%4 into row i therefore leaves keys 16h..16h+15
// of the 32-key slab in registers 0..15 of half-wave h, in order.
__device__ __forceinline__ int key_of_row(int i) {
    return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// K tile swizzle: 16-byte column c of key row `key` is stored at c ^ kswz(key).
// The 8 lanes of one LDS read phase hold keys that differ in bits 0, 1, 4.
__device__ __forceinline__ int kswz(int key) { return (key & 3) | ((key >> 2) & 4); }
// V^T tile swizzle: 16-byte key group c of row d is stored at c ^ vswz(d).
__device__ __forceinline__ int vswz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32); }

template <int D, int QS>
struct Cfg {
    static constexpr int RW = 32 * QS;             // query rows per wave
    static constexpr int DSTEPS = D / 16;          // k-steps of S^T
    static constexpr int DB = D / 32;              // 32-row blocks of O^T
    static constexpr int KCH = kBK * D / 8;        // 16-byte chunks per K tile
    static constexpr int KPT = KCH / kThreads;     // chunks per thread
    static constexpr int VTASKS = 16 * (D / 8);    // (4 keys x 8 dims) tasks per V tile
    static constexpr int DH = D / 64;              // waves sharing a key quad
    static_assert(KCH % kThreads == 0, "K tile must split evenly");
    static_assert(VTASKS <= kThreads, "V tile tasks must fit the workgroup");
};

template <int D, int QS>
__device__ __forceinline__ void load_tile_regs(const __bf16* __restrict__ kb,
                                               const __bf16* __restrict__ vb, long long rs,
                                               int key0, int kv_len, int tid,
                                               u32x4 (&kreg)[Cfg<D, QS>::KPT], u32x4 (&vreg)[4]) {
    using C = Cfg<D, QS>;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
        const int c = tid + kThreads * i;
        const int key = c / (D / 8), col = c % (D / 8);
        const int gk = key0 + key;
        kreg[i] = gk < kv_len
                      ? *reinterpret_cast<const u32x4*>(kb + (long long)gk * rs + col * 8)
                      : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < C::VTASKS) {
        const int lane = tid & 63, w = tid >> 6;
        const int kq = (lane & 1) | (((lane >> 4) & 3) << 1) | ((w / C::DH) << 3);
        const int dg = ((lane >> 1) & 7) | ((w % C::DH) << 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int gk = key0 + 4 * kq + i;
            vreg[i] = gk < kv_len ? *reinterpret_cast<const u32x4*>(vb + (long long)gk * rs + dg * 8)
                                  : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

template <int D, int QS>
__device__ __forceinline__ void store_tile_lds(u32x4* __restrict__ ks, u32x4* __restrict__ vt,
                                               int tid, const u32x4 (&kreg)[Cfg<D, QS>::KPT],
                                               const u32x4 (&vreg)[4]) {
    using C = Cfg<D, QS>;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
        const int c = tid + kThreads * i;
        const int key = c / (D / 8), col = c % (D / 8);
        ks[key * (D / 8) + (col ^ kswz(key))] = kreg[i];
    }
    if (tid < C::VTASKS) {
        const int lane = tid & 63, w = tid >> 6;
        const int kq = (lane & 1) | (((lane >> 4) & 3) << 1) | ((w / C::DH) << 3);
        const int dg = ((lane >> 1) & 7) | ((w % C::DH) << 3);
        char* vbytes = reinterpret_cast<char*>(vt);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            const int d = dg * 8 + dd;
            const int w32 = dd >> 1;
            unsigned lo, hi;
            if (dd & 1) {
                lo = (vreg[0][w32] >> 16) | (vreg[1][w32] & 0xFFFF0000u);
                hi = (vreg[2][w32] >> 16) | (vreg[3][w32] & 0xFFFF0000u);
            } else {
                lo = (vreg[0][w32] & 0xFFFFu) | (vreg[1][w32] << 16);
                hi = (vreg[2][w32] & 0xFFFFu) | (vreg[3][w32] << 16);
            }
            const int unit = d * 8 + ((kq >> 1) ^ vswz(d));
            *reinterpret_cast<u32x2*>(vbytes + unit * 16 + (kq & 1) * 8) = u32x2{lo, hi};
        }
    }
}

// Number of keys of a block this workgroup must look at: all of them, or
// (causal) those at positions <= its last query position.
__device__ __forceinline__ int keys_needed(const FwdArgs& a, int t, long long last_q_pos) {
    const int len = a.kv_len[t];
    if (!a.causal) return len;
    const long long n = last_q_pos - a.kv_off[t] + 1;
    return n <= 0 ? 0 : (n < len ? (int)n : len);
}

template <int D, int QS>
__global__ void __launch_bounds__(kThreads)
fwd_bf16_kernel(const FwdArgs a) {
    using C = Cfg<D, QS>;
    constexpr int RW = C::RW;
    __shared__ u32x4 ks[C::KCH];          // K tile, [64 keys][D], swizzled
    __shared__ u32x4 vt[D * kBK / 8];     // V^T tile, [D][64 keys], swizzled

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- workgroup -> (batch, kv head, query tile); XCD-contiguous order ----
    const int bid = blockIdx.x;
    const int per = a.n_wg / 8, rem = a.n_wg % 8;
    const int xcd = bid % 8, idx = bid / 8;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + idx;
    const int bg = logical / a.wg_per_bg;
    const int qt = a.wg_per_bg - 1 - (logical % a.wg_per_bg);  // heaviest first
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int npblk = (a.Tq + RW - 1) / RW;

    const int task = qt * kWaves + wave;
    const int pblk = task / G;
    const int h = g * G + task % G;
    const bool wave_valid = pblk < npblk;
    const int row0 = pblk * RW;
    // rows of the whole workgroup (for how far into each block to read)
    int last_pblk = (qt * kWaves + kWaves - 1) / G;
    if (last_pblk > npblk - 1) last_pblk = npblk - 1;
    const int wg_last_row = min(a.Tq, (last_pblk + 1) * RW) - 1;
    const long long wg_last_pos = a.q_off + wg_last_row;
    const int wave_rows = wave_valid ? min(RW, a.Tq - row0) : 0;
    const long long wave_first_pos = a.q_off + row0;
    const long long wave_last_pos = a.q_off + row0 + wave_rows - 1;

    const long long q_rs = (long long)a.Hq * D;     // query row stride (elements)
    const long long kv_rs = (long long)a.Hkv * D;   // key/value row stride

    // ---- Q^T fragments (B operand): lane (l32, hh) holds Q[row][16s+8hh .. +7] ----
    u32x4 qf[QS][C::DSTEPS];
    {
        const __bf16* qb = static_cast<const __bf16*>(a.q) + ((long long)b * a.Tq) * q_rs +
                           (long long)h * D;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int row = row0 + 32 * qs + l32;
            const bool ok = wave_valid && row < a.Tq;
#pragma unroll
            for (int s = 0; s < C::DSTEPS; ++s)
                qf[qs][s] = ok ? *reinterpret_cast<const u32x4*>(qb + row * q_rs + 16 * s + 8 * hh)
                               : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // ---- running state: lane owns query column l32 of each 32-row slab ----
    float m_run[QS], l_run[QS];
    f32x16 o_acc[QS][C::DB];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        m_run[qs] = -INFINITY;
        l_run[qs] = 0.f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o_acc[qs][db][r] = 0.f;
    }
    if (a.load_state && wave_valid) {
        const float log2e = 1.44269504088896341f;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int row = row0 + 32 * qs + l32;
            const bool ok = row < a.Tq;
            const long long si = ((long long)b * a.Hq + h) * a.Tq + (ok ? row : 0);
            const float mv = ok ? a.m[si] : -INFINITY;
            const float lv = ok ? a.l[si] : 0.f;
            m_run[qs] = mv * log2e;
            l_run[qs] = hh == 0 ? lv : 0.f;
            const float* orow = a.o + (((long long)b * a.Tq + (ok ? row : 0)) * a.Hq + h) * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                f32x16 acc;
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    const f32x4 x = ok ? *reinterpret_cast<const f32x4*>(orow + 32 * db + 8 * ib + 4 * hh)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[4 * ib + jj] = x[jj];
                }
                o_acc[qs][db] = acc;
            }
        }
    }

    unsigned long long n_full = 0, n_masked = 0;

    // ---- walk the blocks in the given (ring) order, 64 keys at a time ----
    int bi = 0, ti = 0;
    while (bi < a.n_blocks && keys_needed(a, bi, wg_last_pos) == 0) ++bi;
    u32x4 kreg[C::KPT], vreg[4];
    if (bi < a.n_blocks) {
        const long long base = ((long long)b * a.kv_len[bi]) * kv_rs + (long long)g * D;
        load_tile_regs<D, QS>(static_cast<const __bf16*>(a.k[bi]) + base,
                              static_cast<const __bf16*>(a.v[bi]) + base, kv_rs, 0,
                              a.kv_len[bi], tid, kreg, vreg);
    }
    while (bi < a.n_blocks) {
        const int need = keys_needed(a, bi, wg_last_pos);
        const int key0 = ti * kBK;
        // next tile
        int nbi = bi, nti = ti + 1;
        if (nti * kBK >= need) {
            nti = 0;
            ++nbi;
            while (nbi < a.n_blocks && keys_needed(a, nbi, wg_last_pos) == 0) ++nbi;
        }
        __syncthreads();
        store_tile_lds<D, QS>(ks, vt, tid, kreg, vreg);
        __syncthreads();
        if (nbi < a.n_blocks) {
            const long long base = ((long long)b * a.kv_len[nbi]) * kv_rs + (long long)g * D;
            load_tile_regs<D, QS>(static_cast<const __bf16*>(a.k[nbi]) + base,
                                  static_cast<const __bf16*>(a.v[nbi]) + base, kv_rs,
                                  nti * kBK, a.kv_len[nbi], tid, kreg, vreg);
        }

        const int kv_len = a.kv_len[bi];
        const long long kpos0 = a.kv_off[bi] + key0;                 // first key position
        const int tile_keys = min(kBK, kv_len - key0);
        const long long kpos_last = kpos0 + tile_keys - 1;
        const bool compute = wave_valid && !(a.causal && kpos0 > wave_last_pos);
        if (compute) {
            // tile classes per 32-row slab (for the counters)
#pragma unroll
            for (int qs = 0; qs < QS; ++qs) {
                const int r0 = row0 + 32 * qs;
                if (r0 < a.Tq) {
                    const long long p0 = a.q_off + r0;
                    const long long p1 = a.q_off + min(r0 + 32, a.Tq) - 1;
                    if (!a.causal || kpos_last <= p0) ++n_full;
                    else if (kpos0 <= p1) ++n_masked;
                }
            }
            const bool need_mask = (a.causal && kpos_last > wave_first_pos) || tile_keys < kBK;

            // S^T = K Q^T : s[qs][kb][r] = score(query row0+32qs+l32, key key0+32kb+16hh+r)
            f32x16 s[QS][2];
#pragma unroll
            for (int qs = 0; qs < QS; ++qs)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[qs][kb][r] = 0.f;
#pragma unroll
            for (int st = 0; st < C::DSTEPS; ++st) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int key = 32 * kb + key_of_row(l32);
                    const u32x4 kf = ks[key * (D / 8) + ((2 * st + hh) ^ kswz(key))];
#pragma unroll
                    for (int qs = 0; qs < QS; ++qs)
                        s[qs][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(kf), as_bf16x8(qf[qs][st]), s[qs][kb], 0, 0, 0);
                }
            }

            // Scores leave the accumulators as plain floats; the mask is one
            // limit per (lane, 16-key run): key 16*hh + r of slab kb is kept
            // iff r <= lim. Selects only -- no per-element branches.
            float sv[QS][2][16];
#pragma unroll
            for (int qs = 0; qs < QS; ++qs)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sv[qs][kb][r] = s[qs][kb][r];
            if (need_mask) {
#pragma unroll
                for (int qs = 0; qs < QS; ++qs) {
                    const long long qpos = a.q_off + row0 + 32 * qs + l32;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const int run0 = 32 * kb + 16 * hh;       // tile key of r = 0
                        long long lim = tile_keys - 1 - run0;    // keys that exist
                        if (a.causal) {
                            const long long lc = qpos - (kpos0 + run0);
                            lim = lc < lim ? lc : lim;
                        }
                        const int lm = lim < -1 ? -1 : (lim > 15 ? 15 : (int)lim);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            sv[qs][kb][r] = r <= lm ? sv[qs][kb][r] : -INFINITY;
                    }
                }
            }

            // online softmax (log2 domain: t = score * scale * log2 e)
            u32x4 pb[QS][2][2];
            float alpha[QS];
#pragma unroll
            for (int qs = 0; qs < QS; ++qs) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[qs][kb][r]);
                mx = fmaxf(mx, xhalf(mx));
                const float m_new = fmaxf(m_run[qs], mx * a.scale_log2);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                alpha[qs] = fast_exp2(m_run[qs] - m_use);
                float rs = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        f32x8 p;
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            p[t] = fast_exp2(__builtin_fmaf(sv[qs][kb][8 * j + t], a.scale_log2, -m_use));
                            rs += p[t];
                        }
                        pb[qs][kb][j] = __builtin_bit_cast(u32x4, __builtin_convertvector(p, bf16x8));
                    }
                }
                l_run[qs] = l_run[qs] * alpha[qs] + rs;
                m_run[qs] = m_new;
            }
            // Rescale O only when some row's maximum moved (a wave-uniform
            // test; rows whose maximum did not move have alpha = 1).
            bool moved = false;
#pragma unroll
            for (int qs = 0; qs < QS; ++qs) moved |= alpha[qs] != 1.f;
            if (__any(moved)) {
#pragma unroll
                for (int qs = 0; qs < QS; ++qs)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) o_acc[qs][db] *= alpha[qs];
            }

            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const int d = 32 * db + l32;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int c16 = 4 * kb + 2 * hh + j;
                        const u32x4 vf = vt[d * 8 + (c16 ^ vswz(d))];
#pragma unroll
                        for (int qs = 0; qs < QS; ++qs)
                            o_acc[qs][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                as_bf16x8(vf), as_bf16x8(pb[qs][kb][j]), o_acc[qs][db], 0, 0, 0);
                    }
            }
        }
        bi = nbi;
        ti = nti;
    }

    // ---- epilogue: store state, or finalise into out / lse ----
    if (wave_valid) {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int row = row0 + 32 * qs + l32;
            const float l_tot = l_run[qs] + xhalf(l_run[qs]);
            if (row < a.Tq) {
                const long long si = ((long long)b * a.Hq + h) * a.Tq + row;
                const long long oi = (((long long)b * a.Tq + row) * a.Hq + h) * D;
                if (a.store_state) {
                    if (hh == 0) {
                        a.m[si] = m_run[qs] * kLn2;
                        a.l[si] = l_tot;
                    }
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int ib = 0; ib < 4; ++ib) {
                            f32x4 x;
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) x[jj] = o_acc[qs][db][4 * ib + jj];
                            *reinterpret_cast<f32x4*>(a.o + oi + 32 * db + 8 * ib + 4 * hh) = x;
                        }
                } else {
                    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                    if (hh == 0 && a.lse)
                        a.lse[si] = l_tot > 0.f ? (m_run[qs] + __log2f(l_tot)) * kLn2 : -INFINITY;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int ib = 0; ib < 4; ++ib) {
                            f32x4 x;
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) x[jj] = o_acc[qs][db][4 * ib + jj] * inv;
                            const int d = 32 * db + 8 * ib + 4 * hh;
                            if (a.out_bf16) {
                                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                                *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.out) + oi + d) =
                                    __builtin_convertvector(x, bf16x4);
                            } else {
                                *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + oi + d) = x;
                            }
                        }
                }
            }
        }
    }
    if (a.counters && lane == 0 && (n_full | n_masked)) {
        atomicAdd(a.counters + 0, n_full);
        atomicAdd(a.counters + 1, n_masked);
    }
}

template <int D, int QS>
int launch(const FwdArgs& a, void* stream) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QS>), dim3(a.n_wg), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace

int fwd_bf16_wg_rows(int rows_per_wave) { return kWaves * rows_per_wave; }

int launch_fwd_bf16(const FwdArgs& a, int D, int rows_per_wave, void* stream) {
    if (D == 128) return rows_per_wave == 64 ? launch<128, 2>(a, stream) : launch<128, 1>(a, stream);
    if (D == 64) return rows_per_wave == 64 ? launch<64, 2>(a, stream) : launch<64, 1>(a, stream);
    return (int)hipErrorInvalidValue;
}

}  // namespace cakv
