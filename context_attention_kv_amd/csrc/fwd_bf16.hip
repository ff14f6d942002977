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
// Work decomposition (MI355X: 256 CUs in 8 XCDs, 4 SIMDs per CU, 64-wide waves):
//   * a workgroup is NW waves serving one (batch, kv head); each wave owns 32
//     query rows of one query head. With grouped heads the waves take
//     different query heads of the same positions, so a key/value tile staged
//     once in LDS feeds every head that reads it. With 8 waves two waves share
//     each SIMD and the hardware overlaps one wave's softmax ALU work with the
//     other's matrix instructions.
//   * K and V tiles (64 keys) go from HBM straight into LDS with
//     global_load_lds_dwordx4 (no staging registers), double-buffered: the
//     next tile streams in while the current one is multiplied, with one
//     barrier per tile.
//   * per tile: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as the A
//     operand, Q^T held in registers as the B operand), so a lane owns one
//     query column and its scores sit in its own registers: the row max/sum
//     need one permlane32 swap and the rescale of O is per lane. K rows are
//     read in a permuted order so each half-wave holds 16 consecutive keys;
//     P^T (bf16) then feeds O^T += V^T P^T directly as the B operand, and the
//     V^T operand comes from the row-major V tile through ds_read_b64_tr_b16.
//   * LDS tiles are XOR-swizzled (16-byte units for K, 32-byte units for V)
//     so the operand reads are free of bank conflicts; the swizzle is applied
//     by choosing which global chunk each lane fetches.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 64;  // keys per tile
constexpr float kLn2 = 0.69314718055994531f;

// A-operand row i of a 32x32 product lands in output row i, which the
// 32x32 layout gives to half-wave (i/4)%2 at register 4*(i/8) + i%4. Loading
// key 16*((i/4)%2) + 4*(i/8) + i%4 into row i therefore leaves keys 16h..16h+15
// of the 32-key slab in registers 0..15 of half-wave h, in order.
__device__ __forceinline__ int key_of_row(int i) {
    return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// K tile: 16-byte unit c of key row `key` sits at unit c ^ kswz(key). The 8
// lanes of one ds_read_b128 phase hold keys that differ in bits 0, 1 and 4.
__device__ __forceinline__ int kswz(int key) { return (key & 3) | ((key >> 2) & 4); }
// V tile: 16-byte unit u of key row `key` sits at unit u ^ vswz(key): 32-byte
// units rotate with key % 4, so the four rows one 16-lane group of a
// transposing read touches fall in four different 32-byte bank ranges.
__device__ __forceinline__ int vswz(int key) { return 2 * (key & 3); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a lane's value with the lane 32 away (same query column)
__device__ __forceinline__ float half_max(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int NW>
struct Cfg {
    static constexpr int DSTEPS = D / 16;          // k-steps of S^T
    static constexpr int DB = D / 32;              // 32-row blocks of O^T
    static constexpr int ROW_BYTES = D * 2;        // one key row of a tile
    static constexpr int TILE_BYTES = kBK * ROW_BYTES;
    static constexpr int UNITS = D / 8;            // 16-byte units per row
    static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;   // rows one wave load fills
    static constexpr int REGIONS = kBK / ROWS_PER_KB;      // 1 KB regions per tile
    static constexpr int LOADS = REGIONS / NW;             // per wave, per tensor
    static_assert(REGIONS % NW == 0, "tile regions must split over the waves");
};

// Issue the direct-to-LDS loads of one K and one V tile (keys key0..key0+63
// of a block; rows past kv_len re-read the last key, which the mask drops).
template <int D, int NW>
__device__ __forceinline__ void issue_tile(const __bf16* __restrict__ kg,
                                           const __bf16* __restrict__ vg, long long rs,
                                           int key0, int kv_len, char* kdst, char* vdst,
                                           int wave, int lane) {
    using C = Cfg<D, NW>;
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) {
        const int region = n * NW + wave;
        const int row = region * C::ROWS_PER_KB + lane / C::UNITS;
        const int p = lane % C::UNITS;
        const int gk = min(key0 + row, kv_len - 1);
        const long long roff = (long long)gk * rs;
        __builtin_amdgcn_global_load_lds(kg + roff + 8 * (p ^ kswz(row)),
                                         (lds_void*)(kdst + region * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vg + roff + 8 * (p ^ vswz(row)),
                                         (lds_void*)(vdst + region * 1024), 16, 0, 0);
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

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW)
fwd_bf16_kernel(const FwdArgs a) {
    using C = Cfg<D, NW>;
    constexpr int RW = 32;
    // [buffer][K | V][64 keys][D] bf16
    __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * C::TILE_BYTES];

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

    const int task = qt * NW + wave;
    const int pblk = task / G;
    const int h = g * G + task % G;
    const bool wave_valid = pblk < npblk;
    const int row0 = pblk * RW;
    int last_pblk = (qt * NW + NW - 1) / G;
    if (last_pblk > npblk - 1) last_pblk = npblk - 1;
    const int wg_last_row = min(a.Tq, (last_pblk + 1) * RW) - 1;
    const long long wg_last_pos = a.q_off + wg_last_row;
    const int wave_rows = wave_valid ? min(RW, a.Tq - row0) : 0;
    const long long wave_first_pos = a.q_off + row0;
    const long long wave_last_pos = a.q_off + row0 + wave_rows - 1;
    const long long qpos = a.q_off + row0 + l32;      // this lane's query position

    const long long q_rs = (long long)a.Hq * D;
    const long long kv_rs = (long long)a.Hkv * D;

    // ---- Q^T fragments (B operand): lane (l32, hh) holds Q[row][16s+8hh .. +7] ----
    u32x4 qf[C::DSTEPS];
    {
        const int row = row0 + l32;
        const bool ok = wave_valid && row < a.Tq;
        const __bf16* qb = static_cast<const __bf16*>(a.q) +
                           ((long long)b * a.Tq + (ok ? row : 0)) * q_rs + (long long)h * D;
#pragma unroll
        for (int s = 0; s < C::DSTEPS; ++s)
            qf[s] = ok ? *reinterpret_cast<const u32x4*>(qb + 16 * s + 8 * hh)
                       : u32x4{0u, 0u, 0u, 0u};
    }

    // ---- running state: lane owns query column l32 ----
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o_acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[db][r] = 0.f;
    if (a.load_state && wave_valid) {
        const float log2e = 1.44269504088896341f;
        const int row = row0 + l32;
        const bool ok = row < a.Tq;
        const long long si = ((long long)b * a.Hq + h) * a.Tq + (ok ? row : 0);
        const float mv = ok ? a.m[si] : -INFINITY;
        const float lv = ok ? a.l[si] : 0.f;
        m_run = mv * log2e;
        l_run = hh == 0 ? lv : 0.f;
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
            o_acc[db] = acc;
        }
    }

    // ---- lane-constant LDS offsets of the operand reads ----
    // K (A operand of S^T): key 32kb + key_of_row(l32), 16-byte unit 2st + hh;
    // the K swizzle of that key does not depend on kb.
    const int k_row = key_of_row(l32) * C::ROW_BYTES;
    const int kx = kswz(key_of_row(l32));
    // V^T (A operand of O^T) through the transposing read: in each 16-lane
    // group g16, source lane 4k + q points at key (base + k) and dims
    // 16*(g16 % 2) + 4q .. +3 of the 32-dim block; the group then receives
    // 4 consecutive keys of one dim per lane. Key bases are multiples of 4,
    // so key % 4 == k and the V swizzle of the row is vswz(k).
    const int g16 = lane >> 4, src = lane & 15;
    const int v_key = 16 * (g16 >> 1) + (src >> 2);     // + 32kb + 8j (+4 for items 4..7)
    const int v_dim = 16 * (g16 & 1) + 4 * (src & 3);    // + 32db
    const int v_sw = vswz(src >> 2);

    unsigned long long n_full = 0, n_masked = 0;

    // ---- walk the blocks in the given (ring) order, 64 keys at a time ----
    int bi = 0;
    while (bi < a.n_blocks && keys_needed(a, bi, wg_last_pos) == 0) ++bi;
    int ti = 0, buf = 0;
    if (bi < a.n_blocks) {
        const long long base = ((long long)b * a.kv_len[bi]) * kv_rs + (long long)g * D;
        issue_tile<D, NW>(static_cast<const __bf16*>(a.k[bi]) + base,
                          static_cast<const __bf16*>(a.v[bi]) + base, kv_rs, 0, a.kv_len[bi],
                          smem, smem + C::TILE_BYTES, wave, lane);
    }
    while (bi < a.n_blocks) {
        const int need = keys_needed(a, bi, wg_last_pos);
        const int key0 = ti * kBK;
        int nbi = bi, nti = ti + 1;
        if (nti * kBK >= need) {
            nti = 0;
            ++nbi;
            while (nbi < a.n_blocks && keys_needed(a, nbi, wg_last_pos) == 0) ++nbi;
        }
        // This wave's loads of the current tile are complete; after the
        // barrier every wave's are, and every wave is done reading the other
        // buffer, which the next tile's loads may now overwrite.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (nbi < a.n_blocks) {
            const long long base = ((long long)b * a.kv_len[nbi]) * kv_rs + (long long)g * D;
            char* nk = smem + (buf ^ 1) * 2 * C::TILE_BYTES;
            issue_tile<D, NW>(static_cast<const __bf16*>(a.k[nbi]) + base,
                              static_cast<const __bf16*>(a.v[nbi]) + base, kv_rs, nti * kBK,
                              a.kv_len[nbi], nk, nk + C::TILE_BYTES, wave, lane);
        }
        const lds_char* kt = (const lds_char*)(smem + buf * 2 * C::TILE_BYTES);
        const lds_char* vt = kt + C::TILE_BYTES;

        const int kv_len = a.kv_len[bi];
        const long long kpos0 = a.kv_off[bi] + key0;
        const int tile_keys = min(kBK, kv_len - key0);
        const long long kpos_last = kpos0 + tile_keys - 1;
        const bool compute = wave_valid && !(a.causal && kpos0 > wave_last_pos);
        if (compute) {
            if (!a.causal || kpos_last <= wave_first_pos) ++n_full;
            else ++n_masked;
            const bool need_mask = (a.causal && kpos_last > wave_first_pos) || tile_keys < kBK;

            // S^T = K Q^T : s[kb][r] = score(query row0 + l32, key key0 + 32kb + 16hh + r)
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int st = 0; st < C::DSTEPS; ++st) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 kf = *(const lds_u32x4*)(kt + kb * 32 * C::ROW_BYTES + k_row +
                                                         16 * ((2 * st + hh) ^ kx));
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf),
                                                                    as_bf16x8(qf[st]), s[kb], 0, 0, 0);
                }
            }

            // scores as plain floats; the mask keeps r <= lim of each 16-key run
            float sv[2][16];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sv[kb][r] = s[kb][r];
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int run0 = 32 * kb + 16 * hh;
                    long long lim = tile_keys - 1 - run0;
                    if (a.causal) {
                        const long long lc = qpos - (kpos0 + run0);
                        lim = lc < lim ? lc : lim;
                    }
                    const int lm = lim < -1 ? -1 : (lim > 15 ? 15 : (int)lim);
#pragma unroll
                    for (int r = 0; r < 16; ++r) sv[kb][r] = r <= lm ? sv[kb][r] : -INFINITY;
                }
            }

            // online softmax (log2 domain: t = score * scale * log2 e)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[kb][r]);
            mx = half_max(mx);
            const float m_new = fmaxf(m_run, mx * a.scale_log2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            u32x4 pb[2][2];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    f32x8 p;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        p[t] = fast_exp2(__builtin_fmaf(sv[kb][8 * j + t], a.scale_log2, -m_use));
                        rs += p[t];
                    }
                    pb[kb][j] = __builtin_bit_cast(u32x4, __builtin_convertvector(p, bf16x8));
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
            // rescale O only when some row's maximum moved (wave-uniform test;
            // rows whose maximum did not move have alpha = 1)
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db) o_acc[db] *= alpha;
            }

            // O^T += V^T P^T; V^T fragments through transposing LDS reads
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) {
                        const int key = 32 * kb + 8 * j + v_key;
                        const int d = 32 * db + v_dim;
                        const int off = key * C::ROW_BYTES + 16 * ((d >> 3) ^ v_sw) + 2 * (d & 7);
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)(vt + off + 4 * C::ROW_BYTES));
                        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
                        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
                        const u32x4 vf = {l2[0], l2[1], h2[0], h2[1]};
                        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(vf), as_bf16x8(pb[kb][j]), o_acc[db], 0, 0, 0);
                    }
        }
        bi = nbi;
        ti = nti;
        buf ^= 1;
    }

    // ---- epilogue: store state, or finalise into out / lse ----
    if (wave_valid) {
        const int row = row0 + l32;
        const float l_tot = half_sum(l_run);
        if (row < a.Tq) {
            const long long si = ((long long)b * a.Hq + h) * a.Tq + row;
            const long long oi = (((long long)b * a.Tq + row) * a.Hq + h) * D;
            if (a.store_state) {
                if (hh == 0) {
                    a.m[si] = m_run * kLn2;
                    a.l[si] = l_tot;
                }
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
                        f32x4 x;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) x[jj] = o_acc[db][4 * ib + jj];
                        *reinterpret_cast<f32x4*>(a.o + oi + 32 * db + 8 * ib + 4 * hh) = x;
                    }
            } else {
                const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                if (hh == 0 && a.lse)
                    a.lse[si] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
                        f32x4 x;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) x[jj] = o_acc[db][4 * ib + jj] * inv;
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
    if (a.counters && lane == 0 && (n_full | n_masked)) {
        atomicAdd(a.counters + 0, n_full);
        atomicAdd(a.counters + 1, n_masked);
    }
}

template <int D, int NW>
int launch(const FwdArgs& a, void* stream) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW>), dim3(a.n_wg), dim3(64 * NW), 0,
                       static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace

int fwd_bf16_wg_rows(int waves) { return waves * 32; }

int launch_fwd_bf16(const FwdArgs& a, int D, int waves, void* stream) {
    if (D == 128) return waves == 4 ? launch<128, 4>(a, stream) : launch<128, 8>(a, stream);
    if (D == 64) return waves == 4 ? launch<64, 4>(a, stream) : launch<64, 8>(a, stream);
    return (int)hipErrorInvalidValue;
}

}  // namespace cakv
