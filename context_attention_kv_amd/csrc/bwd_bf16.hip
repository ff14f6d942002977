// bwd_bf16.hip -- gradients of one rank's attention against key/value blocks.
//
// The pages use sequence parallelism for training as well as inference (web
// page "Sequence parallelism -- splitting the token dimension across GPUs",
// section "Training and inference stress this dimension differently") but
// give no backward formulas; these kernels apply the chain rule to the
// definition softmax(Q K^T / sqrt(d_k)) V (section "Attention wants keys and
// values from other tokens"), with the probabilities recomputed from the
// forward's log-sum-exp instead of stored:
//   p_ij = e^{s_ij - lse_i},  delta_i = dout_i . out_i,
//   ds_ij = p_ij (dout_i . v_j - delta_i),
//   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,  dv_j = sum_i p_ij dout_i,
// the causal rule by global position as in the forward.
//
// bwd_delta_kernel: delta per query row (one wave per row).
// bwd_dq_kernel: query-stationary, 4 waves per workgroup, each wave 32 rows of
//   one query head (grouped heads share the workgroup's K/V tiles). Per
//   64-key tile, copied from HBM straight into LDS (double buffer):
//   S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16 (K, V as A
//   operands, Q^T and dO^T in registers as B), dS = P (dP - delta), then
//   dQ^T += K^T dS^T with K^T read through ds_read_b64_tr_b16.
// bwd_dkdv_kernel: key-stationary, 8 waves of 32 keys (K^T and V^T in
//   registers, both B operands) over every 32-row
//   query tile of the kv head's query heads, copied into LDS: S = Q K^T and
//   dP = dO V^T (query rows in output registers), dV^T += dO^T P and
//   dK^T += Q^T dS with dO^T and Q^T read through ds_read_b64_tr_b16.
// Both kernels run two waves per SIMD (dq: two 4-wave workgroups per CU; dk/dv:
// one 8-wave workgroup, so that each query tile copied serves 256 keys), and
// one wave's products overlap the other's softmax work and barrier waits.
// Tile copies use buffer loads that write LDS directly: no staging registers,
// and the range check of a per-tile buffer resource zero-fills rows past the
// end of a block or of the query range.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "bwd_args.h"

namespace cakv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr float kLog2e = 1.44269504088896341f;

// Row i of a 32-row A operand lands in output row i, which the 32x32 layout
// gives to half-wave (i/4)%2 at register 4*(i/8) + i%4; reading row
// 16*((i/4)%2) + 4*(i/8) + i%4 of a tile into operand row i leaves rows
// 16h..16h+15 in registers 0..15 of half-wave h, in order.
__device__ __forceinline__ int perm_row(int i) {
    return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// XOR swizzle of the 16-byte units of a tile row. Every tile here is read
// both ways: as A-operand rows (16-byte reads, rows perm_row(l32)) and through
// the transposing 8-byte reads (four consecutive rows per 16-lane group). The
// swizzle keeps both free of bank conflicts whether the LDS serves a 16-byte
// read 8 lanes per cycle over 128 bytes or 16 lanes over 256 bytes, and an
// 8-byte read 16 or 32 lanes per cycle: the row reads need it to be one-to-one
// on row bits {0,1,2,4} (on {0,1,4} modulo 8), the transposing reads on row
// bits {0,1} into unit bits {2,3} and {1,2}. (Unit bits for d = 128; for
// d = 64 two rows share 256 bytes and the unit has three bits.)
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128)
        return (row & 3) | (((row ^ (row >> 4)) & 1) << 2) | ((((row >> 1) ^ (row >> 2)) & 1) << 3);
    else
        return ((row >> 1) & 1) | (((row ^ (row >> 2)) & 1) << 1) | ((((row >> 1) ^ (row >> 4)) & 1) << 2);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct BCfg {
    static constexpr int DSTEPS = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int UNITS = D / 8;   // 16-byte units per row
};

// 16-byte operand unit `unit` of tile row `row` (swizzled layout)
template <int D>
__device__ __forceinline__ u32x4 tile_unit(const lds_char* t, int row, int unit) {
    return *(const lds_u32x4*)(t + row * BCfg<D>::ROW_BYTES + 16 * (unit ^ swz<D>(row)));
}
// Transposed operand (rows as the contraction index): fragment f = (j, db)
// of a 32-row block, through ds_read_b64_tr_b16. In each 16-lane group g16,
// source lane 4k + q points at row base + k and dims 16 (g16 % 2) + 4q .. +3
// of the 32-dim block; the group receives 4 consecutive rows of one dim per
// lane. Rows of step j: 8j + 16 (g16 / 2) + k, and 4 more for the high half.
template <int D>
__device__ __forceinline__ u32x4 tile_tr(const lds_char* t, int lane, int j, int db) {
    constexpr int RB = BCfg<D>::ROW_BYTES;
    const int g16 = lane >> 4, src = lane & 15;
    const int row = 8 * j + 16 * (g16 >> 1) + (src >> 2);
    const int d = 32 * db + 16 * (g16 & 1) + 4 * (src & 3);
    const int lo = row * RB + 16 * ((d >> 3) ^ swz<D>(row)) + 2 * (d & 7);
    const int hi = (row + 4) * RB + 16 * ((d >> 3) ^ swz<D>(row + 4)) + 2 * (d & 7);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + lo));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + hi));
    const u32x2 a2 = __builtin_bit_cast(u32x2, a);
    const u32x2 b2 = __builtin_bit_cast(u32x2, b);
    return u32x4{a2[0], a2[1], b2[0], b2[1]};
}

// Buffer resource of `bytes` bytes at `base` (raw: stride 0, 32-bit data
// format). Lanes whose offset falls at or past `bytes` read zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
    const unsigned long long p = reinterpret_cast<unsigned long long>(base);
    i32x4 r;
    r[0] = (int)(unsigned)p;
    r[1] = (int)((p >> 32) & 0xFFFFu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}
// Buffer -> LDS copies: lane i's 16 (4) bytes from byte offset voff of the
// resource land at LDS address lds_base + 16 i (+ 4 i). Inline assembly, so
// that the compiler does not wait for them before unrelated LDS reads; the
// issuing wave waits for them (wait_vmem) before the barrier that publishes
// the tile.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, unsigned voff, unsigned lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(lds_base)
        : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(i32x4 rsrc, unsigned voff, unsigned lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(lds_base)
        : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Lane-constant byte offset of copy region `lr` (1 KB of a swizzled tile of
// rows of `rs` elements): this lane fetches 16-byte unit p of tile row `row`
// such that it lands at its swizzled place.
template <int D>
__device__ __forceinline__ unsigned region_off(int lr, int lane, long long rs) {
    constexpr int RPK = 1024 / BCfg<D>::ROW_BYTES;   // rows per 1 KB region
    const int row = lr * RPK + lane / BCfg<D>::UNITS;
    const int p = lane % BCfg<D>::UNITS;
    return (unsigned)(2 * (row * rs + 8 * (p ^ swz<D>(row))));
}

// Workgroup id -> logical id. Ids are dealt to the 8 XCDs round robin; this
// gives each XCD a contiguous range of logical ids, so the workgroups that
// stream the same key/value (or query) head run on one XCD and share its L2.
__device__ __forceinline__ int xcd_logical(int bid, int n) {
    const int per = n / 8, rem = n % 8;
    const int xcd = bid % 8, idx = bid / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// ---------------------------------------------------------------- delta
// Per query row, negated: -delta and -lse / scale (-inf for a row without
// keys, so that every p of that row is 0). The dk/dv kernel starts its S and
// dP accumulators from them, so that its products give s - lse / scale and
// dP - delta directly.
template <int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const BwdArgs a) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // over [B, Tq, Hq]
    if (row >= (long long)a.B * a.Tq * a.Hq) return;
    const __bf16* dO = static_cast<const __bf16*>(a.dout) + row * D + lane * PER;
    const float* o = a.out + row * D + lane * PER;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) s += (float)dO[e] * o[e];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) {
        const long long h = row % a.Hq, bi = row / a.Hq;
        const long long i = bi % a.Tq, b = bi / a.Tq;
        const long long si = (b * a.Hq + h) * a.Tq + i;
        a.ndelta[si] = -s;
        const float l = a.lse[si];
        a.nlse[si] = l == -INFINITY ? -INFINITY : -l / a.scale;
    }
}

// ---------------------------------------------------------------- dq
template <int D>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(const BwdArgs a) {
    using C = BCfg<D>;
    constexpr int KT = 64, TB = KT * C::ROW_BYTES;
    constexpr int NCP = TB / 1024 / 4;   // copies per wave per K (or V) tile
    __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TB];   // 2 x [K | V]
    const unsigned lds0 = (unsigned)(unsigned long)(const lds_char*)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;

    const int logical = wg_permute(xcd_logical(blockIdx.x, gridDim.x), gridDim.x, a.wg_mul, a.wg_add);
    const int bg = logical / a.wg_per_bg;
    const int qt = a.wg_per_bg - 1 - logical % a.wg_per_bg;   // heaviest (latest rows) first
    const int b = bg / a.Hkv, g = bg % a.Hkv, G = a.Hq / a.Hkv;
    const int npblk = (a.Tq + 31) / 32;
    const int task = qt * 4 + wave, pblk = task / G, h = g * G + task % G;
    const bool wave_valid = pblk < npblk;
    const int row = pblk * 32 + l32;
    const bool row_ok = wave_valid && row < a.Tq;
    int last_pblk = (qt * 4 + 3) / G;
    if (last_pblk > npblk - 1) last_pblk = npblk - 1;
    const long long wg_last_pos = a.q_off + min(a.Tq, (last_pblk + 1) * 32) - 1;
    const long long qpos = a.q_off + row;
    const long long q_rs = (long long)a.Hq * D, kv_rs = (long long)a.Hkv * D;

    // Q^T and dO^T (B operands): lane (l32, hh) holds [row][16s + 8hh .. +7]
    u32x4 qf[C::DSTEPS], df[C::DSTEPS];
    {
        const long long ro = ((long long)b * a.Tq + (row_ok ? row : 0)) * q_rs + (long long)h * D;
        const __bf16* qb = static_cast<const __bf16*>(a.q) + ro;
        const __bf16* db_ = static_cast<const __bf16*>(a.dout) + ro;
#pragma unroll
        for (int s = 0; s < C::DSTEPS; ++s) {
            qf[s] = row_ok ? *reinterpret_cast<const u32x4*>(qb + 16 * s + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
            df[s] = row_ok ? *reinterpret_cast<const u32x4*>(db_ + 16 * s + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // this row's lse (log2 units) and delta; rows without any key or past
    // the end get p = 0 (lse2 = +inf)
    float lse2 = INFINITY, dlt = 0.f;
    if (row_ok) {
        const long long si = ((long long)b * a.Hq + h) * a.Tq + row;
        const float l = a.lse[si];
        lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
        dlt = -a.ndelta[si];
    }
    f32x16 dq_acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.f;

    // tiles: blocks in order, 64 keys at a time, only keys at or before the
    // workgroup's last query (causal)
    auto need = [&](int t) -> int {
        const int len = a.kv_len[t];
        if (!a.causal) return len;
        const long long n = wg_last_pos - a.kv_off[t] + 1;
        return n <= 0 ? 0 : (n < len ? (int)n : len);
    };
    int bi = 0, ti = 0;
    while (bi < a.n_blocks && need(bi) == 0) ++bi;
    // copy n of this wave fills 1 KB region 4n + wave of the K and of the V tile
    unsigned cp_off[NCP];
#pragma unroll
    for (int n = 0; n < NCP; ++n) cp_off[n] = region_off<D>(4 * n + wave, lane, kv_rs);
    auto issue = [&](int blk, int tile, unsigned dst) {
        const int key0 = tile * KT;
        const int rows = min(KT, a.kv_len[blk] - key0);
        const long long base = ((long long)b * a.kv_len[blk] + key0) * kv_rs + (long long)g * D;
        const unsigned bytes = (unsigned)(rows * kv_rs * 2);
        const i32x4 rk = make_rsrc(static_cast<const __bf16*>(a.k[blk]) + base, bytes);
        const i32x4 rv = make_rsrc(static_cast<const __bf16*>(a.v[blk]) + base, bytes);
#pragma unroll
        for (int n = 0; n < NCP; ++n) {
            copy16_to_lds(rk, cp_off[n], dst + (4 * n + wave) * 1024);
            copy16_to_lds(rv, cp_off[n], dst + TB + (4 * n + wave) * 1024);
        }
    };
    auto advance = [&](int& blk, int& tile) {
        if (++tile * KT >= need(blk)) {
            tile = 0;
            ++blk;
            while (blk < a.n_blocks && need(blk) == 0) ++blk;
        }
    };
    // the Q, dO, lse and delta loads above, in a form the compiler's wait
    // tracking sees, so that no wait for them lands in the loop (where it
    // would also wait for the tile copies in flight)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    int buf = 0;
    if (bi < a.n_blocks) issue(bi, ti, lds0);
    wait_vmem<0>();
    __syncthreads();
    while (bi < a.n_blocks) {
        int nbi = bi, nti = ti;
        advance(nbi, nti);
        // the other buffer was last read before the barrier that ended the
        // previous step
        if (nbi < a.n_blocks) issue(nbi, nti, lds0 + (buf ^ 1) * 2 * TB);
        const lds_char* kt = (const lds_char*)smem + buf * 2 * TB;
        const lds_char* vt = kt + TB;
        const int key0 = ti * KT;
        const int tile_keys = min(KT, a.kv_len[bi] - key0);
        const long long kpos0 = a.kv_off[bi] + key0;
        if (wave_valid) {
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] = 0.f;
                    dp[kb][r] = 0.f;
                }
            // S^T = K Q^T, dP^T = V dO^T: s[kb][r] = score(row, key 32kb + 16hh + r).
            // Products issue at raised wave priority, so that on a SIMD shared
            // with a wave in its vector phase they follow each other.
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int f = 0; f < 2 * C::DSTEPS; ++f) {
                const int st = f / 2, kb = f % 2;
                const int krow = 32 * kb + perm_row(l32);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(tile_unit<D>(kt, krow, 2 * st + hh)), as_bf16x8(qf[st]), s[kb], 0, 0, 0);
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(tile_unit<D>(vt, krow, 2 * st + hh)), as_bf16x8(df[st]), dp[kb], 0, 0, 0);
            }
            // pipeline: four operand reads ahead, then one read per product
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int f = 0; f < 4 * C::DSTEPS - 4; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_s_setprio(0);
            // P and dS = P (dP - delta); keys past the tile or (causal) after
            // this row get p = 0
            const long long dq64 = qpos - kpos0;
            const int dqp = dq64 > (1 << 30) ? (1 << 30) : (dq64 < -(1 << 30) ? -(1 << 30) : (int)dq64);
            // every key of the tile visible to every row of the wave (wave-uniform)
            const bool full = tile_keys == KT && (!a.causal || a.q_off + pblk * 32 - kpos0 >= KT - 1);
            u32x4 dsb[2][2];
            auto scores_to_ds = [&](auto masked_c) {
                constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int run0 = 32 * kb + 16 * hh;
                    int lim = tile_keys - 1 - run0;
                    if (a.causal) lim = min(lim, dqp - run0);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        f32x8 d8;
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int r = 8 * j + u;
                            const float e = fast_exp2(__builtin_fmaf(s[kb][r], a.scale_log2, -lse2));
                            const float p = !MASKED || r <= lim ? e : 0.f;
                            d8[u] = p * (dp[kb][r] - dlt);
                        }
                        dsb[kb][j] = __builtin_bit_cast(u32x4, __builtin_convertvector(d8, bf16x8));
                    }
                }
            };
            if (full) scores_to_ds(std::false_type{});
            else scores_to_ds(std::true_type{});
            // dQ^T += K^T dS^T
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int f = 0; f < 4 * C::DB; ++f) {
                const int db = f % C::DB, j = (f / C::DB) % 2, kb = f / (2 * C::DB);
                dq_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(tile_tr<D>(kt + kb * 32 * C::ROW_BYTES, lane, j, db)),
                    as_bf16x8(dsb[kb][j]), dq_acc[db], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int f = 0; f < 4 * C::DB - 4; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_s_setprio(0);
        }
        wait_vmem<0>();
        __syncthreads();
        bi = nbi;
        ti = nti;
        buf ^= 1;
    }
    if (row_ok) {
        float* dq = a.dq + (((long long)b * a.Tq + row) * a.Hq + h) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                f32x4 x;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) x[jj] = dq_acc[db][4 * ib + jj] * a.scale;
                *reinterpret_cast<f32x4*>(dq + 32 * db + 8 * ib + 4 * hh) = x;
            }
    }
}

// ---------------------------------------------------------------- dk, dv
template <int D>
__global__ void __launch_bounds__(512) bwd_dkdv_kernel(const BwdArgs a) {
    using C = BCfg<D>;
    constexpr int QR = 32, TB = QR * C::ROW_BYTES;
    constexpr int REG = TB / 1024;                // 1 KB regions per Q (or dO) tile
    // 2 x [Q | dO | -lse/scale (64 floats) | -delta (64 floats) | pad]
    constexpr int BUF = 2 * TB + 1024;
    __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
    const unsigned lds0 = (unsigned)(unsigned long)(const lds_char*)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;

    const int ntiles = a.kt0[a.n_blocks];
    // key tiles of one head in order on one XCD
    int id = wg_permute(xcd_logical(blockIdx.x, gridDim.x), gridDim.x, a.wg_mul, a.wg_add);
    const int kt = id % ntiles;
    id /= ntiles;
    const int g = id % a.Hkv, b = id / a.Hkv, G = a.Hq / a.Hkv;
    int blk = 0;
    while (blk + 1 < a.n_blocks && a.kt0[blk + 1] <= kt) ++blk;
    const int len = a.kv_len[blk];
    const int wkey0 = (kt - a.kt0[blk]) * kBwdKeyTile;   // the workgroup's first key
    // this lane's key: keys of the wave in the permuted order of the A-operand
    // rows (the order is the same everywhere: K^T, V^T, the mask and the dK,
    // dV rows written)
    const int wkey = 32 * wave + perm_row(l32);          // key within the workgroup's tile
    const int key = wkey0 + wkey;
    const bool key_ok = key < len;
    const long long wg_first_kpos = a.kv_off[blk] + wkey0;
    const int lane_rel = 16 * hh - wkey;   // row 16hh of a tile minus this lane's key, relative
    const bool wave_keys_all = wkey0 + 32 * wave + 32 <= len;   // all 32 keys of the wave present
    const long long q_rs = (long long)a.Hq * D, kv_rs = (long long)a.Hkv * D;

    // K^T and V^T (B operands) for the whole loop: lane (l32, hh) holds
    // K[key][16s + 8hh .. +7] and V[key][16s + 8hh .. +7]; keys past the
    // block's end are zeros
    u32x4 kf[C::DSTEPS], vf[C::DSTEPS];
    {
        const long long ko = ((long long)b * len + (key_ok ? key : 0)) * kv_rs + (long long)g * D;
        const __bf16* kb_ = static_cast<const __bf16*>(a.k[blk]) + ko;
        const __bf16* vb_ = static_cast<const __bf16*>(a.v[blk]) + ko;
#pragma unroll
        for (int s = 0; s < C::DSTEPS; ++s) {
            kf[s] = key_ok ? *reinterpret_cast<const u32x4*>(kb_ + 16 * s + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
            vf[s] = key_ok ? *reinterpret_cast<const u32x4*>(vb_ + 16 * s + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    f32x16 dk_acc[C::DB], dv_acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk_acc[db][r] = 0.f;
            dv_acc[db][r] = 0.f;
        }

    // query tiles: (head j of the group, 32-row block), skipping blocks whose
    // last row comes before the workgroup's first key (causal)
    const int nrt = (a.Tq + QR - 1) / QR;
    auto tile_ok = [&](int rt) -> bool {
        return !a.causal || a.q_off + min(a.Tq, (rt + 1) * QR) - 1 >= wg_first_kpos;
    };
    int rt0 = 0;
    while (rt0 < nrt && !tile_ok(rt0)) ++rt0;
    const int nq = (nrt - rt0) * G;   // query tiles to visit: (head, row block)
    // copy n of this wave fills 1 KB region 4n + wave of the Q and of the dO
    // tile; waves 0 and 1 also copy the tile's 32 -lse/scale and -delta values
    const unsigned cp_off = region_off<D>(wave < REG ? wave : 0, lane, q_rs);
    // query tiles go head-fastest: tile n is head n % G of row block
    // rt0 + n / G; running counters instead of divisions
    int i_hj = 0, i_rt = rt0;   // the next tile to copy
    auto issue = [&](unsigned dst) {
        const int hj = i_hj, rt = i_rt;
        if (++i_hj == G) {
            i_hj = 0;
            ++i_rt;
        }
        const int h = g * G + hj;
        const int r0 = rt * QR, rows = min(QR, a.Tq - r0);
        const long long base = ((long long)b * a.Tq + r0) * q_rs + (long long)h * D;
        const unsigned bytes = (unsigned)(rows * q_rs * 2);
        const i32x4 rq = make_rsrc(static_cast<const __bf16*>(a.q) + base, bytes);
        const i32x4 rd = make_rsrc(static_cast<const __bf16*>(a.dout) + base, bytes);
        if (wave < REG) {   // wave w copies region w of the Q and of the dO tile
            copy16_to_lds(rq, cp_off, dst + wave * 1024);
            copy16_to_lds(rd, cp_off, dst + TB + wave * 1024);
        }
        if (wave < 2) {
            const long long si = ((long long)b * a.Hq + h) * a.Tq + r0;
            const i32x4 rs = make_rsrc(wave == 0 ? a.nlse + si : a.ndelta + si, (unsigned)(rows * 4));
            copy4_to_lds(rs, (unsigned)(4 * lane), dst + 2 * TB + 256 * wave);
        }
    };
    // the K and V loads above, in a form the compiler's wait tracking sees
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (nq > 0) issue(lds0);
    // the tile being computed: head c_hj of its group; c_tq = position of its
    // first row minus the workgroup's first key, saturated at 2^30 (with the
    // causal rule the first visited tile has c_tq >= -31, and it only grows)
    int c_hj = 0, c_tq;
    {
        const long long rel0 = a.q_off + (long long)rt0 * QR - wg_first_kpos;
        c_tq = rel0 > (1 << 30) ? (1 << 30) : (rel0 < -(1 << 30) ? -(1 << 30) : (int)rel0);
    }
    wait_vmem<0>();
    __syncthreads();
    for (int n = 0; n < nq; ++n) {
        const int buf = n & 1;
        // the other buffer was last read before the barrier that ended the
        // previous step
        if (n + 1 < nq) issue(lds0 + (buf ^ 1) * BUF);
        const lds_char* qt = (const lds_char*)smem + buf * BUF;
        const lds_char* dt = qt + TB;
        {
            // S = Q K^T - lse / scale, dP = dO V^T - delta, from accumulators
            // that start at the rows' -lse / scale and -delta (copied with
            // the tile): s[r] belongs to row r0 + 16hh + r and this lane's key
            f32x16 s, dp;
            {
                const lds_char* lt = qt + 2 * TB + 64 * hh;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 l4 = *(const lds_f32x4*)(lt + 16 * i);
                    const f32x4 d4 = *(const lds_f32x4*)(lt + 256 + 16 * i);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        s[4 * i + k] = l4[k];
                        dp[4 * i + k] = d4[k];
                    }
                }
            }
            __builtin_amdgcn_s_setprio(1);   // products first on a shared SIMD
#pragma unroll
            for (int st = 0; st < C::DSTEPS; ++st) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(tile_unit<D>(qt, perm_row(l32), 2 * st + hh)), as_bf16x8(kf[st]), s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(tile_unit<D>(dt, perm_row(l32), 2 * st + hh)),
                    as_bf16x8(vf[st]), dp, 0, 0, 0);
            }
            // pipeline: one step's two operand reads ahead of its products
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int f = 0; f < C::DSTEPS - 1; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_s_setprio(0);
            // allowed: key present and (causal) at or before the row's
            // position: r + dlo >= 0, dlo = position of row 16hh minus this
            // lane's key (the tile's part is scalar, clamped to 32 bits), or
            // +-2^30 for every / no row. Only tiles where some score is not
            // allowed (the wave's last keys, the causal diagonal) apply the
            // mask, as s = -inf (p = 0); the rest skip it (wave-uniform test:
            // the wave's largest key is 32 wave + 31)
            if (!wave_keys_all || (a.causal && c_tq < 32 * wave + 31)) {
                int dlo = a.causal ? c_tq + lane_rel : (1 << 30);
                if (!key_ok) dlo = -(1 << 30);
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = r + dlo >= 0 ? s[r] : -INFINITY;
            }
            u32x4 pb[2], dsb[2];
            // p = e^{scale (s_ij - lse_i / scale)}, ds = p (dP - delta)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x8 p8, d8;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int r = 8 * j + u;
                    const float p = fast_exp2(s[r] * a.scale_log2);
                    p8[u] = p;
                    d8[u] = p * dp[r];
                }
                pb[j] = __builtin_bit_cast(u32x4, __builtin_convertvector(p8, bf16x8));
                dsb[j] = __builtin_bit_cast(u32x4, __builtin_convertvector(d8, bf16x8));
            }
            // dV^T += dO^T P, dK^T += Q^T dS
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int f = 0; f < 2 * C::DB; ++f) {
                const int db = f % C::DB, j = f / C::DB;
                dv_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(tile_tr<D>(dt, lane, j, db)), as_bf16x8(pb[j]), dv_acc[db], 0, 0, 0);
                dk_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(tile_tr<D>(qt, lane, j, db)), as_bf16x8(dsb[j]), dk_acc[db], 0, 0, 0);
            }
            // pipeline: two fragments read ahead of the products
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int f = 0; f < 4 * C::DB - 2; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_s_setprio(0);
        }
        if (++c_hj == G) {   // next row block: its first row is QR positions later
            c_hj = 0;
            c_tq = min(c_tq, (1 << 30) - QR) + QR;
        }
        wait_vmem<0>();
        __syncthreads();
    }
    if (key_ok) {
        const long long ko = (((long long)b * len + key) * a.Hkv + g) * D;
        float* dk = a.dk[blk] + ko;
        float* dv = a.dv[blk] + ko;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                f32x4 xk, xv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    xk[jj] = dk_acc[db][4 * ib + jj] * a.scale;
                    xv[jj] = dv_acc[db][4 * ib + jj];
                }
                *reinterpret_cast<f32x4*>(dk + 32 * db + 8 * ib + 4 * hh) = xk;
                *reinterpret_cast<f32x4*>(dv + 32 * db + 8 * ib + 4 * hh) = xv;
            }
    }
}

template <int D>
int launch_all(const BwdArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const long long rows = (long long)a.B * a.Tq * a.Hq;
    const long long n_dq = (long long)a.B * a.Hkv * a.wg_per_bg;
    const long long n_kv = (long long)a.B * a.Hkv * a.kt0[a.n_blocks];
    if (rows > 0) {
        hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    if (n_dq > 0) {
        BwdArgs aq = a;
        const WgPerm pm = wg_perm(a.wg_order, n_dq);
        aq.wg_mul = pm.mul;
        aq.wg_add = pm.add;
        hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)n_dq), dim3(256), 0, s, aq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    if (n_kv > 0) {
        BwdArgs ak = a;
        const WgPerm pm = wg_perm(a.wg_order, n_kv);
        ak.wg_mul = pm.mul;
        ak.wg_add = pm.add;
        hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)n_kv), dim3(512), 0, s, ak);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return (int)hipSuccess;
}

}  // namespace

int launch_bwd(const BwdArgs& a, int D, void* stream) {
    if (D == 128) return launch_all<128>(a, stream);
    if (D == 64) return launch_all<64>(a, stream);
    return (int)hipErrorInvalidValue;
}

}  // namespace cakv
