// decode_bf16.hip -- a few new queries against a long key/value history that
// is split into portions (web page "Sequence parallelism -- splitting the
// token dimension across GPUs", section "Training and inference stress this
// dimension differently": the new query is evaluated against the portions of
// the KV history and the partial attention results are combined).
//
// On one GPU the portions sit in device memory. The history is read once, so
// the work is bound by HBM bandwidth, not by the matrix cores: the kernel
// spreads the history over many independent waves (split-KV) so that enough
// bytes are in flight, and a second kernel merges the waves' partial
// online-softmax states row by row with the log-sum-exp rule.
//
// decode_split_kernel: wave (split s, batch b, kv head g, row block rb) owns
// 32 query rows -- row r = i * G + j is new query i of query head g * G + j,
// G = Hq / Hkv -- and folds the 32-key tiles of split s into a running state
// (m, l, o) exactly as the forward kernel does for one tile: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 (K from LDS as A, Q^T in registers as B), mask
// from global positions where a tile reaches past a row's position or past
// its portion's end, online softmax in the log2 domain, O^T += V^T P^T with
// V^T read through ds_read_b64_tr_b16. Tiles are 32 keys; each wave copies
// its K and V tiles from HBM into its own ring of LDS tile buffers with
// buffer_load_dwordx4 ... lds, issuing the next tiles before it waits for the
// one it computes. A workgroup holds the waves of HPW neighbouring kv heads
// of one split (four when Hkv allows, with a two-buffer ring each: 128 KB of
// LDS at d=128, one workgroup per CU), so the same keys of those heads --
// neighbouring 256-byte pieces of the history's 2 KB rows -- are read at the
// same time on one CU; the waves never wait for each other.
// decode_merge_kernel: one workgroup per row: M = max_s m_s,
// L = sum_s 2^(m_s-M) l_s, out = sum_s 2^(m_s-M) o_s / L, lse = (M + log2 L) ln 2.
#include <hip/hip_runtime.h>

#include <mutex>

#include "decode_args.h"

// Scratch of the allocation-free decode entry point (cakv_decode_noalloc):
// the splits' (m, l, o) states live here instead of in a caller workspace.
// One copy per GPU, held until the process ends. Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device, resolved once per device by decode_scratch_address below.
static __device__ __align__(256) char scratch[CAKV_DECODE_SCRATCH_BYTES];

namespace cakv {

int decode_scratch_address(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return 0;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr float kLn2 = 0.69314718055994531f;

// Row i of a 32-row A operand lands in output row i, which the 32x32 layout
// gives to half-wave (i/4)%2 at register 4*(i/8) + i%4; reading key
// 16*((i/4)%2) + 4*(i/8) + i%4 into row i leaves keys 16h..16h+15 of a 32-key
// slab in registers 0..15 of half-wave h, in order.
__device__ __forceinline__ int key_of_row(int i) {
    return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}
// XOR swizzles of 16-byte units in the K and V tiles (conflict-free operand
// reads; the same layouts as the forward kernel's tiles)
template <int D>
__device__ __forceinline__ int kswz(int key) {
    if constexpr (D == 128)
        return (key & 3) | (((key >> 4) & 1) << 2) | (((key >> 2) & 1) << 3);
    else
        return ((key >> 1) & 1) | (((key >> 4) & 1) << 1) | (((key ^ (key >> 2)) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int vswz(int key) {
    return (D == 128 ? 11 : 3) * (key & 1) + 4 * ((key >> 1) & 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// raw buffer resource of `bytes` bytes at `base`; lanes at or past the end
// read zeros
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
    const unsigned long long p = reinterpret_cast<unsigned long long>(base);
    i32x4 r;
    r[0] = (int)(unsigned)p;
    r[1] = (int)((p >> 32) & 0xFFFFu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}
// 16 bytes per lane from byte offset voff of the resource into LDS at
// lds_base + 16 * lane; completion is awaited with wait_vmem. The history is
// read once, so the loads are non-temporal (nt): 8 % faster than the default
// policy on the million-token history.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, unsigned voff, unsigned lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
        :
        : "v"(voff), "s"(rsrc), "s"(lds_base)
        : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D>
struct DCfg {
    static constexpr int DSTEPS = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int TILE_BYTES = kDecTile * ROW_BYTES;    // one K or one V tile
    static constexpr int BUF_BYTES = 2 * TILE_BYTES;           // [K | V]
    static constexpr int UNITS = D / 8;                        // 16-byte units per row
    static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;
    static constexpr int REGIONS = kDecTile / ROWS_PER_KB;     // 1 KB copies per K (or V) tile
};

// workgroup id -> logical id, so that each XCD (ids are dealt to the 8 XCDs
// round robin) takes a contiguous range: the row blocks of one split and
// head, which read the same tiles, then share that XCD's L2
__device__ __forceinline__ int xcd_logical(int bid, int n) {
    const int per = n / 8, rem = n % 8;
    const int xcd = bid % 8, idx = bid / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// HPW: waves (kv heads) per workgroup; NB: tile buffers per wave
template <int D, int HPW, int NB>
__global__ void __launch_bounds__(64 * HPW) decode_split_kernel(const DecArgs a) {
    using C = DCfg<D>;
    static_assert(NB == 2 || NB == 3, "two or three tile buffers per wave");
    __shared__ __attribute__((aligned(1024))) char smem_wg[HPW * NB * C::BUF_BYTES];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    char* smem = smem_wg + wv * NB * C::BUF_BYTES;   // this wave's ring
    const int l32 = lane & 31, hh = lane >> 5;
    const unsigned lds0 = (unsigned)(unsigned long)(const lds_char*)smem;

    int id = wg_permute(xcd_logical(blockIdx.x, gridDim.x), gridDim.x, a.wg_mul, a.wg_add);
    const int rb = id % a.nrb;
    id /= a.nrb;
    const int g = (id % (a.Hkv / HPW)) * HPW + wv;
    id /= a.Hkv / HPW;
    const int b = id % a.B;
    const int sp = id / a.B;
    const int G = a.Hq / a.Hkv, R = G * a.Tn;
    const int r = rb * 32 + l32;
    const bool row_ok = r < R;
    const int qi = row_ok ? r / G : 0;
    const int h = g * G + (row_ok ? r % G : 0);
    const long long q_rs = (long long)a.Hq * D;
    const long long kv_rs = (long long)a.Hkv * D;

    // Q^T fragments (B operand): lane (l32, hh) holds Q[row][16s + 8hh .. +7]
    u32x4 qf[C::DSTEPS];
    {
        const __bf16* qb = static_cast<const __bf16*>(a.q) + ((long long)b * a.Tn + qi) * q_rs +
                           (long long)h * D;
#pragma unroll
        for (int s = 0; s < C::DSTEPS; ++s)
            qf[s] = row_ok ? *reinterpret_cast<const u32x4*>(qb + 16 * s + 8 * hh)
                           : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the Q loads, before any tile copy
    // positions: this lane's query, and the first / last query of the block
    const long long qpos = a.q_off + qi;
    const int r_last = min(R, rb * 32 + 32) - 1;
    const long long wq_first = a.q_off + (rb * 32) / G;
    const long long wq_last = a.q_off + r_last / G;

    const int n_tiles_all = a.tile0[a.n_portions];
    const int t0 = sp * a.tiles_per_split;
    const int t1 = min(n_tiles_all, t0 + a.tiles_per_split);
    const int ntiles = t1 - t0;
    int p0 = 0;   // portion of tile t0 (skipping empty portions)
    while (p0 + 1 < a.n_portions && a.tile0[p0 + 1] <= t0) ++p0;

    // lane-constant parts of the copies: copy n fills 1 KB region n of the K
    // (or V) tile; this lane fetches 16-byte unit p of tile row `row`,
    // placed at its swizzled unit
    auto copy_off = [&](int n, bool is_v) -> unsigned {
        const int row = n * C::ROWS_PER_KB + lane / C::UNITS;
        const int p = lane % C::UNITS;
        const int sw = is_v ? vswz<D>(row) : kswz<D>(row);
        return (unsigned)(2 * (row * kv_rs + 8 * (p ^ sw)));
    };
    auto issue_tile = [&](int t, int pj, unsigned buf) {
        const int key0 = (t - a.tile0[pj]) * kDecTile;
        const int rows = min(kDecTile, a.kv_len[pj] - key0);
        const long long base = ((long long)b * a.kv_len[pj] + key0) * kv_rs + (long long)g * D;
        const unsigned bytes = (unsigned)(rows * kv_rs * 2);
        const i32x4 rk = make_rsrc(static_cast<const __bf16*>(a.k[pj]) + base, bytes);
        const i32x4 rv = make_rsrc(static_cast<const __bf16*>(a.v[pj]) + base, bytes);
#pragma unroll
        for (int n = 0; n < C::REGIONS; ++n) copy16_to_lds(rk, copy_off(n, false), buf + n * 1024);
#pragma unroll
        for (int n = 0; n < C::REGIONS; ++n)
            copy16_to_lds(rv, copy_off(n, true), buf + C::TILE_BYTES + n * 1024);
    };
    auto next_tile = [&](int& t, int& pj) {
        ++t;
        while (pj + 1 < a.n_portions && a.tile0[pj + 1] <= t) ++pj;
    };

    // operand reads: K fragment st, V^T fragment i = (j, db) of the 32-key tile
    const int k_row = key_of_row(l32) * C::ROW_BYTES;
    const int kx = kswz<D>(key_of_row(l32));
    const int g16 = lane >> 4, src = lane & 15;
    const int v_key = 16 * (g16 >> 1) + (src >> 2);
    const int v_dim = 16 * (g16 & 1) + 4 * (src & 3);
    const int v_sw = vswz<D>(src >> 2);
    auto k_frag = [&](const lds_char* kt, int st) -> u32x4 {
        return *(const lds_u32x4*)(kt + k_row + 16 * ((2 * st + hh) ^ kx));
    };
    auto v_frag = [&](const lds_char* vt, int i) -> u32x4 {
        const int db = i % C::DB, j = i / C::DB;
        const int key = 8 * j + v_key;
        const int d = 32 * db + v_dim;
        const int off = key * C::ROW_BYTES + 16 * ((d >> 3) ^ v_sw) + 2 * (d & 7);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off + 4 * C::ROW_BYTES));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };

    float m_run = -INFINITY, l_run = 0.f;   // log2 units
    f32x16 o_acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int q = 0; q < 16; ++q) o_acc[db][q] = 0.f;

    int tc = t0, pc = p0;   // next tile to copy
#pragma unroll
    for (int k = 0; k < NB - 1; ++k)
        if (k < ntiles) {
            issue_tile(tc, pc, lds0 + k * C::BUF_BYTES);
            next_tile(tc, pc);
        }
    int tq = t0, pq = p0;   // tile being computed
    int cur = 0;            // its buffer
    for (int i = 0; i < ntiles; ++i) {
        // the buffer of tile i-1, whose products have consumed their
        // operands, takes tile i + NB - 1 first; then wait for tile i with
        // the tiles after it still in flight
        if (i + NB - 1 < ntiles) {
            const int nb = cur == 0 ? NB - 1 : cur - 1;
            issue_tile(tc, pc, lds0 + nb * C::BUF_BYTES);
            next_tile(tc, pc);
        }
        const int later = min(NB - 1, ntiles - 1 - i);
        if (later >= 2) wait_vmem<4 * C::REGIONS>();
        else if (later == 1) wait_vmem<2 * C::REGIONS>();
        else wait_vmem<0>();
        const lds_char* kt = (const lds_char*)(smem + cur * C::BUF_BYTES);
        const lds_char* vt = (const lds_char*)(smem + cur * C::BUF_BYTES + C::TILE_BYTES);
        const int key0 = (tq - a.tile0[pq]) * kDecTile;
        const int tile_keys = min(kDecTile, a.kv_len[pq] - key0);
        const long long kpos0 = a.kv_off[pq] + key0;
        const long long kpos_last = kpos0 + tile_keys - 1;
        const bool skip = a.causal && kpos0 > wq_last;
        if (!skip) {
            // S^T = K Q^T: s[q] = score(row, key 16hh + q)
            f32x16 s;
#pragma unroll
            for (int q = 0; q < 16; ++q) s[q] = 0.f;
#pragma unroll
            for (int st = 0; st < C::DSTEPS; ++st)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k_frag(kt, st)),
                                                            as_bf16x8(qf[st]), s, 0, 0, 0);
            if ((a.causal && kpos_last > wq_first) || tile_keys < kDecTile) {
                const long long dq64 = qpos - kpos0;
                const int dq = dq64 > (1 << 30) ? (1 << 30) : (dq64 < -(1 << 30) ? -(1 << 30) : (int)dq64);
                const int run0 = 16 * hh;
                int lim = tile_keys - 1 - run0;
                if (a.causal) lim = min(lim, dq - run0);
                const i32x16 ridx = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15};
                const f32x16 ninf = -INFINITY;
                s = ridx <= lim ? s : ninf;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[q]);
            mx = half_max(mx);
            const float m_new = fmaxf(m_run, mx * a.scale_log2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db) o_acc[db] *= alpha;
            }
            float rs = 0.f;
            u32x4 pb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x8 p;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    p[u] = fast_exp2(__builtin_fmaf(s[8 * j + u], a.scale_log2, -m_use));
                    rs += p[u];
                }
                pb[j] = __builtin_bit_cast(u32x4, __builtin_convertvector(p, bf16x8));
            }
            l_run = l_run * alpha + rs;
            m_run = m_new;
            // O^T += V^T P^T
#pragma unroll
            for (int f = 0; f < 2 * C::DB; ++f) {
                const int db = f % C::DB, j = f / C::DB;
                o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v_frag(vt, f)),
                                                                    as_bf16x8(pb[j]), o_acc[db], 0, 0, 0);
            }
        }
        next_tile(tq, pq);
        cur = cur == NB - 1 ? 0 : cur + 1;
    }
    wait_vmem<0>();

    // partial state of the 32 rows of this block
    const long long wrow = (((long long)sp * a.B + b) * a.Hkv + g) * (a.nrb * 32) + r;
    const float l_tot = half_sum(l_run);
    if (hh == 0) {
        a.ws_m[wrow] = m_run;
        a.ws_l[wrow] = l_tot;
    }
    float* orow = a.ws_o + wrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            f32x4 x;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) x[jj] = o_acc[db][4 * ib + jj];
            *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * ib + 4 * hh) = x;
        }
}

// one workgroup of four waves per (batch, kv head, row < R): each wave
// combines a quarter of the splits' states against its own maximum (the
// splits' weights computed lane-parallel into LDS first, then the o rows
// read with several splits in flight), then the first wave combines the four
constexpr int kMergeMaxSplits = 4096;   // weights staged in LDS per workgroup

template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(const DecArgs a) {
    constexpr int PER = D / 64;   // dims per lane
    __shared__ float red_m[4], red_l[4];
    __shared__ float red_o[4][D];
    __shared__ float wgt[kMergeMaxSplits];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int G = a.Hq / a.Hkv, R = G * a.Tn;
    int id = blockIdx.x;
    const int r = id % R;
    id /= R;
    const int g = id % a.Hkv;
    const int b = id / a.Hkv;
    const int RP = a.nrb * 32;
    const long long sstride = (long long)a.B * a.Hkv * RP;   // rows per split
    const long long row0 = ((long long)b * a.Hkv + g) * RP + r;
    const int S = a.n_splits;
    const int s_lo = (int)((long long)S * wv / 4), s_hi = (int)((long long)S * (wv + 1) / 4);
    float mw = -INFINITY;
    for (int s = s_lo + lane; s < s_hi; s += 64) mw = fmaxf(mw, a.ws_m[s * sstride + row0]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
    float L = 0.f;
    for (int s = s_lo + lane; s < s_hi; s += 64) {
        const float ms = a.ws_m[s * sstride + row0];
        const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - mw);
        wgt[s] = w;
        L += w * a.ws_l[s * sstride + row0];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    __syncthreads();   // the weights in LDS are complete
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    if (mw != -INFINITY) {
#pragma unroll 8
        for (int s = s_lo; s < s_hi; ++s) {
            const float* o = a.ws_o + (s * sstride + row0) * D + lane * PER;
            const float w = wgt[s];
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += w * o[e];
        }
    }
    if (lane == 0) {
        red_m[wv] = mw;
        red_l[wv] = L;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) red_o[wv][lane * PER + e] = acc[e];
    __syncthreads();
    if (wv != 0) return;
    float M = red_m[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w]);
    float Lt = 0.f;
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sc = red_m[w] == -INFINITY ? 0.f : fast_exp2(red_m[w] - M);
            Lt += sc * red_l[w];
#pragma unroll
            for (int e = 0; e < PER; ++e) o[e] += sc * red_o[w][lane * PER + e];
        }
    }
    const int qi = r / G, h = g * G + r % G;
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    const long long oi = (((long long)b * a.Tn + qi) * a.Hq + h) * D + lane * PER;
    if (a.out_bf16) {
        __bf16* out = static_cast<__bf16*>(a.out);
#pragma unroll
        for (int e = 0; e < PER; ++e) out[oi + e] = (__bf16)(o[e] * inv);
    } else {
        float* out = static_cast<float*>(a.out);
#pragma unroll
        for (int e = 0; e < PER; ++e) out[oi + e] = o[e] * inv;
    }
    if (lane == 0 && a.lse)
        a.lse[((long long)b * a.Hq + h) * a.Tn + qi] = Lt > 0.f ? (M + __log2f(Lt)) * kLn2 : -INFINITY;
}

}  // namespace

namespace {
template <int HPW, int NB>
int launch_split(const DecArgs& args, int D, hipStream_t s) {
    const int grid = args.n_splits * args.B * (args.Hkv / HPW) * args.nrb;
    DecArgs a = args;
    const WgPerm pm = wg_perm(a.wg_order, grid);
    a.wg_mul = pm.mul;
    a.wg_add = pm.add;
    if (D == 128)
        hipLaunchKernelGGL((decode_split_kernel<128, HPW, NB>), dim3(grid), dim3(64 * HPW), 0, s, a);
    else if (D == 64)
        hipLaunchKernelGGL((decode_split_kernel<64, HPW, NB>), dim3(grid), dim3(64 * HPW), 0, s, a);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}
}  // namespace

// Four or two kv heads per workgroup with two tile buffers per wave (128 or
// 64 KB of LDS at d = 128), or one with three (48 KB). Measured on the
// million-token history (32 query heads on 8, one new token), each against
// the one-head, three-buffer kernel on one MI355X: four heads 6,208-6,249 GB/s
// against 5,983-5,987 at the same split count, two heads with three buffers
// 6,121, two heads with two 6,034-6,046; issuing the next tile before the
// wait +0.3 %.
int launch_decode_split(const DecArgs& args, int D, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (decode_heads_per_wg(args.Hkv)) {
        case 4: return launch_split<4, 2>(args, D, s);
        case 2: return launch_split<2, 2>(args, D, s);
        default: return launch_split<1, 3>(args, D, s);
    }
}

int launch_decode_merge(const DecArgs& a, int D, void* stream) {
    const int grid = a.B * a.Hkv * (a.Hq / a.Hkv) * a.Tn;
    if (D == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(grid), dim3(256), 0,
                           static_cast<hipStream_t>(stream), a);
    else if (D == 64)
        hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(grid), dim3(256), 0,
                           static_cast<hipStream_t>(stream), a);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace cakv
