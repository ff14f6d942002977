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
//   * a workgroup is 8 waves serving one (batch, kv head); each wave owns 32
//     query rows of one query head. With grouped heads the waves take
//     different query heads of the same positions, so a key/value tile staged
//     once in LDS feeds every head that reads it.
//   * two waves share each SIMD, one from each group of four (waves 0-3 and
//     4-7), and the groups run one phase apart: while one group does its
//     matrix phase (P V of the previous tile, then Q K^T of this tile) the
//     other does its softmax phase, so the SIMD's matrix core and vector ALU
//     work at the same time. A workgroup barrier separates the phases.
//   * K and V tiles (64 keys) go from HBM straight into LDS with
//     buffer_load_dwordx4 ... lds (no staging registers) into a ring of 4
//     tile buffers, two tiles ahead; each group issues its share (K or V)
//     during its matrix phase, where the wave's issue slots are free.
//   * per tile: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as the A
//     operand, Q^T held in registers as the B operand), so a lane owns one
//     query column and its scores sit in its own registers: the row max/sum
//     need one permlane32 swap and the rescale of O is per lane. K rows are
//     read in a permuted order so each half-wave holds 16 consecutive keys;
//     P^T (bf16) then feeds O^T += V^T P^T directly as the B operand, and the
//     V^T operand comes from the row-major V tile through ds_read_b64_tr_b16.
//   * LDS tiles are XOR-swizzled in 16-byte units so the operand reads are
//     free of bank conflicts; the swizzle is applied by choosing which global
//     chunk each lane fetches.
//   * workgroup ids are remapped so that each XCD works through a contiguous
//     range of (batch, kv head) pairs (their K/V stream then hits that XCD's
//     L2), heaviest query tiles first.
// That ping-pong kernel serves d = 128 shares whose grid fills the CUs. The
// others (d = 64; small d = 128 grids with one query head per kv head) go to
// a four-wave kernel with the same tile arithmetic: one wave per SIMD,
// several workgroups per CU running free of each other, a double buffer of
// tiles and one barrier per tile (fwd_bf16_4w_kernel below), which cuts the
// key range of small grids into parts merged by log-sum-exp.
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
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
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
// LDS swizzles: 16-byte unit c of key row `key` of a K tile sits at unit
// c ^ kswz(key), of a V tile at c ^ vswz(key). They are chosen so that every
// operand read is free of bank conflicts whether the LDS serves a 16-byte
// read 8 lanes per cycle over 32 banks or 16 lanes per cycle over 64 banks
// (and an 8-byte read 16 or 32 lanes per cycle): in one cycle the K reads
// touch keys that differ in bits 0, 1, 2, 4, the transposing V reads touch
// four consecutive keys (bits 0, 1) at 2 or 4 adjacent units.
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

template <int D>
struct Cfg {
    static constexpr int NW = 8;                   // waves: two groups of four
    static constexpr int NB = 4;                   // tile buffers in the LDS ring
    static constexpr int DSTEPS = D / 16;          // k-steps of S^T
    static constexpr int DB = D / 32;              // 32-row blocks of O^T
    static constexpr int ROW_BYTES = D * 2;        // one key row of a tile
    static constexpr int TILE_BYTES = kBK * ROW_BYTES;     // one K or one V tile
    static constexpr int BUF_BYTES = 2 * TILE_BYTES;       // K tile, then V tile
    static constexpr int UNITS = D / 8;            // 16-byte units per row
    static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;   // rows one wave load fills
    static constexpr int REGIONS = kBK / ROWS_PER_KB;      // 1 KB regions per tile
    static constexpr int LOADS = REGIONS / 4;              // copies per wave per tile
};

// Buffer resource of `bytes` bytes at `base` (raw: stride 0, 32-bit data
// format). Lanes whose offset falls at or past `bytes` read nothing: the
// range check returns zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    i32x4 r;
    r[0] = (int)(unsigned)a;
    r[1] = (int)((a >> 32) & 0xFFFFu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

// One buffer -> LDS copy of 16 bytes per lane: lane i's 16 bytes, from byte
// offset voff of the resource, land at LDS address lds_base + 16 i. Issued as
// inline assembly so that the compiler does not treat the copy as a pending
// LDS write to wait for before every later LDS read: completion is awaited
// explicitly (wait_vmem) before the workgroup barrier that publishes the
// tile. Vector-memory loads retire in issue order, so these extra loads only
// make the compiler's own waits stricter, never weaker.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, unsigned voff, unsigned lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(lds_base)
        : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Number of keys of a block this workgroup must look at: all of them, or
// (causal) those at positions <= its last query position.
__device__ __forceinline__ int keys_needed(const FwdArgs& a, int t, long long last_q_pos) {
    const int len = a.kv_len[t];
    if (!a.causal) return len;
    const long long n = last_q_pos - a.kv_off[t] + 1;
    return n <= 0 ? 0 : (n < len ? (int)n : len);
}

// Position in the tile sequence: block (in ring order) and 64-key tile in
// it, with that block's numbers cached so that stepping costs no loads.
struct Cursor {
    int bi, ti;
    int need, len;          // keys needed / present in block bi
    long long off;          // global position of the block's key 0
    const __bf16* kp;       // block bi's K and V at row 0 of (batch b, kv head g)
    const __bf16* vp;
    // block bi against the rows of this wave: rel = position of its key 0
    // minus the wave's first query position, clamped into 32 bits (only
    // read when the block is neither wholly before nor wholly after them)
    bool all_full;          // every key at or before the wave's first row (or no mask)
    int rel;
};
// (batch, kv head) coordinates of the workgroup, for the block pointers
struct HeadAt {
    int b, g;
    long long rs;           // key row stride (elements) = Hkv * D
    int D;
    long long last;         // last query position of the workgroup
    long long wfirst;       // first query position of this wave
    int causal;
};
__device__ __forceinline__ void cursor_load(const FwdArgs& a, const HeadAt& at, Cursor& c) {
    for (; c.bi < a.n_blocks; ++c.bi) {
        c.need = keys_needed(a, c.bi, at.last);
        if (c.need > 0) {
            c.len = a.kv_len[c.bi];
            c.off = a.kv_off[c.bi];
            const long long base = (long long)at.b * c.len * at.rs + (long long)at.g * at.D;
            c.kp = static_cast<const __bf16*>(a.k[c.bi]) + base;
            c.vp = static_cast<const __bf16*>(a.v[c.bi]) + base;
            c.all_full = !at.causal || c.off + c.len - 1 <= at.wfirst;
            const long long rel = c.off - at.wfirst;
            c.rel = c.all_full ? 0 : (rel > (1 << 30) ? (1 << 30) : (int)rel);
            return;
        }
    }
    c.need = 0;
}
__device__ __forceinline__ Cursor cursor_first(const FwdArgs& a, const HeadAt& at) {
    Cursor c;
    c.bi = 0;
    c.ti = 0;
    cursor_load(a, at, c);
    return c;
}
__device__ __forceinline__ void cursor_next(const FwdArgs& a, const HeadAt& at, Cursor& c) {
    if (++c.ti * kBK >= c.need) {
        c.ti = 0;
        ++c.bi;
        cursor_load(a, at, c);
    }
}

// Move cursor c forward by n tiles of its sequence.
__device__ __forceinline__ void cursor_skip(const FwdArgs& a, const HeadAt& at, Cursor& c, int n) {
    while (n > 0 && c.need > 0) {
        const int left = (c.need + kBK - 1) / kBK - c.ti;   // tiles left in block c.bi
        if (n < left) {
            c.ti += n;
            return;
        }
        n -= left;
        c.ti = 0;
        ++c.bi;
        cursor_load(a, at, c);
    }
}

// Tiles (64 keys) that a workgroup whose tile sequence has T tiles never
// visits: whole blocks after its last query (causal), the tails of blocks
// past it, and the tiles of blocks the host's schedule left out of the list.
// For each of its waves these are skipped tiles.
__device__ __forceinline__ unsigned skipped_unvisited(const FwdArgs& a, int T) {
    long long all = a.skip_tiles;
    for (int t = 0; t < a.n_blocks; ++t) all += (a.kv_len[t] + kBK - 1) / kBK;
    return (unsigned)(all - T);
}

// COUNT: tally the tiles of each wave's rows (computed full / masked, skipped)
// into a.counters
template <int D, bool COUNT>
__global__ void __launch_bounds__(512)
fwd_bf16_kernel(const FwdArgs a) {
    using C = Cfg<D>;
    constexpr int NW = C::NW;
    constexpr int RW = 32;
    // ring of NB buffers: [K tile | V tile], each [64 keys][D] bf16, swizzled
    __shared__ __attribute__((aligned(1024))) char smem[C::NB * C::BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int l32 = lane & 31, hh = lane >> 5;
    const bool loader = wave < 4;       // first group: issues the tile loads
    const unsigned lds0 = (unsigned)(unsigned long)(const lds_char*)smem;   // LDS address of the ring

    // ---- workgroup -> (batch, kv head, query tile); XCD-contiguous order ----
    const int bid = blockIdx.x;
    const int per = a.n_wg / 8, rem = a.n_wg % 8;
    const int xcd = bid % 8, idx = bid / 8;
    const int logical = wg_permute(xcd * per + (xcd < rem ? xcd : rem) + idx, a.n_wg, a.wg_mul, a.wg_add);
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
    // the K swizzle of that key does not depend on kb (bit 5).
    const int k_row = key_of_row(l32) * C::ROW_BYTES;
    const int kx = kswz<D>(key_of_row(l32));
    // V^T (A operand of O^T) through the transposing read: in each 16-lane
    // group g16, source lane 4k + q points at key (base + k) and dims
    // 16*(g16 % 2) + 4q .. +3 of the 32-dim block; the group then receives
    // 4 consecutive keys of one dim per lane. Key bases are multiples of 4,
    // so key % 4 == k and the V swizzle (a function of key % 4) is vswz(k).
    const int g16 = lane >> 4, src = lane & 15;
    const int v_key = 16 * (g16 >> 1) + (src >> 2);     // + 32kb + 8j (+4 for items 4..7)
    const int v_dim = 16 * (g16 & 1) + 4 * (src & 3);    // + 32db
    const int v_sw = vswz<D>(src >> 2);

    // The Q (and state) loads above are predicated; wait for them here, in a
    // form the compiler's wait tracking understands, so that no wait for them
    // lands inside the loop (where it would also wait for the tile copies).
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // tiles of this wave's rows: computed unmasked / masked, and skipped
    unsigned n_full = 0, n_masked = 0, n_skip = 0;

    // ---- tile sequence: blocks in the given (ring) order, 64 keys at a time ----
    const HeadAt at{b, g, kv_rs, D, wg_last_pos, wave_first_pos, a.causal};
    int T = 0;
    for (int t = 0; t < a.n_blocks; ++t) T += (keys_needed(a, t, wg_last_pos) + kBK - 1) / kBK;
    if constexpr (COUNT) n_skip = wave_valid ? skipped_unvisited(a, T) : 0u;

    // Tile copies: the first group copies K tiles, the second V tiles, each
    // two tiles ahead, into a ring of NB buffers [K | V].
    const bool copies_v = !loader;
    const int wl = wave & 3;
    Cursor ld = cursor_first(a, at);   // next tile this wave copies its share of
    // Lane-constant parts of the copies: copy n fills 1 KB region n*4 + wl of
    // the K (first group) or V (second group) tile; this lane fetches the
    // 16-byte unit p of key row `row` of the tile, swizzled (byte offset).
    unsigned cp_off[C::LOADS];
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) {
        const int row = (n * 4 + wl) * C::ROWS_PER_KB + lane / C::UNITS;
        const int p = lane % C::UNITS;
        cp_off[n] = (unsigned)(2 * (row * kv_rs + 8 * (p ^ (copies_v ? vswz<D>(row) : kswz<D>(row)))));
    }
    // Resource covering the rows of the tile at cursor `ld` that exist in its
    // block (rows past the block's end read as zeros, which the mask drops),
    // or nothing.
    auto tile_rsrc = [&](bool any) -> i32x4 {
        const int key0 = ld.ti * kBK;
        const int rows = any ? min(kBK, ld.len - key0) : 0;
        return make_rsrc((copies_v ? ld.vp : ld.kp) + (long long)key0 * kv_rs,
                         (unsigned)(rows * kv_rs * 2));
    };
    auto copy_part = [&](i32x4 rsrc, unsigned buf, int n) {
        copy16_to_lds(rsrc, cp_off[n], buf + (copies_v ? C::TILE_BYTES : 0) + (n * 4 + wl) * 1024);
    };
    auto issue = [&](unsigned buf) {
        const i32x4 rsrc = tile_rsrc(true);
#pragma unroll
        for (int n = 0; n < C::LOADS; ++n) copy_part(rsrc, buf, n);
        cursor_next(a, at, ld);
    };
    if (T > 0) issue(lds0);
    if (T > 1) issue(lds0 + C::BUF_BYTES);
    if (T > 1) wait_vmem<C::LOADS>();
    else wait_vmem<0>();
    __syncthreads();
    if (!loader) __syncthreads();   // the second group runs one phase behind

    // V^T fragment i of a tile (i = (kb, j, db), db fastest) and K fragment i
    // (i = (st, kb), kb fastest); both are A operands of 32x32x16 products.
    auto v_frag = [&](const lds_char* vt, int i) -> u32x4 {
        const int db = i % C::DB, j = (i / C::DB) % 2, kb = i / (2 * C::DB);
        const int key = 32 * kb + 8 * j + v_key;
        const int d = 32 * db + v_dim;
        const int off = key * C::ROW_BYTES + 16 * ((d >> 3) ^ v_sw) + 2 * (d & 7);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vt + off + 4 * C::ROW_BYTES));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    auto k_frag = [&](const lds_char* kt, int i) -> u32x4 {
        const int st = i / 2, kb = i % 2;
        return *(const lds_u32x4*)(kt + kb * 32 * C::ROW_BYTES + k_row + 16 * ((2 * st + hh) ^ kx));
    };
    constexpr int NPV = 4 * C::DB;       // P V products per tile
    constexpr int NQK = 2 * C::DSTEPS;   // Q K^T products per tile

    Cursor cq = cursor_first(a, at);   // tile of this wave's Q K^T
    bool have_p = false;       // P of the previous tile is waiting for its P V
    u32x4 pb[2][2];            // P^T of the previous tile (bf16), B operand of P V
    constexpr int NPRE = 4;    // V^T fragments of the previous tile read ahead
    u32x4 vpre[NPRE];
    for (int t = 0; t <= T; ++t) {
        // ================= matrix phase: P V (tile t-1), Q K^T (tile t) =================
        const lds_char* vt = (const lds_char*)(smem + ((t + C::NB - 1) % C::NB) * C::BUF_BYTES +
                                               C::TILE_BYTES);
        const lds_char* kt = (const lds_char*)(smem + (t % C::NB) * C::BUF_BYTES);
        // the matrix phase issues first on the SIMD it shares with the other
        // group's softmax phase, so that its products follow each other
        __builtin_amdgcn_s_setprio(1);
        // the first K fragments of Q K^T are read before P V, which hides
        // their latency behind the P V products
        u32x4 kpre[NPRE];
#pragma unroll
        for (int i = 0; i < NPRE; ++i) kpre[i] = k_frag(kt, i);
        if (have_p) {
#pragma unroll
            for (int i = 0; i < NPV; ++i) {
                const u32x4 vf = i < NPRE ? vpre[i] : v_frag(vt, i);
                const int db = i % C::DB, j = (i / C::DB) % 2, kb = i / (2 * C::DB);
                o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(vf), as_bf16x8(pb[kb][j]), o_acc[db], 0, 0, 0);
            }
            // pipeline: the first NPRE fragments were read in the softmax
            // phase; each product is followed by the reads of the fragment
            // NPRE ahead
#pragma unroll
            for (int i = 0; i < NPV - NPRE; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NPRE, 0);
        }
        // This group's share of tile t+2 goes into the buffer of tile t-2,
        // which no wave reads any more (see the phase schedule). The copies
        // are issued here, between the P V and the Q K^T products, rather
        // than in the softmax phase: that phase is the longer of the two,
        // and its wave then issues only the softmax (measured: 20 % fewer
        // cycles per launch). In the last two phases there is no tile t+2.
        if (t + 2 < T) {
            const unsigned cbuf = lds0 + ((t + 2) % C::NB) * C::BUF_BYTES;
            const i32x4 crsrc = tile_rsrc(true);
#pragma unroll
            for (int n = 0; n < C::LOADS; ++n) copy_part(crsrc, cbuf, n);
            cursor_next(a, at, ld);
        }
        // S^T = K Q^T : s[kb][r] = score(query row0 + l32, key key0 + 32kb + 16hh + r).
        // Computed for every tile (and once past the last one, on a stale
        // but finite buffer) so that no branch delays the products; the
        // softmax phase drops the scores of tiles this wave skips.
        f32x16 s[2];
        {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int i = 0; i < NQK; ++i) {
                const u32x4 kf = i < NPRE ? kpre[i] : k_frag(kt, i);
                s[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(kf), as_bf16x8(qf[i / 2]), s[i % 2], 0, 0, 0);
            }
            // pipeline: one MFMA, then the read of the fragment NPRE ahead
#pragma unroll
            for (int i = 0; i < NQK - NPRE; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NPRE, 0);
        }
        // tile t against this wave's rows (scalar work, after the products
        // are issued): k0r = position of the tile's key 0 minus the wave's
        // first query position
        // (branch-free; past the last tile the cursor's numbers are stale
        // and only cmp = false matters)
        const int key0 = cq.ti * kBK;
        const int tile_keys = min(kBK, cq.len - key0);
        const int k0r = cq.all_full ? -(1 << 30) : min(cq.rel, kBK) + key0;
        const bool full = k0r + tile_keys - 1 <= 0;
        const bool cmp = t < T && wave_valid && k0r <= wave_rows - 1;
        const bool need_mask = !full || tile_keys < kBK;
        if constexpr (COUNT) {
            n_full += cmp && full ? 1u : 0u;
            n_masked += cmp && !full ? 1u : 0u;
            n_skip += t < T && wave_valid && !cmp ? 1u : 0u;
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        if (t == T) break;

        // ================= softmax phase (tile t) =================
        if (cmp) {
            // the first V^T fragments of this tile for the next phase's P V
            // (its V tile was published two phases ago)
            {
                const lds_char* vcur = (const lds_char*)(smem + (t % C::NB) * C::BUF_BYTES +
                                                         C::TILE_BYTES);
#pragma unroll
                for (int i = 0; i < NPRE; ++i) vpre[i] = v_frag(vcur, i);
            }
            if (need_mask) {
                // keep key r of each 16-key run where r <= lim
                // query minus key position at key 0 of the tile
                const int dq = l32 - k0r;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int run0 = 32 * kb + 16 * hh;
                    int lim = tile_keys - 1 - run0;
                    if (a.causal) lim = min(lim, dq - run0);
                    const i32x16 ridx = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15};
                    const f32x16 ninf = -INFINITY;
                    s[kb] = ridx <= lim ? s[kb] : ninf;
                }
            }
            // online softmax (log2 domain: t = score * scale * log2 e)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = half_max(mx);
            const float m_new = fmaxf(m_run, mx * a.scale_log2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            // rescale O only when some row's maximum moved (wave-uniform test;
            // rows whose maximum did not move have alpha = 1)
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db) o_acc[db] *= alpha;
            }
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    f32x8 p;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        p[u] = fast_exp2(__builtin_fmaf(s[kb][8 * j + u], a.scale_log2, -m_use));
                        rs += p[u];
                    }
                    pb[kb][j] = __builtin_bit_cast(u32x4, __builtin_convertvector(p, bf16x8));
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
        }
        have_p = cmp;
        cursor_next(a, at, cq);
        // this wave's share of tile t+1 must have landed before the barrier
        // that opens the phase reading it; the copies of tile t+2 may still
        // be in flight
        if (t + 2 < T) wait_vmem<C::LOADS>();
        else wait_vmem<0>();
        __syncthreads();
    }
    if (loader) __syncthreads();    // match the second group's extra barrier

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
    if (COUNT && lane == 0 && (n_full | n_masked | n_skip)) {
        atomicAdd(a.counters + 0, (unsigned long long)n_full);
        atomicAdd(a.counters + 1, (unsigned long long)n_masked);
        atomicAdd(a.counters + 2, (unsigned long long)n_skip);
    }
}

// Four-wave variant: one wave per SIMD, several workgroups per CU running
// free of each other (no phase lock): each tile is copied into a double
// buffer, then every wave runs Q K^T, the softmax and P V on it at raised
// priority for the products, and one barrier ends the step. It keeps more
// independent waves per CU at d = 64 (four workgroups) and fills small grids;
// the ping-pong kernel above serves grouped-query shares at d = 128, whose
// long K/V streams favour its larger workgroups.
template <int D, bool COUNT>
__global__ void __launch_bounds__(256, 2)
fwd_bf16_4w_kernel(const FwdArgs a) {
    using C = Cfg<D>;
    constexpr int NW = 4;
    constexpr int RW = 32;
    // double buffer: [K tile | V tile], each [64 keys][D] bf16, swizzled
    __shared__ __attribute__((aligned(1024))) char smem[2 * C::BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int l32 = lane & 31, hh = lane >> 5;
    const unsigned lds0 = (unsigned)(unsigned long)(const lds_char*)smem;   // LDS address of the buffers

    // ---- workgroup -> (batch, kv head, query tile, key split); XCD-contiguous order ----
    // With S = a.n_split > 1 (small grids), S workgroups share a query tile,
    // each folding one contiguous part of its tile sequence into a partial
    // state that split_merge_kernel combines.
    const int S = a.n_split;
    const int bid = blockIdx.x;
    const int n_all = a.n_wg * S;
    const int per = n_all / 8, rem = n_all % 8;
    const int xcd = bid % 8, idx = bid / 8;
    const int logical = wg_permute(xcd * per + (xcd < rem ? xcd : rem) + idx, n_all, a.wg_mul, a.wg_add);
    const int sp = logical % S;
    const int lwg = logical / S;
    const int bg = lwg / a.wg_per_bg;
    const int qt = a.wg_per_bg - 1 - (lwg % a.wg_per_bg);  // heaviest first
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
    const int k_row = key_of_row(l32) * C::ROW_BYTES;
    const int kx = kswz<D>(key_of_row(l32));
    const int g16 = lane >> 4, src = lane & 15;
    const int v_key = 16 * (g16 >> 1) + (src >> 2);
    const int v_dim = 16 * (g16 & 1) + 4 * (src & 3);
    const int v_sw = vswz<D>(src >> 2);

    unsigned n_full = 0, n_masked = 0, n_skip = 0;

    // ---- tile sequence: blocks in the given (ring) order, 64 keys at a time ----
    const HeadAt at{b, g, kv_rs, D, wg_last_pos, wave_first_pos, a.causal};
    int T_all = 0;
    for (int t = 0; t < a.n_blocks; ++t) T_all += (keys_needed(a, t, wg_last_pos) + kBK - 1) / kBK;
    if constexpr (COUNT) n_skip = wave_valid && sp == 0 ? skipped_unvisited(a, T_all) : 0u;
    // this workgroup's part of the sequence: tiles [t_lo, t_lo + T)
    const int t_lo = (int)((long long)T_all * sp / S);
    const int T = (int)((long long)T_all * (sp + 1) / S) - t_lo;

    // Tile copies: copy n of every wave fills 1 KB region 4n + wave of the K
    // and of the V tile.
    constexpr int LOADS = C::REGIONS / 4;
    unsigned cpk[LOADS], cpv[LOADS];
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
        const int row = (n * 4 + wave) * C::ROWS_PER_KB + lane / C::UNITS;
        const int p = lane % C::UNITS;
        cpk[n] = (unsigned)(2 * (row * kv_rs + 8 * (p ^ kswz<D>(row))));
        cpv[n] = (unsigned)(2 * (row * kv_rs + 8 * (p ^ vswz<D>(row))));
    }
    Cursor ld = cursor_first(a, at);   // next tile to copy
    cursor_skip(a, at, ld, t_lo);
    auto issue = [&](unsigned buf) {
        const int key0 = ld.ti * kBK;
        const int rows = min(kBK, ld.len - key0);
        const unsigned bytes = (unsigned)(rows * kv_rs * 2);
        const i32x4 rk = make_rsrc(ld.kp + (long long)key0 * kv_rs, bytes);
        const i32x4 rv = make_rsrc(ld.vp + (long long)key0 * kv_rs, bytes);
#pragma unroll
        for (int n = 0; n < LOADS; ++n) {
            copy16_to_lds(rk, cpk[n], buf + (n * 4 + wave) * 1024);
            copy16_to_lds(rv, cpv[n], buf + C::TILE_BYTES + (n * 4 + wave) * 1024);
        }
        cursor_next(a, at, ld);
    };
    if (T > 0) issue(lds0);
    // the Q and state loads and the first tile's copies are in flight
    // together; this compiler-visible wait covers both
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();

    auto v_frag = [&](const lds_char* vt, int i) -> u32x4 {
        const int db = i % C::DB, j = (i / C::DB) % 2, kb = i / (2 * C::DB);
        const int key = 32 * kb + 8 * j + v_key;
        const int d = 32 * db + v_dim;
        const int off = key * C::ROW_BYTES + 16 * ((d >> 3) ^ v_sw) + 2 * (d & 7);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vt + off + 4 * C::ROW_BYTES));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    auto k_frag = [&](const lds_char* kt, int i) -> u32x4 {
        const int st = i / 2, kb = i % 2;
        return *(const lds_u32x4*)(kt + kb * 32 * C::ROW_BYTES + k_row + 16 * ((2 * st + hh) ^ kx));
    };
    constexpr int NPV = 4 * C::DB;       // P V products per tile
    constexpr int NQK = 2 * C::DSTEPS;   // Q K^T products per tile

    Cursor cq = cursor_first(a, at);   // tile this wave computes
    cursor_skip(a, at, cq, t_lo);
    for (int t = 0; t < T; ++t) {
        const int buf = t & 1;
        // the other buffer was last read before the barrier that ended the
        // previous step
        if (t + 1 < T) issue(lds0 + (buf ^ 1) * C::BUF_BYTES);
        const lds_char* kt = (const lds_char*)(smem + buf * C::BUF_BYTES);
        const lds_char* vt = kt + C::TILE_BYTES;
        // tile t against this wave's rows: k0r = position of the tile's key 0
        // minus the wave's first query position
        const int key0 = cq.ti * kBK;
        const int tile_keys = min(kBK, cq.len - key0);
        const int k0r = cq.all_full ? -(1 << 30) : min(cq.rel, kBK) + key0;
        const bool full = k0r + tile_keys - 1 <= 0;
        const bool cmp = wave_valid && k0r <= wave_rows - 1;
        const bool need_mask = !full || tile_keys < kBK;
        if constexpr (COUNT) {
            n_full += cmp && full ? 1u : 0u;
            n_masked += cmp && !full ? 1u : 0u;
            n_skip += wave_valid && !cmp ? 1u : 0u;
        }
        if (cmp) {
            // S^T = K Q^T : s[kb][r] = score(query row0 + l32, key key0 + 32kb + 16hh + r)
            __builtin_amdgcn_s_setprio(1);   // products first on the shared SIMD
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int i = 0; i < NQK; ++i)
                s[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(k_frag(kt, i)), as_bf16x8(qf[i / 2]), s[i % 2], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < NQK - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_s_setprio(0);
            if (need_mask) {
                const int dq = l32 - k0r;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int run0 = 32 * kb + 16 * hh;
                    int lim = tile_keys - 1 - run0;
                    if (a.causal) lim = min(lim, dq - run0);
                    const i32x16 ridx = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15};
                    const f32x16 ninf = -INFINITY;
                    s[kb] = ridx <= lim ? s[kb] : ninf;
                }
            }
            // online softmax (log2 domain: t = score * scale * log2 e)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = half_max(mx);
            const float m_new = fmaxf(m_run, mx * a.scale_log2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db) o_acc[db] *= alpha;
            }
            float rs = 0.f;
            u32x4 pb[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    f32x8 p;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        p[u] = fast_exp2(__builtin_fmaf(s[kb][8 * j + u], a.scale_log2, -m_use));
                        rs += p[u];
                    }
                    pb[kb][j] = __builtin_bit_cast(u32x4, __builtin_convertvector(p, bf16x8));
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
            // O^T += V^T P^T
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < NPV; ++i) {
                const int db = i % C::DB, j = (i / C::DB) % 2, kb = i / (2 * C::DB);
                o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(v_frag(vt, i)), as_bf16x8(pb[kb][j]), o_acc[db], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < NPV - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_s_setprio(0);
        }
        cursor_next(a, at, cq);
        // this wave's copies of tile t+1 must have landed before the barrier
        // that publishes it
        wait_vmem<0>();
        __syncthreads();
    }

    // ---- epilogue: store state, a split's partial state, or finalise into out / lse ----
    if (wave_valid) {
        const int row = row0 + l32;
        const float l_tot = half_sum(l_run);
        if (row < a.Tq) {
            const long long si = ((long long)b * a.Hq + h) * a.Tq + row;
            const long long oi = (((long long)b * a.Tq + row) * a.Hq + h) * D;
            if (S > 1) {
                // m in log2 units (-inf when the split saw no key of the row),
                // l, and the unnormalised o of split sp; o is stored with the
                // non-temporal (streaming) policy, as the merge kernel reads
                // it once (measured +1.5 % on the sharp-head shares)
                const long long wi = (long long)sp * a.split_rows + si;
                if (hh == 0) {
                    a.split_m[wi] = m_run;
                    a.split_l[wi] = l_tot;
                }
                float* orow = a.split_o + wi * D;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
                        f32x4 x;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) x[jj] = o_acc[db][4 * ib + jj];
                        __builtin_nontemporal_store(
                            x, reinterpret_cast<f32x4*>(orow + 32 * db + 8 * ib + 4 * hh));
                    }
            } else if (a.store_state) {
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
    if (COUNT && lane == 0 && (n_full | n_masked | n_skip)) {
        atomicAdd(a.counters + 0, (unsigned long long)n_full);
        atomicAdd(a.counters + 1, (unsigned long long)n_masked);
        atomicAdd(a.counters + 2, (unsigned long long)n_skip);
    }
}

// Which kernel serves a shape: the ping-pong kernel at d = 128 (grouped
// query heads: 1,039 against 910 TFLOP/s on the million-token share), the
// four-wave kernel at d = 64 (bidirectional share +43 %) and for small grids
// (which it also splits by key range, more workgroups than CUs).
// tasks = 32-row wave tasks of the launch (B * Hq * ceil(Tq / 32)).
bool use_four_waves(int D, int G, long long tasks) {
    if (D == 64) return true;
    // one query head per kv head: the ping-pong kernel once its grid fills
    // the CUs (one 8-wave workgroup each; 1,105 against 1,012 TFLOP/s on the
    // B8 H64 T32768 share), the four-wave kernel with key splits below that
    return G == 1 && tasks < 256LL * Cfg<128>::NW;
}

// Combine the S partial states of each row (log-sum-exp rule in log2 units):
// M = max_s m_s, L = sum_s 2^(m_s - M) l_s, out = sum_s 2^(m_s - M) o_s / L,
// lse = (M + log2 L) ln 2; a row no split saw gives out = 0, lse = -inf.
// D / 4 threads per row, 4 elements each.
template <int D>
__global__ void __launch_bounds__(256) split_merge_kernel(const FwdArgs a) {
    constexpr int TPR = D / 4;
    const long long rows = a.split_rows;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long si = i / TPR;
    if (si >= rows) return;
    const int c = (int)(i % TPR) * 4;
    const int S = a.n_split;
    float M = -INFINITY;
    for (int sp = 0; sp < S; ++sp) M = fmaxf(M, a.split_m[sp * rows + si]);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M > -INFINITY) {
        for (int sp = 0; sp < S; ++sp) {
            const long long wi = sp * rows + si;
            const float w = fast_exp2(a.split_m[wi] - M);
            L += w * a.split_l[wi];
            const f32x4 x = *reinterpret_cast<const f32x4*>(a.split_o + wi * D + c);
            o += w * x;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    o *= inv;
    // si = (b * Hq + h) * Tq + row
    const long long row = si % a.Tq, bh = si / a.Tq;
    const long long h = bh % a.Hq, b = bh / a.Hq;
    const long long oi = ((b * a.Tq + row) * a.Hq + h) * D + c;
    if (a.out_bf16) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.out) + oi) = __builtin_convertvector(o, bf16x4);
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + oi) = o;
    }
    if (c == 0 && a.lse) a.lse[si] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
int launch(const FwdArgs& args, void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    FwdArgs a = args;   // the launcher fills in the workgroup-order permutation for its grid
    if (use_four_waves(D, a.Hq / a.Hkv, (long long)a.B * a.Hq * ((a.Tq + 31) / 32))) {
        const unsigned grid = (unsigned)((long long)a.n_wg * a.n_split);
        const WgPerm pm = wg_perm(a.wg_order, grid);
        a.wg_mul = pm.mul;
        a.wg_add = pm.add;
        if (a.counters)
            hipLaunchKernelGGL((fwd_bf16_4w_kernel<D, true>), dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((fwd_bf16_4w_kernel<D, false>), dim3(grid), dim3(256), 0, s, a);
        if (a.n_split > 1) {
            const int e = (int)hipGetLastError();
            if (e) return e;
            const long long threads = a.split_rows * (D / 4);
            hipLaunchKernelGGL((split_merge_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                               dim3(256), 0, s, a);
        }
    } else if (a.counters) {
        const WgPerm pm = wg_perm(a.wg_order, a.n_wg);
        a.wg_mul = pm.mul;
        a.wg_add = pm.add;
        hipLaunchKernelGGL((fwd_bf16_kernel<D, true>), dim3(a.n_wg), dim3(64 * Cfg<D>::NW), 0, s, a);
    } else {
        const WgPerm pm = wg_perm(a.wg_order, a.n_wg);
        a.wg_mul = pm.mul;
        a.wg_add = pm.add;
        hipLaunchKernelGGL((fwd_bf16_kernel<D, false>), dim3(a.n_wg), dim3(64 * Cfg<D>::NW), 0, s, a);
    }
    return (int)hipGetLastError();
}

}  // namespace

int fwd_bf16_waves(int D, int G, long long tasks) {
    return use_four_waves(D, G, tasks) ? 4 : Cfg<128>::NW;
}

int launch_fwd_bf16(const FwdArgs& a, int D, void* stream) {
    if (D == 128) return launch<128>(a, stream);
    if (D == 64) return launch<64>(a, stream);
    return (int)hipErrorInvalidValue;
}

}  // namespace cakv
