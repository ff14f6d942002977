// api.cpp -- the C ABI of libcakv: argument checks, the ring schedule, and the
// launch of the kernels. Declarations, layouts and error rules: include/cakv.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "cakv.h"
#include "cakv_diag.h"
#include "bwd_args.h"
#include "decode_args.h"
#include "fwd_args.h"

namespace {

thread_local std::string g_err;
// workgroup-order permutation the launchers apply (cakv_diag_set_workgroup_order)
std::atomic<int> g_wg_order{0};

// Named ranges for timeline tools (rocprofv3 --marker-trace): every entry
// point that enqueues kernels is one range, and its enqueue step a range
// inside it, so a timeline shows the host's checks and scheduling apart from
// the launches. Nearly free when no tool is attached.
struct Range {
    explicit Range(const char* name) { roctxRangePushA(name); }
    ~Range() { roctxRangePop(); }
    Range(const Range&) = delete;
    Range& operator=(const Range&) = delete;
};

cakv_status fail(cakv_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

cakv_status ok() {
    g_err.clear();
    return CAKV_OK;
}

cakv_status hip_status(int err, const char* what) {
    if (err == (int)hipSuccess) return ok();
    return fail(CAKV_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

cakv_class classify(int64_t q_off, int64_t q_len, int64_t kv_off, int64_t kv_len, int causal) {
    if (q_len <= 0 || kv_len <= 0) return CAKV_SKIP;
    if (!causal) return CAKV_FULL;
    const int64_t q_last = q_off + q_len - 1, kv_last = kv_off + kv_len - 1;
    if (kv_off > q_last) return CAKV_SKIP;
    if (kv_last <= q_off) return CAKV_FULL;
    return CAKV_DIAG;
}

constexpr long long kMaxHeadsTimesD = 1LL << 24;

cakv_status check_common(int dtype, int B, int Hq, int Hkv, int Tq, int Tkv, int D) {
    if (dtype != CAKV_F32 && dtype != CAKV_BF16)
        return fail(CAKV_ERR_DTYPE, "dtype %d is neither CAKV_F32 nor CAKV_BF16", dtype);
    if (B < 0 || Tq < 0 || Tkv < 0)
        return fail(CAKV_ERR_SHAPE, "negative size (B=%d Tq=%d Tkv=%d)", B, Tq, Tkv);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return fail(CAKV_ERR_SHAPE, "heads must be positive with Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                    Hq, Hkv);
    if (D != 64 && D != 128) return fail(CAKV_ERR_SHAPE, "D=%d unsupported (64 or 128)", D);
    // the kernels' per-tile buffer ranges (up to 64 rows of Hq * D bf16) are 32-bit
    if ((long long)Hq * D > kMaxHeadsTimesD)
        return fail(CAKV_ERR_SHAPE, "Hq * D = %lld above %lld", (long long)Hq * D, kMaxHeadsTimesD);
    return CAKV_OK;
}

float resolve_scale(float scale, int D) {
    return scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
}

// Fill the workgroup geometry of a forward launch (the grid is at most
// 2^31 - 1 workgroups).
cakv_status set_grid(cakv::FwdArgs& a, int dtype, int D) {
    long long per_bg, n_wg;
    if (dtype == CAKV_BF16) {
        const long long G = a.Hq / a.Hkv;
        const long long npblk = (a.Tq + 31LL) / 32;   // 32 query rows per wave
        const long long nw = cakv::fwd_bf16_waves(D, (int)G, (long long)a.B * a.Hq * npblk);
        per_bg = (G * npblk + nw - 1) / nw;
        n_wg = (long long)a.B * a.Hkv * per_bg;
    } else {
        const long long rows = cakv::fwd_f32_wg_rows();
        per_bg = (a.Tq + rows - 1) / rows;
        n_wg = (long long)a.B * a.Hq * per_bg;
    }
    if (n_wg > 2147483647LL) return fail(CAKV_ERR_SHAPE, "forward grid too large (%lld workgroups)", n_wg);
    a.wg_per_bg = (int)per_bg;
    a.n_wg = (int)n_wg;
    a.n_split = 1;
    return CAKV_OK;
}

// Key splits and workspace bytes of the split path for a whole-shard forward
// (bf16 four-wave shapes whose grid leaves resident slots empty); 1 / 0 when
// the grid is not split.
struct SplitPlan {
    int n_split;
    long long rows;
    long long bytes;
};
SplitPlan split_plan(int dtype, int B, int Hq, int Hkv, int Tq, int D) {
    SplitPlan p{1, (long long)B * Hq * Tq, 0};
    if (dtype != CAKV_BF16 || p.rows == 0) return p;
    const long long G = Hq / Hkv;
    const long long nw = cakv::fwd_bf16_waves(D, (int)G, (long long)B * Hq * ((Tq + 31LL) / 32));
    if (nw != 4) return p;   // only the four-wave kernel splits
    const long long per_bg = (G * ((Tq + 31LL) / 32) + nw - 1) / nw;
    const long long n_wg = (long long)B * Hkv * per_bg;
    // enough parts that the grid fills the resident workgroup slots of the
    // four-wave kernel (256 CUs x 2 workgroups at d = 128, x 4 at d = 64, as
    // its registers and LDS allow), at most 8
    const long long slots = 256LL * (D == 64 ? 4 : 2);
    if (n_wg >= slots) return p;
    const int S = (int)std::min(8LL, (slots + n_wg - 1) / n_wg);
    if (S <= 1) return p;
    p.n_split = S;
    const long long ml = 2LL * S * p.rows;
    p.bytes = ((ml + 3) / 4 * 4 + (long long)S * p.rows * D) * 4;
    return p;
}

// Use the split path when the caller's workspace holds it.
void apply_split(cakv::FwdArgs& a, const SplitPlan& p, void* workspace, int64_t workspace_bytes) {
    if (p.n_split <= 1 || !workspace || workspace_bytes < p.bytes) return;
    float* w = static_cast<float*>(workspace);
    const long long ml = 2LL * p.n_split * p.rows;
    a.n_split = p.n_split;
    a.split_rows = p.rows;
    a.split_m = w;
    a.split_l = w + (long long)p.n_split * p.rows;
    a.split_o = w + (ml + 3) / 4 * 4;
}

int launch_fwd(const cakv::FwdArgs& a, int dtype, int D, void* stream) {
    if (dtype == CAKV_BF16) return cakv::launch_fwd_bf16(a, D, stream);
    return cakv::launch_fwd_f32(a, D, stream);
}

// Decode plan: how many splits the history's 32-key tiles are cut into,
// each split at least one tile. Few, long splits read the history fastest:
// 768 waves in all (192 workgroups of four kv heads, on three quarters of the
// CUs) when heads are grouped, 512 single-head waves otherwise. Measured on
// the million-token history, one MI355X, four-head workgroups: 512 waves
// 5,958-5,969 GB/s, 640 6,696-6,710, 768 6,935-6,940, 896 6,819-6,822, 1,024
// 6,738-6,747, 1,536 6,256-6,259 (another MI355X: 2,048 6,115-6,154, 3,072
// 6,068-6,074, 4,096 6,001-6,020); single-head waves 512 6,686, 1,536 5,957.
struct DecodePlan {
    int nrb;               // 32-row blocks per (batch, kv head)
    long long tiles;       // tiles of all portions
    int tiles_per_split;
    int n_splits;
    long long ws_bytes;    // m, l, o of every split's rows
};

cakv_status decode_plan(int B, int Hq, int Hkv, int Tn, int D, const int64_t* kv_len,
                        int n_portions, DecodePlan* p) {
    if (B < 0 || Tn < 0) return fail(CAKV_ERR_SHAPE, "negative size (B=%d Tn=%d)", B, Tn);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return fail(CAKV_ERR_SHAPE, "heads must be positive with Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                    Hq, Hkv);
    if (D != 64 && D != 128) return fail(CAKV_ERR_SHAPE, "D=%d unsupported (64 or 128)", D);
    if ((long long)Hq * D > kMaxHeadsTimesD)
        return fail(CAKV_ERR_SHAPE, "Hq * D = %lld above %lld", (long long)Hq * D, kMaxHeadsTimesD);
    if (n_portions < 1 || n_portions > CAKV_MAX_CHUNKS)
        return fail(CAKV_ERR_RANGE, "n_portions=%d outside [1, %d]", n_portions, CAKV_MAX_CHUNKS);
    if (!kv_len) return fail(CAKV_ERR_NULL, "kv_len_host is NULL");
    long long tiles = 0;
    for (int j = 0; j < n_portions; ++j) {
        if (kv_len[j] < 0 || kv_len[j] > 2147483647LL - cakv::kDecTile)
            return fail(CAKV_ERR_SHAPE, "portion %d length %lld out of range", j, (long long)kv_len[j]);
        tiles += (kv_len[j] + cakv::kDecTile - 1) / cakv::kDecTile;
    }
    if (tiles > 2147483647LL) return fail(CAKV_ERR_SHAPE, "too many key tiles (%lld)", tiles);
    const long long R = (long long)(Hq / Hkv) * Tn;
    p->nrb = (int)((R + 31) / 32);
    p->tiles = tiles;
    const long long per_split = std::max(1LL, (long long)B * Hkv * p->nrb);
    const long long waves = cakv::decode_heads_per_wg(Hkv) > 1 ? 768 : 512;
    long long want = std::max(1LL, (waves + per_split - 1) / per_split);
    want = std::min(want, std::max(1LL, tiles));
    const long long tps = std::max(1LL, (tiles + want - 1) / want);
    p->tiles_per_split = (int)tps;
    p->n_splits = (int)std::max(1LL, (tiles + tps - 1) / tps);   // <= 4096 (merge weights in LDS)
    if (p->n_splits > 4096) return fail(CAKV_ERR_INTERNAL, "decode plan: %d splits", p->n_splits);
    p->ws_bytes = (long long)p->n_splits * per_split * 32 * (D + 2) * 4;
    if ((long long)p->n_splits * per_split > 2147483647LL)
        return fail(CAKV_ERR_SHAPE, "decode grid too large");
    return CAKV_OK;
}

}  // namespace

extern "C" {

int cakv_abi_version(void) { return CAKV_ABI_VERSION; }

const char* cakv_status_str(int status) {
    switch (status) {
        case CAKV_OK: return "CAKV_OK";
        case CAKV_ERR_NULL: return "CAKV_ERR_NULL";
        case CAKV_ERR_SHAPE: return "CAKV_ERR_SHAPE";
        case CAKV_ERR_DTYPE: return "CAKV_ERR_DTYPE";
        case CAKV_ERR_ALIGN: return "CAKV_ERR_ALIGN";
        case CAKV_ERR_RANGE: return "CAKV_ERR_RANGE";
        case CAKV_ERR_HIP: return "CAKV_ERR_HIP";
        case CAKV_ERR_INTERNAL: return "CAKV_ERR_INTERNAL";
        default: return "CAKV_UNKNOWN_STATUS";
    }
}

const char* cakv_last_error(void) { return g_err.c_str(); }

cakv_status cakv_classify_block(int64_t q_offset, int64_t q_len, int64_t kv_offset,
                                int64_t kv_len, int causal, int8_t* class_host) {
    if (!class_host) return fail(CAKV_ERR_NULL, "class_host is NULL");
    if (q_len < 0 || kv_len < 0) return fail(CAKV_ERR_SHAPE, "negative length");
    *class_host = (int8_t)classify(q_offset, q_len, kv_offset, kv_len, causal);
    return ok();
}

cakv_status cakv_schedule(int rank, int n_chunks, int64_t chunk_len, int causal,
                          int32_t* blocks_host, int8_t* class_host) {
    if (!blocks_host || !class_host) return fail(CAKV_ERR_NULL, "output array is NULL");
    if (n_chunks < 1 || n_chunks > CAKV_MAX_CHUNKS)
        return fail(CAKV_ERR_RANGE, "n_chunks=%d outside [1, %d]", n_chunks, CAKV_MAX_CHUNKS);
    if (rank < 0 || rank >= n_chunks)
        return fail(CAKV_ERR_RANGE, "rank=%d outside [0, %d)", rank, n_chunks);
    if (chunk_len < 0) return fail(CAKV_ERR_SHAPE, "chunk_len=%lld < 0", (long long)chunk_len);
    for (int k = 0; k < n_chunks; ++k) {
        const int j = ((rank - k) % n_chunks + n_chunks) % n_chunks;
        blocks_host[k] = j;
        class_host[k] = (int8_t)classify((int64_t)rank * chunk_len, chunk_len,
                                         (int64_t)j * chunk_len, chunk_len, causal);
    }
    return ok();
}

cakv_status cakv_state_init(float* m, float* l, float* o, int B, int Hq, int Tq, int D,
                            void* stream) {
    const Range range("cakv_state_init");
    if (B < 0 || Hq < 0 || Tq < 0) return fail(CAKV_ERR_SHAPE, "negative size");
    if (D != 64 && D != 128) return fail(CAKV_ERR_SHAPE, "D=%d unsupported (64 or 128)", D);
    const long long rows = (long long)B * Hq * Tq;
    if (rows == 0) return ok();
    if (!m || !l || !o) return fail(CAKV_ERR_NULL, "state pointer is NULL");
    if (!aligned16(o)) return fail(CAKV_ERR_ALIGN, "o not 16-byte aligned");
    const Range enq("enqueue");
    return hip_status(cakv::launch_state_init(m, l, o, rows, D, stream), "state_init launch");
}

cakv_status cakv_block_update(const void* q, const void* k, const void* v, int dtype, int B,
                              int Hq, int Hkv, int Tq, int Tkv, int D, int64_t q_offset,
                              int64_t kv_offset, int causal, float scale, float* m, float* l,
                              float* o, int64_t* tile_counters, void* stream) {
    const Range range("cakv_block_update");
    cakv_status s = check_common(dtype, B, Hq, Hkv, Tq, Tkv, D);
    if (s != CAKV_OK) return s;
    if (B == 0 || Tq == 0) return ok();
    if (!q || !m || !l || !o) return fail(CAKV_ERR_NULL, "q or state pointer is NULL");
    if (Tkv > 0 && (!k || !v)) return fail(CAKV_ERR_NULL, "k or v is NULL");
    if (!aligned16(q) || !aligned16(o) || (Tkv > 0 && (!aligned16(k) || !aligned16(v))))
        return fail(CAKV_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
    if (tile_counters && (reinterpret_cast<uintptr_t>(tile_counters) & 7u))
        return fail(CAKV_ERR_ALIGN, "tile_counters not 8-byte aligned");
    if (classify(q_offset, Tq, kv_offset, Tkv, causal) == CAKV_SKIP) {
        if (!tile_counters) return ok();
        // nothing to compute: every tile of the block is skipped
        const unsigned long long tiles = (unsigned long long)B * Hq *
                                         (unsigned long long)((Tq + CAKV_TILE_Q - 1) / CAKV_TILE_Q) *
                                         (unsigned long long)((Tkv + CAKV_TILE_K - 1) / CAKV_TILE_K);
        if (tiles == 0) return ok();
        return hip_status(cakv::launch_counter_add(
                              reinterpret_cast<unsigned long long*>(tile_counters) + 2, tiles,
                              stream),
                          "block_update counter launch");
    }

    cakv::FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.wg_order = g_wg_order.load(std::memory_order_relaxed);
    a.q = q;
    a.k[0] = k;
    a.v[0] = v;
    a.kv_off[0] = kv_offset;
    a.kv_len[0] = Tkv;
    a.n_blocks = 1;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq;
    a.q_off = q_offset;
    a.scale_log2 = resolve_scale(scale, D) * 1.4426950408889634f;
    a.causal = causal ? 1 : 0;
    a.m = m; a.l = l; a.o = o;
    a.load_state = 1;
    a.store_state = 1;
    a.counters = reinterpret_cast<unsigned long long*>(tile_counters);
    s = set_grid(a, dtype, D);
    if (s != CAKV_OK) return s;
    const Range enq("enqueue");
    return hip_status(launch_fwd(a, dtype, D, stream), "block_update launch");
}

cakv_status cakv_finalize(const float* m, const float* l, const float* o, void* out,
                          int out_dtype, float* lse, int B, int Hq, int Tq, int D, void* stream) {
    const Range range("cakv_finalize");
    if (out_dtype != CAKV_F32 && out_dtype != CAKV_BF16)
        return fail(CAKV_ERR_DTYPE, "out_dtype %d unknown", out_dtype);
    if (B < 0 || Hq < 0 || Tq < 0) return fail(CAKV_ERR_SHAPE, "negative size");
    if (D != 64 && D != 128) return fail(CAKV_ERR_SHAPE, "D=%d unsupported (64 or 128)", D);
    if ((long long)B * Hq * Tq == 0) return ok();
    if (!m || !l || !o || !out) return fail(CAKV_ERR_NULL, "m, l, o or out is NULL");
    if (!aligned16(o) || !aligned16(out)) return fail(CAKV_ERR_ALIGN, "o/out not 16-byte aligned");
    const Range enq("enqueue");
    return hip_status(cakv::launch_finalize(m, l, o, out, out_dtype == CAKV_BF16, lse, B, Hq, Tq,
                                            D, stream),
                      "finalize launch");
}

cakv_status cakv_lse_merge(const float* o_a, const float* lse_a, const float* o_b,
                           const float* lse_b, float* o_out, float* lse_out, int B, int Hq,
                           int Tq, int D, void* stream) {
    const Range range("cakv_lse_merge");
    if (B < 0 || Hq < 0 || Tq < 0) return fail(CAKV_ERR_SHAPE, "negative size");
    if (D != 64 && D != 128) return fail(CAKV_ERR_SHAPE, "D=%d unsupported (64 or 128)", D);
    if ((long long)B * Hq * Tq == 0) return ok();
    if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out)
        return fail(CAKV_ERR_NULL, "merge operand is NULL");
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out))
        return fail(CAKV_ERR_ALIGN, "o operands must be 16-byte aligned");
    const Range enq("enqueue");
    return hip_status(cakv::launch_lse_merge(o_a, lse_a, o_b, lse_b, o_out, lse_out, B, Hq, Tq, D,
                                             stream),
                      "lse_merge launch");
}

cakv_status cakv_local_shard_forward(const void* q_local, const void* const* k_blocks_host,
                                     const void* const* v_blocks_host, int dtype, int B,
                                     int Hq, int Hkv, int chunk_len, int n_chunks, int D,
                                     int rank, int causal, float scale, void* out,
                                     int out_dtype, float* lse, void* workspace,
                                     int64_t workspace_bytes, int64_t* tile_counters,
                                     void* stream) {
    const Range range("cakv_local_shard_forward");
    cakv_status s = check_common(dtype, B, Hq, Hkv, chunk_len, chunk_len, D);
    if (s != CAKV_OK) return s;
    if (out_dtype != CAKV_F32 && out_dtype != CAKV_BF16)
        return fail(CAKV_ERR_DTYPE, "out_dtype %d unknown", out_dtype);
    if (n_chunks < 1 || n_chunks > CAKV_MAX_CHUNKS)
        return fail(CAKV_ERR_RANGE, "n_chunks=%d outside [1, %d]", n_chunks, CAKV_MAX_CHUNKS);
    if (rank < 0 || rank >= n_chunks)
        return fail(CAKV_ERR_RANGE, "rank=%d outside [0, %d)", rank, n_chunks);
    if (B == 0 || chunk_len == 0) return ok();
    if (!q_local || !out) return fail(CAKV_ERR_NULL, "q_local or out is NULL");
    if (!k_blocks_host || !v_blocks_host) return fail(CAKV_ERR_NULL, "block pointer array is NULL");
    if (!aligned16(q_local) || !aligned16(out))
        return fail(CAKV_ERR_ALIGN, "q_local/out not 16-byte aligned");
    if (workspace && !aligned16(workspace)) return fail(CAKV_ERR_ALIGN, "workspace not 16-byte aligned");
    if (workspace_bytes < 0) return fail(CAKV_ERR_SHAPE, "negative workspace size");
    if (tile_counters && (reinterpret_cast<uintptr_t>(tile_counters) & 7u))
        return fail(CAKV_ERR_ALIGN, "tile_counters not 8-byte aligned");

    int32_t order[CAKV_MAX_CHUNKS];
    int8_t cls[CAKV_MAX_CHUNKS];
    s = cakv_schedule(rank, n_chunks, chunk_len, causal, order, cls);
    if (s != CAKV_OK) return s;

    cakv::FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.wg_order = g_wg_order.load(std::memory_order_relaxed);
    int n = 0;
    for (int t = 0; t < n_chunks; ++t) {
        if (cls[t] == CAKV_SKIP) {
            a.skip_tiles += (chunk_len + CAKV_TILE_K - 1) / CAKV_TILE_K;
            continue;
        }
        const int j = order[t];
        const void* kp = k_blocks_host[j];
        const void* vp = v_blocks_host[j];
        if (!kp || !vp) return fail(CAKV_ERR_NULL, "block %d pointer is NULL", j);
        if (!aligned16(kp) || !aligned16(vp))
            return fail(CAKV_ERR_ALIGN, "block %d not 16-byte aligned", j);
        a.k[n] = kp;
        a.v[n] = vp;
        a.kv_off[n] = (long long)j * chunk_len;
        a.kv_len[n] = chunk_len;
        ++n;
    }
    a.q = q_local;
    a.n_blocks = n;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = chunk_len;
    a.q_off = (long long)rank * chunk_len;
    a.scale_log2 = resolve_scale(scale, D) * 1.4426950408889634f;
    a.causal = causal ? 1 : 0;
    a.load_state = 0;
    a.store_state = 0;
    a.out = out;
    a.out_bf16 = out_dtype == CAKV_BF16;
    a.lse = lse;
    a.counters = reinterpret_cast<unsigned long long*>(tile_counters);
    s = set_grid(a, dtype, D);
    if (s != CAKV_OK) return s;
    apply_split(a, split_plan(dtype, B, Hq, Hkv, chunk_len, D), workspace, workspace_bytes);
    const Range enq("enqueue");
    return hip_status(launch_fwd(a, dtype, D, stream), "local_shard_forward launch");
}

cakv_status cakv_forward_blocks(const void* q, const void* const* k_blocks_host,
                                const void* const* v_blocks_host, const int64_t* kv_len_host,
                                const int64_t* kv_off_host, int n_blocks, int dtype, int B,
                                int Hq, int Hkv, int Tq, int D, int64_t q_offset, int causal,
                                float scale, void* out, int out_dtype, float* lse,
                                void* workspace, int64_t workspace_bytes,
                                int64_t* tile_counters, void* stream) {
    const Range range("cakv_forward_blocks");
    cakv_status s = check_common(dtype, B, Hq, Hkv, Tq, 0, D);
    if (s != CAKV_OK) return s;
    if (out_dtype != CAKV_F32 && out_dtype != CAKV_BF16)
        return fail(CAKV_ERR_DTYPE, "out_dtype %d unknown", out_dtype);
    if (n_blocks < 1 || n_blocks > CAKV_MAX_CHUNKS)
        return fail(CAKV_ERR_RANGE, "n_blocks=%d outside [1, %d]", n_blocks, CAKV_MAX_CHUNKS);
    if (!kv_len_host || !kv_off_host) return fail(CAKV_ERR_NULL, "block length / offset array is NULL");
    for (int t = 0; t < n_blocks; ++t)
        if (kv_len_host[t] < 0 || kv_len_host[t] > 2147483647LL)
            return fail(CAKV_ERR_SHAPE, "block %d length %lld out of range", t,
                        (long long)kv_len_host[t]);
    if (B == 0 || Tq == 0) return ok();
    if (!q || !out) return fail(CAKV_ERR_NULL, "q or out is NULL");
    if (!k_blocks_host || !v_blocks_host) return fail(CAKV_ERR_NULL, "block pointer array is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(CAKV_ERR_ALIGN, "q/out not 16-byte aligned");
    if (workspace && !aligned16(workspace)) return fail(CAKV_ERR_ALIGN, "workspace not 16-byte aligned");
    if (workspace_bytes < 0) return fail(CAKV_ERR_SHAPE, "negative workspace size");
    if (tile_counters && (reinterpret_cast<uintptr_t>(tile_counters) & 7u))
        return fail(CAKV_ERR_ALIGN, "tile_counters not 8-byte aligned");

    cakv::FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.wg_order = g_wg_order.load(std::memory_order_relaxed);
    int n = 0;
    for (int t = 0; t < n_blocks; ++t) {
        if (classify(q_offset, Tq, kv_off_host[t], kv_len_host[t], causal) == CAKV_SKIP) {
            a.skip_tiles += (kv_len_host[t] + CAKV_TILE_K - 1) / CAKV_TILE_K;
            continue;
        }
        const void* kp = k_blocks_host[t];
        const void* vp = v_blocks_host[t];
        if (!kp || !vp) return fail(CAKV_ERR_NULL, "block %d pointer is NULL", t);
        if (!aligned16(kp) || !aligned16(vp))
            return fail(CAKV_ERR_ALIGN, "block %d not 16-byte aligned", t);
        a.k[n] = kp;
        a.v[n] = vp;
        a.kv_off[n] = kv_off_host[t];
        a.kv_len[n] = (int)kv_len_host[t];
        ++n;
    }
    a.q = q;
    a.n_blocks = n;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq;
    a.q_off = q_offset;
    a.scale_log2 = resolve_scale(scale, D) * 1.4426950408889634f;
    a.causal = causal ? 1 : 0;
    a.out = out;
    a.out_bf16 = out_dtype == CAKV_BF16;
    a.lse = lse;
    a.counters = reinterpret_cast<unsigned long long*>(tile_counters);
    s = set_grid(a, dtype, D);
    if (s != CAKV_OK) return s;
    apply_split(a, split_plan(dtype, B, Hq, Hkv, Tq, D), workspace, workspace_bytes);
    const Range enq("enqueue");
    return hip_status(launch_fwd(a, dtype, D, stream), "forward_blocks launch");
}

cakv_status cakv_forward_workspace_size(int dtype, int B, int Hq, int Hkv, int Tq, int D,
                                        int64_t* bytes_host) {
    if (!bytes_host) return fail(CAKV_ERR_NULL, "bytes_host is NULL");
    const cakv_status s = check_common(dtype, B, Hq, Hkv, Tq, 0, D);
    if (s != CAKV_OK) return s;
    *bytes_host = split_plan(dtype, B, Hq, Hkv, Tq, D).bytes;
    return ok();
}

cakv_status cakv_backward_workspace_size(int B, int Hq, int Tq, int64_t* bytes_host) {
    if (!bytes_host) return fail(CAKV_ERR_NULL, "bytes_host is NULL");
    if (B < 0 || Hq < 0 || Tq < 0) return fail(CAKV_ERR_SHAPE, "negative size");
    *bytes_host = (int64_t)B * Hq * Tq * 8;   // -delta, then -lse / scale, per row
    return ok();
}

cakv_status cakv_backward_blocks(const void* q, const void* const* k_blocks_host,
                                 const void* const* v_blocks_host, const int64_t* kv_len_host,
                                 const int64_t* kv_off_host, int n_blocks, int dtype, int B,
                                 int Hq, int Hkv, int Tq, int D, int64_t q_offset, int causal,
                                 float scale, const float* out, const float* lse,
                                 const void* dout, float* dq, float* const* dk_blocks_host,
                                 float* const* dv_blocks_host, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
    const Range range("cakv_backward_blocks");
    cakv_status s = check_common(dtype, B, Hq, Hkv, Tq, 0, D);
    if (s != CAKV_OK) return s;
    if (dtype != CAKV_BF16) return fail(CAKV_ERR_DTYPE, "cakv_backward_blocks takes bf16 inputs only");
    if (n_blocks < 1 || n_blocks > CAKV_MAX_CHUNKS)
        return fail(CAKV_ERR_RANGE, "n_blocks=%d outside [1, %d]", n_blocks, CAKV_MAX_CHUNKS);
    if (!kv_len_host || !kv_off_host) return fail(CAKV_ERR_NULL, "block length / offset array is NULL");
    long long key_tiles = 0;
    for (int t = 0; t < n_blocks; ++t) {
        if (kv_len_host[t] < 0 || kv_len_host[t] > 2147483647LL - cakv::kBwdKeyTile)
            return fail(CAKV_ERR_SHAPE, "block %d length %lld out of range", t,
                        (long long)kv_len_host[t]);
        key_tiles += (kv_len_host[t] + cakv::kBwdKeyTile - 1) / cakv::kBwdKeyTile;
    }
    if (B == 0) return ok();
    if (!k_blocks_host || !v_blocks_host || !dk_blocks_host || !dv_blocks_host)
        return fail(CAKV_ERR_NULL, "block pointer array is NULL");
    if (Tq > 0 && (!q || !out || !lse || !dout || !dq))
        return fail(CAKV_ERR_NULL, "q, out, lse, dout or dq is NULL");
    if (Tq > 0 && !workspace) return fail(CAKV_ERR_NULL, "workspace is NULL");
    if (workspace_bytes < (int64_t)B * Hq * Tq * 8)
        return fail(CAKV_ERR_SHAPE, "workspace of %lld bytes, %lld needed",
                    (long long)workspace_bytes, (long long)B * Hq * Tq * 8);
    if ((Tq > 0 && (!aligned16(q) || !aligned16(out) || !aligned16(dout) || !aligned16(dq))) ||
        !aligned16(workspace))
        return fail(CAKV_ERR_ALIGN, "q/out/dout/dq/workspace not 16-byte aligned");
    if (key_tiles > 2147483647LL / ((long long)B * Hkv))
        return fail(CAKV_ERR_SHAPE, "too many key tiles");

    cakv::BwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.wg_order = g_wg_order.load(std::memory_order_relaxed);
    int kt = 0;
    for (int t = 0; t < n_blocks; ++t) {
        a.kt0[t] = kt;
        a.kv_len[t] = (int)kv_len_host[t];
        a.kv_off[t] = kv_off_host[t];
        if (kv_len_host[t] > 0) {
            if (!k_blocks_host[t] || !v_blocks_host[t] || !dk_blocks_host[t] || !dv_blocks_host[t])
                return fail(CAKV_ERR_NULL, "block %d pointer is NULL", t);
            if (!aligned16(k_blocks_host[t]) || !aligned16(v_blocks_host[t]) ||
                !aligned16(dk_blocks_host[t]) || !aligned16(dv_blocks_host[t]))
                return fail(CAKV_ERR_ALIGN, "block %d not 16-byte aligned", t);
            a.k[t] = k_blocks_host[t];
            a.v[t] = v_blocks_host[t];
            a.dk[t] = dk_blocks_host[t];
            a.dv[t] = dv_blocks_host[t];
        }
        kt += (int)((kv_len_host[t] + cakv::kBwdKeyTile - 1) / cakv::kBwdKeyTile);
    }
    a.kt0[n_blocks] = kt;
    a.n_blocks = n_blocks;
    a.q = q;
    a.dout = dout;
    a.out = out;
    a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq;
    a.q_off = q_offset;
    a.scale = resolve_scale(scale, D);
    a.scale_log2 = a.scale * 1.4426950408889634f;
    a.causal = causal ? 1 : 0;
    a.ndelta = static_cast<float*>(workspace);
    a.nlse = a.ndelta + (long long)B * Hq * Tq;
    a.dq = dq;
    const int G = Hq / Hkv;
    const long long npblk = (Tq + 31) / 32;
    const long long dq_per_bg = (G * npblk + 3) / 4;
    if ((long long)B * Hkv * dq_per_bg > 2147483647LL)
        return fail(CAKV_ERR_SHAPE, "backward grid too large");
    a.wg_per_bg = (int)dq_per_bg;
    if (Tq == 0) {
        // no queries: every key gradient is zero (the dK/dV kernel visits no query tile)
        a.wg_per_bg = 0;
    }
    if (kt == 0 && Tq == 0) return ok();
    const Range enq("enqueue");
    return hip_status(cakv::launch_bwd(a, D, stream), "backward launch");
}

cakv_status cakv_decode_workspace_size(int B, int Hq, int Hkv, int Tn, int D,
                                       const int64_t* kv_len_host, int n_portions,
                                       int64_t* bytes_host) {
    if (!bytes_host) return fail(CAKV_ERR_NULL, "bytes_host is NULL");
    DecodePlan p;
    const cakv_status s = decode_plan(B, Hq, Hkv, Tn, D, kv_len_host, n_portions, &p);
    if (s != CAKV_OK) return s;
    *bytes_host = (B == 0 || Tn == 0) ? 0 : p.ws_bytes;
    return ok();
}

}  // extern "C"

namespace {

// Checks of cakv_decode shared with cakv_decode_noalloc (everything but the
// workspace); fills the plan. `*empty` is set when there is nothing to do.
cakv_status decode_check(const void* q, const void* const* k_portions_host,
                         const void* const* v_portions_host, const int64_t* kv_len_host,
                         const int64_t* kv_off_host, int n_portions, int dtype, int B, int Hq,
                         int Hkv, int Tn, int D, void* out, int out_dtype, DecodePlan* p,
                         bool* empty) {
    *empty = false;
    if (dtype != CAKV_BF16 && dtype != CAKV_F32)
        return fail(CAKV_ERR_DTYPE, "dtype %d is neither CAKV_F32 nor CAKV_BF16", dtype);
    if (dtype != CAKV_BF16)
        return fail(CAKV_ERR_DTYPE, "cakv_decode takes bf16 inputs only");
    if (out_dtype != CAKV_F32 && out_dtype != CAKV_BF16)
        return fail(CAKV_ERR_DTYPE, "out_dtype %d unknown", out_dtype);
    cakv_status s = decode_plan(B, Hq, Hkv, Tn, D, kv_len_host, n_portions, p);
    if (s != CAKV_OK) return s;
    if (B == 0 || Tn == 0) {
        *empty = true;
        return ok();
    }
    if (!q || !out) return fail(CAKV_ERR_NULL, "q or out is NULL");
    if (!k_portions_host || !v_portions_host || !kv_off_host)
        return fail(CAKV_ERR_NULL, "portion pointer / offset array is NULL");
    if (!aligned16(q) || !aligned16(out)) return fail(CAKV_ERR_ALIGN, "q/out not 16-byte aligned");
    for (int j = 0; j < n_portions; ++j) {
        if (kv_len_host[j] == 0) continue;
        const void* kp = k_portions_host[j];
        const void* vp = v_portions_host[j];
        if (!kp || !vp) return fail(CAKV_ERR_NULL, "portion %d pointer is NULL", j);
        if (!aligned16(kp) || !aligned16(vp))
            return fail(CAKV_ERR_ALIGN, "portion %d not 16-byte aligned", j);
    }
    return ok();
}

// The two decode kernels on a checked problem, with the splits' states in
// `workspace` (at least plan.ws_bytes, 16-byte aligned).
cakv_status decode_launch(const void* q, const void* const* k_portions_host,
                          const void* const* v_portions_host, const int64_t* kv_len_host,
                          const int64_t* kv_off_host, int n_portions, int B, int Hq, int Hkv,
                          int Tn, int D, int64_t q_off, int causal, float scale, void* out,
                          int out_dtype, float* lse, const DecodePlan& p, void* workspace,
                          void* stream) {
    cakv_status s;
    cakv::DecArgs a;
    std::memset(&a, 0, sizeof a);
    a.wg_order = g_wg_order.load(std::memory_order_relaxed);
    int tile = 0;
    for (int j = 0; j < n_portions; ++j) {
        a.tile0[j] = tile;
        a.kv_len[j] = (int)kv_len_host[j];
        a.kv_off[j] = kv_off_host[j];
        if (kv_len_host[j] > 0) {
            a.k[j] = k_portions_host[j];
            a.v[j] = v_portions_host[j];
        }
        tile += (int)((kv_len_host[j] + cakv::kDecTile - 1) / cakv::kDecTile);
    }
    a.tile0[n_portions] = tile;
    a.n_portions = n_portions;
    a.q = q;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tn = Tn;
    a.q_off = q_off;
    a.scale_log2 = resolve_scale(scale, D) * 1.4426950408889634f;
    a.causal = causal ? 1 : 0;
    a.nrb = p.nrb;
    a.tiles_per_split = p.tiles_per_split;
    a.n_splits = p.n_splits;
    const long long rows = (long long)p.n_splits * B * Hkv * p.nrb * 32;
    a.ws_m = static_cast<float*>(workspace);
    a.ws_l = a.ws_m + rows;
    a.ws_o = a.ws_l + rows + ((4 - (2 * rows) % 4) % 4);   // 16-byte aligned rows
    a.out = out;
    a.out_bf16 = out_dtype == CAKV_BF16;
    a.lse = lse;
    const Range enq("enqueue");
    s = hip_status(cakv::launch_decode_split(a, D, stream), "decode split launch");
    if (s != CAKV_OK) return s;
    return hip_status(cakv::launch_decode_merge(a, D, stream), "decode merge launch");
}

}  // namespace

extern "C" {

cakv_status cakv_decode(const void* q, const void* const* k_portions_host,
                        const void* const* v_portions_host, const int64_t* kv_len_host,
                        const int64_t* kv_off_host, int n_portions, int dtype, int B, int Hq,
                        int Hkv, int Tn, int D, int64_t q_off, int causal, float scale, void* out,
                        int out_dtype, float* lse, void* workspace, int64_t workspace_bytes,
                        void* stream) {
    const Range range("cakv_decode");
    DecodePlan p;
    bool empty = false;
    cakv_status s = decode_check(q, k_portions_host, v_portions_host, kv_len_host, kv_off_host,
                                 n_portions, dtype, B, Hq, Hkv, Tn, D, out, out_dtype, &p, &empty);
    if (s != CAKV_OK || empty) return s;
    if (!workspace) return fail(CAKV_ERR_NULL, "workspace is NULL");
    if (workspace_bytes < p.ws_bytes)
        return fail(CAKV_ERR_SHAPE, "workspace of %lld bytes, %lld needed",
                    (long long)workspace_bytes, p.ws_bytes);
    if (!aligned16(workspace)) return fail(CAKV_ERR_ALIGN, "workspace not 16-byte aligned");
    return decode_launch(q, k_portions_host, v_portions_host, kv_len_host, kv_off_host,
                         n_portions, B, Hq, Hkv, Tn, D, q_off, causal, scale, out, out_dtype, lse,
                         p, workspace, stream);
}

cakv_status cakv_decode_noalloc(const void* q, const void* const* k_portions_host,
                                const void* const* v_portions_host, const int64_t* kv_len_host,
                                const int64_t* kv_off_host, int n_portions, int dtype, int B,
                                int Hq, int Hkv, int Tn, int D, int64_t q_off, int causal,
                                float scale, void* out, int out_dtype, float* lse, void* stream) {
    const Range range("cakv_decode_noalloc");
    DecodePlan p;
    bool empty = false;
    cakv_status s = decode_check(q, k_portions_host, v_portions_host, kv_len_host, kv_off_host,
                                 n_portions, dtype, B, Hq, Hkv, Tn, D, out, out_dtype, &p, &empty);
    if (s != CAKV_OK || empty) return s;
    if (p.ws_bytes > (long long)CAKV_DECODE_SCRATCH_BYTES)
        return fail(CAKV_ERR_SHAPE,
                    "cakv_decode_noalloc: these sizes need %lld bytes of split state, above the "
                    "library's fixed %lld-byte scratch; use cakv_decode with a workspace",
                    p.ws_bytes, (long long)CAKV_DECODE_SCRATCH_BYTES);
    void* ws = nullptr;
    s = hip_status(cakv::decode_scratch_address(&ws), "decode scratch address");
    if (s != CAKV_OK) return s;
    return decode_launch(q, k_portions_host, v_portions_host, kv_len_host, kv_off_host,
                         n_portions, B, Hq, Hkv, Tn, D, q_off, causal, scale, out, out_dtype, lse,
                         p, ws, stream);
}

cakv_status cakv_diag_set_workgroup_order(int order) {
    if (order < 0 || order > 2) return fail(CAKV_ERR_RANGE, "workgroup order %d outside [0, 2]", order);
    g_wg_order.store(order, std::memory_order_relaxed);
    return ok();
}

cakv_status cakv_diag_mfma_burn(int zero_operands, int64_t iters, float* sink, void* stream) {
    if (iters < 0 || iters > 2147483647LL)
        return fail(CAKV_ERR_SHAPE, "iters=%lld outside [0, 2^31)", (long long)iters);
    if (iters == 0) return ok();
    if (!sink) return fail(CAKV_ERR_NULL, "sink is NULL");
    return hip_status(cakv::launch_mfma_burn(zero_operands != 0, (int)iters, sink, stream),
                      "mfma_burn launch");
}

}  // extern "C"
