// fwd_args.h -- argument block shared by the host launchers and the forward
// kernels of libcakv (internal; not part of the C ABI).
#pragma once

#include <stdint.h>

#include "cakv.h"
#include "wg_order.h"

namespace cakv {

// One launch folds n_blocks key/value blocks, in the order given, into the
// running (m, l, o) state of every local query row, then either stores the
// state (per-block call) or finalises it into out/lse (whole-shard call).
struct FwdArgs {
    const void* q;                        // [B, Tq, Hq, D]
    const void* k[CAKV_MAX_CHUNKS];       // block t: [B, kv_len[t], Hkv, D]
    const void* v[CAKV_MAX_CHUNKS];
    long long kv_off[CAKV_MAX_CHUNKS];    // global position of key 0 of block t
    int kv_len[CAKV_MAX_CHUNKS];
    int n_blocks;
    int B, Hq, Hkv, Tq;
    long long q_off;                      // global position of query row 0
    float scale_log2;                     // scale * log2(e)
    int causal;
    float* m;                             // [B, Hq, Tq] running state (natural units)
    float* l;                             // [B, Hq, Tq]
    float* o;                             // [B, Tq, Hq, D], unnormalised
    int load_state;                       // read m, l, o before the first block
    int store_state;                      // write m, l, o (else finalise to out/lse)
    void* out;                            // [B, Tq, Hq, D], fp32 or bf16
    int out_bf16;
    float* lse;                           // [B, Hq, Tq] or null
    unsigned long long* counters;         // [3] full / masked / skipped tiles, or null
    long long skip_tiles;                 // CAKV_TILE_K-key tiles of blocks dropped from the
                                          // list as SKIP, per 32-row tile (counters only)
    int wg_per_bg;                        // workgroups per (batch, kv head)
    int n_wg;                             // total workgroups (per key split)
    // key splits of a small grid (bf16 four-wave kernel, whole-shard calls):
    // n_split workgroups per query tile write partial states here, and a
    // merge kernel finalises them into out / lse; n_split = 1: no split
    int n_split;
    long long split_rows;                 // B * Hq * Tq
    float* split_m;                       // [n_split, rows] max, log2 units
    float* split_l;                       // [n_split, rows]
    float* split_o;                       // [n_split, rows, D] unnormalised
    int wg_order;                         // workgroup-order permutation (wg_order.h), 0 = none
    int wg_mul, wg_add;                   // set by the launcher for its grid
};

// Launchers (return the hipError_t of the launch as int).
int launch_fwd_bf16(const FwdArgs& a, int D, void* stream);
int launch_fwd_f32(const FwdArgs& a, int D, void* stream);
// waves per workgroup (32 query rows each) of the kernel that serves D, G =
// Hq / Hkv and `tasks` = B * Hq * ceil(Tq / 32) wave tasks
int fwd_bf16_waves(int D, int G, long long tasks);
int fwd_f32_wg_rows();

int launch_state_init(float* m, float* l, float* o, long long rows, int D, void* stream);
int launch_counter_add(unsigned long long* counter, unsigned long long value, void* stream);
int launch_mfma_burn(int zero, int iters, float* sink, void* stream);
int launch_finalize(const float* m, const float* l, const float* o, void* out, int out_bf16,
                    float* lse, int B, int Hq, int Tq, int D, void* stream);
int launch_lse_merge(const float* o_a, const float* lse_a, const float* o_b,
                     const float* lse_b, float* o_out, float* lse_out, int B, int Hq, int Tq,
                     int D, void* stream);

}  // namespace cakv
