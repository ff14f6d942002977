// bwd_args.h -- argument block of the backward kernels of libcakv (internal;
// not part of the C ABI).
#pragma once

#include <stdint.h>

#include "cakv.h"
#include "wg_order.h"

namespace cakv {

constexpr int kBwdKeyTile = 256;   // keys per dK/dV workgroup (32 per wave, 8 waves)

// Gradients of the attention of Tq queries (global positions q_off + row)
// against n_blocks key/value blocks, from the forward's out and lse.
struct BwdArgs {
    const void* q;                          // [B, Tq, Hq, D] bf16
    const void* dout;                       // [B, Tq, Hq, D] bf16
    const float* out;                       // [B, Tq, Hq, D] fp32 (forward output)
    const float* lse;                       // [B, Hq, Tq] fp32 (forward lse, natural log)
    const void* k[CAKV_MAX_CHUNKS];         // block t: [B, kv_len[t], Hkv, D] bf16
    const void* v[CAKV_MAX_CHUNKS];
    float* dk[CAKV_MAX_CHUNKS];             // block t: [B, kv_len[t], Hkv, D] fp32
    float* dv[CAKV_MAX_CHUNKS];
    long long kv_off[CAKV_MAX_CHUNKS];
    int kv_len[CAKV_MAX_CHUNKS];
    int kt0[CAKV_MAX_CHUNKS + 1];           // first kBwdKeyTile-key tile of block t; kt0[n] = total
    int n_blocks;
    int B, Hq, Hkv, Tq;
    long long q_off;
    float scale;                            // score scale
    float scale_log2;                       // scale * log2(e)
    int causal;
    float* ndelta;                          // [B, Hq, Tq] workspace: -rowsum(dout * out)
    float* nlse;                            // [B, Hq, Tq] workspace: -lse / scale, -inf for a row without keys
    float* dq;                              // [B, Tq, Hq, D] fp32
    int wg_per_bg;                          // dq kernel: workgroups per (batch, kv head)
    int wg_order;                           // workgroup-order permutation (wg_order.h), 0 = none
    int wg_mul, wg_add;                     // set by the launcher for each grid
};

int launch_bwd(const BwdArgs& a, int D, void* stream);

}  // namespace cakv
