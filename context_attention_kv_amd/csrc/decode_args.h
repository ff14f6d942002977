// decode_args.h -- argument block of the decode kernels of libcakv (internal;
// not part of the C ABI).
#pragma once

#include <stdint.h>

#include "cakv.h"
#include "wg_order.h"

namespace cakv {

constexpr int kDecTile = 32;   // keys per decode tile

// New query rows against key/value history portions, split over many waves.
// The tiles of all portions (32 keys each, a portion's last tile possibly
// short) are numbered portion by portion; split s covers tiles
// [s * tiles_per_split, (s + 1) * tiles_per_split). Wave (s, b, g, rb) folds
// those tiles into an online-softmax state for row block rb (32 rows) of kv
// head g of batch b and writes it to the workspace (a workgroup holds the
// waves of decode_heads_per_wg neighbouring kv heads); the merge kernel then
// combines the splits of every row.
struct DecArgs {
    const void* q;                          // [B, Tn, Hq, D] bf16
    const void* k[CAKV_MAX_CHUNKS];         // portion j: [B, kv_len[j], Hkv, D] bf16
    const void* v[CAKV_MAX_CHUNKS];
    long long kv_off[CAKV_MAX_CHUNKS];      // global position of key 0 of portion j
    int kv_len[CAKV_MAX_CHUNKS];
    int tile0[CAKV_MAX_CHUNKS + 1];         // first tile number of portion j; tile0[n] = total
    int n_portions;
    int B, Hq, Hkv, Tn;
    long long q_off;                        // global position of new query 0
    float scale_log2;                       // scale * log2(e)
    int causal;
    int nrb;                                // 32-row blocks per (batch, kv head)
    int tiles_per_split;
    int n_splits;
    float* ws_m;                            // [S, B, Hkv, nrb*32] running max (log2 units)
    float* ws_l;                            // [S, B, Hkv, nrb*32] normaliser
    float* ws_o;                            // [S, B, Hkv, nrb*32, D] unnormalised output
    void* out;                              // [B, Tn, Hq, D] fp32 or bf16
    int out_bf16;
    float* lse;                             // [B, Hq, Tn] or null
    int wg_order;                           // workgroup-order permutation (wg_order.h), 0 = none
    int wg_mul, wg_add;                     // set by the launcher for the split grid
};

// Device address of this device's decode scratch array
// (CAKV_DECODE_SCRATCH_BYTES); resolved on the first call on each device
// (the device current at the call), then cached. Returns a hipError_t as int.
int decode_scratch_address(void** ptr);

// kv heads per workgroup of the split kernel (one wave each) for Hkv heads
inline int decode_heads_per_wg(int Hkv) { return Hkv % 4 == 0 ? 4 : (Hkv % 2 == 0 ? 2 : 1); }
int launch_decode_split(const DecArgs& a, int D, void* stream);
int launch_decode_merge(const DecArgs& a, int D, void* stream);

}  // namespace cakv
