/*
 * cakv.h -- C ABI of the local-shard ring attention library (libcakv.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes. Source: web page "Sequence parallelism -- splitting the
 * token dimension across GPUs" (llmdaily.org, day 58).
 *   - A sequence of T tokens is cut into N contiguous chunks of C = T/N
 *     tokens; rank r owns positions [r*C, (r+1)*C) (section "Split tokens
 *     across four GPUs"; positions here are 0-based).
 *   - Rank r keeps its queries in place while key/value blocks arrive one at
 *     a time (section "A better mental model: move blocks past the queries").
 *     On one GPU the blocks already sit in device memory and the "ring" is the
 *     order in which they are consumed: r, r-1, ..., wrapping modulo N.
 *   - Each query row computes softmax(q K^T / sqrt(d_k)) V (section
 *     "Attention wants keys and values from other tokens") without ever
 *     holding a full score row: a running max m, normaliser l and value
 *     accumulator o are rescaled and merged per block (section "But softmax
 *     seems to require all attention scores at once").
 *   - Under a causal mask a query sees keys at positions <= its own; blocks
 *     entirely in the future are skipped and only blocks straddling the
 *     diagonal are masked (section "Causal attention gives us another
 *     optimization").
 *   - Partial results over disjoint key sets are combined (section "Training
 *     and inference stress this dimension differently"); here by the
 *     log-sum-exp merge of normalised pairs (o, lse).
 *
 * Conventions for every call.
 *   - Pointers are DEVICE pointers owned by the caller unless marked "host".
 *     The library never allocates, frees or synchronises device memory; all
 *     device work is enqueued asynchronously on `stream` (a hipStream_t cast
 *     to void*, NULL = the default stream).
 *   - Layouts (row-major, innermost dimension last, contiguous):
 *       Q, out, o        [B, Tq, Hq, D]
 *       K, V (one block) [B, Tkv, Hkv, D]
 *       m, l, lse        [B, Hq, Tq]
 *     Query head h reads key/value head h / (Hq / Hkv).
 *   - Running state: m = running maximum of the scaled scores s = q.k*scale
 *     (natural units), l = sum of e^{s - m}, o = sum of e^{s - m} v (NOT
 *     normalised). A row that has seen no allowed key has m = -inf, l = 0,
 *     o = 0. Finalised results: out = o / l, lse = m + ln(l); a row with
 *     l = 0 finalises to out = 0, lse = -inf.
 *   - dtype: CAKV_BF16 inputs are multiplied on bf16 matrix cores with fp32
 *     accumulation (probabilities are rounded to bf16 before P*V); CAKV_F32
 *     inputs are computed in fp32 throughout. State, lse and merge operands
 *     are always fp32.
 *   - scale <= 0 selects 1/sqrt(D).
 *   - Supported: D in {64, 128}; Hq % Hkv == 0; Hq * D <= 2^24 (the
 *     kernels address a tile's rows in 32 bits); 16-byte aligned pointers;
 *     sizes >= 0 (an empty problem returns CAKV_OK and launches nothing).
 *   - Errors: arguments are checked before anything is enqueued; on an error
 *     nothing is launched, outputs are untouched, the status is returned and
 *     cakv_last_error() describes it. A failed kernel launch returns
 *     CAKV_ERR_HIP. Faults inside kernels surface at the caller's next
 *     synchronisation. No C++ exception crosses this interface.
 *   - Thread safety: the library keeps no state besides the thread-local
 *     error message; calls on different streams are independent. Calls that
 *     write the same buffers must be ordered by the caller.
 */
#ifndef CAKV_H
#define CAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CAKV_ABI_VERSION 2 /* 2: tile_counters holds three counts */
#define CAKV_MAX_CHUNKS 64 /* most key/value blocks one forward call takes */
#define CAKV_TILE_Q 32     /* query rows per counted tile */
#define CAKV_TILE_K 64     /* keys per counted tile */
/* bytes of the per-GPU scratch array behind cakv_decode_noalloc (32 MiB) */
#define CAKV_DECODE_SCRATCH_BYTES (32LL << 20)

typedef enum {
    CAKV_OK = 0,
    CAKV_ERR_NULL = 1,     /* a required pointer is NULL */
    CAKV_ERR_SHAPE = 2,    /* negative size, unsupported D, Hq % Hkv != 0, ... */
    CAKV_ERR_DTYPE = 3,    /* unknown dtype */
    CAKV_ERR_ALIGN = 4,    /* pointer not 16-byte aligned */
    CAKV_ERR_RANGE = 5,    /* rank / chunk count / offset out of range */
    CAKV_ERR_HIP = 6,      /* the HIP runtime reported an error */
    CAKV_ERR_INTERNAL = 7
} cakv_status;

typedef enum { CAKV_F32 = 0, CAKV_BF16 = 1 } cakv_dtype;

/* class of a key/value block (or tile) relative to a query range */
typedef enum {
    CAKV_FULL = 0, /* every (query, key) pair is allowed: no mask */
    CAKV_DIAG = 1, /* some pairs allowed: masked from global positions */
    CAKV_SKIP = 2  /* no pair allowed (or nothing to pair): never read */
} cakv_class;

/* CAKV_ABI_VERSION of the loaded library. */
int cakv_abi_version(void);

/* Static text for a status code (never NULL). */
const char* cakv_status_str(int status);

/* Detail of the last error on this thread ("" if none). Valid until the next
 * call from the same thread. */
const char* cakv_last_error(void);

/*
 * Class of one block: keys at global positions [kv_offset, kv_offset+kv_len)
 * against queries at [q_offset, q_offset+q_len). Causal: SKIP if the first
 * key is after the last query (or either range is empty), FULL if the last
 * key is at or before the first query, else DIAG. Bidirectional: FULL unless
 * empty. Host only, pure. Page section "Causal attention gives us another
 * optimization".
 */
cakv_status cakv_classify_block(int64_t q_offset, int64_t q_len, int64_t kv_offset,
                                int64_t kv_len, int causal, int8_t* class_host);

/*
 * Ring schedule of rank `rank` of `n_chunks` equal chunks of `chunk_len`
 * tokens: blocks_host[k] = (rank - k) mod n_chunks for k = 0..n_chunks-1 (the
 * order the blocks pass the rank's stationary queries, page section "A better
 * mental model: move blocks past the queries") and class_host[k] = class of
 * that block for the rank's queries (cakv_classify_block). Host arrays of
 * n_chunks entries, written by the call. Host only, pure.
 * Errors: NULL arrays, n_chunks outside [1, CAKV_MAX_CHUNKS], rank outside
 * [0, n_chunks), chunk_len < 0.
 */
cakv_status cakv_schedule(int rank, int n_chunks, int64_t chunk_len, int causal,
                          int32_t* blocks_host, int8_t* class_host);

/*
 * Empty running state for B*Hq*Tq rows: m = -inf, l = 0, o = 0, the state
 * before the first block of the running update of page section "But softmax
 * seems to require all attention scores at once" (the page leaves the
 * starting values implicit; these are the ones for which folding the first
 * block gives that block's own m, l, o).
 * m, l: [B, Hq, Tq] fp32; o: [B, Tq, Hq, D] fp32, 16-byte aligned.
 * Errors: negative sizes, D not 64 or 128 (CAKV_ERR_SHAPE); NULL state
 * pointers (CAKV_ERR_NULL) or a misaligned o (CAKV_ERR_ALIGN) when there is
 * at least one row. Zero rows returns CAKV_OK and launches nothing.
 */
cakv_status cakv_state_init(float* m, float* l, float* o, int B, int Hq, int Tq, int D,
                            void* stream);

/*
 * One ring step: fold one key/value block into the running state (page
 * section "But softmax seems to require all attention scores at once").
 * q: [B, Tq, Hq, D] queries at global positions q_offset + row;
 * k, v: [B, Tkv, Hkv, D] keys/values at global positions kv_offset + row;
 * dtype: CAKV_BF16 or CAKV_F32 (q, k, v share it); scale <= 0 -> 1/sqrt(D).
 * m, l, o: running state, read and written in place.
 * tile_counters (nullable, device int64[3]): the call ADDS the number of
 * (CAKV_TILE_Q rows x CAKV_TILE_K keys) tiles of the block's grid, summed
 * over batch rows and query heads, that it computed unmasked [0], computed
 * masked [1] and skipped [2] (no allowed pair: never read); the three add up
 * to the whole grid (page section "Causal attention gives us another
 * optimization": fully masked work is not done, only the diagonal is
 * masked). A block with no allowed pair (CAKV_SKIP) returns CAKV_OK and
 * launches nothing, or, when counters are given, only a one-thread kernel
 * that adds its tiles to [2].
 */
cakv_status cakv_block_update(const void* q, const void* k, const void* v, int dtype,
                              int B, int Hq, int Hkv, int Tq, int Tkv, int D,
                              int64_t q_offset, int64_t kv_offset, int causal, float scale,
                              float* m, float* l, float* o, int64_t* tile_counters,
                              void* stream);

/*
 * out = o / l (fp32, or bf16 if out_dtype == CAKV_BF16) and lse = m + ln(l)
 * (fp32); rows with l == 0 give out = 0, lse = -inf. Page section "But
 * softmax seems to require all attention scores at once": o holds the
 * e^{s - m}-weighted sum of values and l the sum of the weights, so the
 * softmax output is their ratio (the page stops before this division; it is
 * the plain reading of an unnormalised accumulator), and m + ln(l) is the
 * log of the row's whole softmax denominator, the quantity partial results
 * are combined by. m, l: [B, Hq, Tq]; o, out: [B, Tq, Hq, D], 16-byte
 * aligned; out may alias o when out_dtype is CAKV_F32. lse may be NULL.
 * Errors: unknown out_dtype (CAKV_ERR_DTYPE); sizes as cakv_state_init;
 * NULL m, l, o or out (CAKV_ERR_NULL); misaligned o / out (CAKV_ERR_ALIGN).
 */
cakv_status cakv_finalize(const float* m, const float* l, const float* o, void* out,
                          int out_dtype, float* lse, int B, int Hq, int Tq, int D,
                          void* stream);

/*
 * Combine two normalised partials of the same rows over disjoint key sets:
 *   M = max(lse_a, lse_b), lse = M + ln(e^{lse_a-M} + e^{lse_b-M}),
 *   o = e^{lse_a-lse} o_a + e^{lse_b-lse} o_b; both -inf gives (0, -inf).
 * o_*: [B, Tq, Hq, D] fp32; lse_*: [B, Hq, Tq] fp32. o_out / lse_out may
 * alias either input. Page section "Training and inference stress this
 * dimension differently" (partial results are combined), with the rescale
 * rule of section "But softmax seems to require all attention scores at
 * once".
 */
cakv_status cakv_lse_merge(const float* o_a, const float* lse_a, const float* o_b,
                           const float* lse_b, float* o_out, float* lse_out, int B, int Hq,
                           int Tq, int D, void* stream);

/*
 * One rank's whole share: attention of the stationary local queries q_local
 * (chunk `rank`, global positions rank*chunk_len + row; page section "Split
 * tokens across four GPUs") against the n_chunks key/value blocks, consumed
 * in ring order rank, rank-1, ... (cakv_schedule; page section "A better
 * mental model: move blocks past the queries"), each folded by the running
 * update of section "But softmax seems to require all attention scores at
 * once", SKIP blocks never read and only DIAG tiles masked (section "Causal
 * attention gives us another optimization"), then finalised as
 * cakv_finalize. The running state stays on chip for the whole ring; nothing
 * but out and lse is written.
 * q_local: [B, chunk_len, Hq, D];
 * k_blocks_host, v_blocks_host: HOST arrays of n_chunks device pointers,
 *   block j = [B, chunk_len, Hkv, D] holding positions [j*chunk_len, ...);
 * out: [B, chunk_len, Hq, D] in out_dtype; lse: [B, Hq, chunk_len] fp32
 *   (nullable);
 * workspace (nullable), workspace_bytes: device scratch owned by the caller,
 *   16-byte aligned. When the share is too small to fill the GPU (few query
 *   rows; bf16 with one query head per key/value head or d_k = 64) and the
 *   workspace holds cakv_forward_workspace_size bytes, each query tile's key
 *   range is cut into parts folded side by side, whose partial states are
 *   combined by the log-sum-exp rule (page section "Training and inference
 *   stress this dimension differently": partial results over key portions
 *   combine). Otherwise, or with NULL, the running state stays on chip for
 *   the whole ring. Both give the same result up to fp32 rounding order;
 *   calls sharing a workspace must not overlap in time;
 * tile_counters: as for cakv_block_update, over the grids of all n_chunks
 *   blocks (nullable).
 * Errors: as above plus rank outside [0, n_chunks), n_chunks outside
 * [1, CAKV_MAX_CHUNKS], a NULL block pointer that the schedule would read.
 */
cakv_status cakv_local_shard_forward(const void* q_local, const void* const* k_blocks_host,
                                     const void* const* v_blocks_host, int dtype, int B,
                                     int Hq, int Hkv, int chunk_len, int n_chunks, int D,
                                     int rank, int causal, float scale, void* out,
                                     int out_dtype, float* lse, void* workspace,
                                     int64_t workspace_bytes, int64_t* tile_counters,
                                     void* stream);

/*
 * The general form of cakv_local_shard_forward: Tq queries at global
 * positions q_offset + row against n_blocks key/value blocks of any lengths
 * at any global offsets, folded in the order given with the running state
 * on chip, then finalised. It covers the cases the ring of equal chunks does
 * not: unequal chunks, keys and values appended across turns, blocks that
 * straddle the query range (page sections "Causal attention gives us
 * another optimization" for the per-position rule and "Training and
 * inference stress this dimension differently" for a KV history that grows).
 * Blocks whose keys all lie after every query (causal) are never read; a
 * block straddling a query's position is masked per tile.
 * q: [B, Tq, Hq, D]; k_blocks_host, v_blocks_host: HOST arrays of n_blocks
 *   device pointers, block t = [B, kv_len_host[t], Hkv, D] with key 0 at
 *   global position kv_off_host[t] (HOST int64 arrays; an empty block's
 *   pointers may be NULL);
 * out, lse, workspace, workspace_bytes, tile_counters, dtype, scale: as for
 *   cakv_local_shard_forward (the workspace size query takes Tq).
 * Errors: as for cakv_block_update, plus n_blocks outside
 * [1, CAKV_MAX_CHUNKS], a block length outside [0, 2^31 - 1], a NULL block
 * pointer that would be read.
 */
cakv_status cakv_forward_blocks(const void* q, const void* const* k_blocks_host,
                                const void* const* v_blocks_host, const int64_t* kv_len_host,
                                const int64_t* kv_off_host, int n_blocks, int dtype, int B,
                                int Hq, int Hkv, int Tq, int D, int64_t q_offset, int causal,
                                float scale, void* out, int out_dtype, float* lse,
                                void* workspace, int64_t workspace_bytes,
                                int64_t* tile_counters, void* stream);

/*
 * Bytes of workspace that lets cakv_local_shard_forward (Tq = chunk_len) or
 * cakv_forward_blocks split the key range of a small share (written to the
 * HOST int64 *bytes_host); 0 when the share fills the GPU without splitting.
 * Errors: NULL bytes_host, and the size and dtype checks of
 * cakv_block_update.
 */
cakv_status cakv_forward_workspace_size(int dtype, int B, int Hq, int Hkv, int Tq, int D,
                                        int64_t* bytes_host);

/*
 * Gradients of cakv_forward_blocks for training (the pages apply sequence
 * parallelism to training as well as inference, section "Training and
 * inference stress this dimension differently", but give no backward
 * formulas): the chain rule through the definition of section "Attention
 * wants keys and values from other tokens", with p = e^{s - lse}
 * recomputed from the forward's lse:
 *   delta_i = dout_i . out_i,  ds_ij = p_ij (dout_i . v_j - delta_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 *   dv_j = sum_i p_ij dout_i   (grouped query heads add into their kv head).
 * q, k_blocks, v_blocks, kv_len, kv_off, q_offset, causal, scale: exactly as
 *   given to the forward (bf16 only);
 * out: [B, Tq, Hq, D] fp32 and lse: [B, Hq, Tq] fp32 from that forward;
 * dout: [B, Tq, Hq, D] bf16, the gradient of the loss with respect to out;
 * dq: [B, Tq, Hq, D] fp32; dk_blocks_host, dv_blocks_host: HOST arrays of
 *   device pointers, block t = [B, kv_len_host[t], Hkv, D] fp32. All outputs
 *   are overwritten (a block no query sees gets zeros).
 * workspace: device buffer of cakv_backward_workspace_size bytes (per
 *   row: -delta = -dout . out and -lse / scale), 16-byte aligned,
 *   owned by the caller.
 * Errors: CAKV_ERR_DTYPE unless dtype = CAKV_BF16; otherwise as for
 * cakv_forward_blocks, plus NULL out / lse / dout / dq / gradient block
 * pointers and a too small workspace (CAKV_ERR_SHAPE).
 */
cakv_status cakv_backward_blocks(const void* q, const void* const* k_blocks_host,
                                 const void* const* v_blocks_host, const int64_t* kv_len_host,
                                 const int64_t* kv_off_host, int n_blocks, int dtype, int B,
                                 int Hq, int Hkv, int Tq, int D, int64_t q_offset, int causal,
                                 float scale, const float* out, const float* lse,
                                 const void* dout, float* dq, float* const* dk_blocks_host,
                                 float* const* dv_blocks_host, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* Bytes of workspace cakv_backward_blocks needs (B * Hq * Tq * 8), written
 * to the HOST int64 *bytes_host. */
cakv_status cakv_backward_workspace_size(int B, int Hq, int Tq, int64_t* bytes_host);

/*
 * Decode over a KV history held in portions (page section "Training and
 * inference stress this dimension differently": during inference each device
 * holds one portion of a long conversation's keys and values, the new query
 * is evaluated against every portion and the partial attention results are
 * combined). On one GPU the portions are device buffers; the call reads each
 * once, cut into many splits processed side by side, and merges the splits'
 * online-softmax states with the log-sum-exp rule (the rescale rule of
 * section "But softmax seems to require all attention scores at once").
 * Called with one portion it yields that portion's normalised partial
 * (out_j, lse_j); cakv_lse_merge combines such partials of disjoint portions.
 *
 * q: [B, Tn, Hq, D] bf16, the Tn new queries at global positions
 *   q_off .. q_off + Tn - 1;
 * k_portions_host, v_portions_host: HOST arrays of n_portions device
 *   pointers, portion j = [B, kv_len_host[j], Hkv, D] bf16 whose key 0 sits at
 *   global position kv_off_host[j] (HOST int64 arrays); portions may come in
 *   any order and need not be adjacent; an empty portion's pointers may be
 *   NULL. causal != 0 hides keys at positions after a query's own (the new
 *   tokens' keys may be part of the last portion); every history key before
 *   q_off is visible either way.
 * out: [B, Tn, Hq, D] in out_dtype; lse: [B, Hq, Tn] fp32 natural log
 *   (nullable). A row that sees no key gets out = 0, lse = -inf.
 * workspace: device buffer of at least cakv_decode_workspace_size bytes for
 *   the splits' states, 16-byte aligned, owned by the caller; its contents
 *   are scratch. Calls that share a workspace must not overlap in time.
 * Errors: CAKV_ERR_DTYPE unless dtype = CAKV_BF16 (fp32 decode is not
 * provided) or for an unknown out_dtype; CAKV_ERR_SHAPE for sizes as in
 * cakv_block_update, a portion length outside [0, 2^31 - 64] or a workspace
 * that is too small; CAKV_ERR_RANGE for n_portions outside
 * [1, CAKV_MAX_CHUNKS]; CAKV_ERR_NULL / CAKV_ERR_ALIGN as usual. B = 0 or
 * Tn = 0 returns CAKV_OK and launches nothing.
 */
cakv_status cakv_decode(const void* q, const void* const* k_portions_host,
                        const void* const* v_portions_host, const int64_t* kv_len_host,
                        const int64_t* kv_off_host, int n_portions, int dtype, int B, int Hq,
                        int Hkv, int Tn, int D, int64_t q_off, int causal, float scale, void* out,
                        int out_dtype, float* lse, void* workspace, int64_t workspace_bytes,
                        void* stream);

/*
 * cakv_decode without a workspace argument, for callers that cannot allocate
 * device memory: code recorded under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The splits' states go to a scratch array
 * of CAKV_DECODE_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU, for the life of the process; the call itself allocates and frees
 * nothing (its first call on a GPU looks up that GPU's array address). All
 * arguments, results and errors are those of cakv_decode, plus
 * CAKV_ERR_SHAPE, before anything is launched, when the sizes need more
 * split state than the array holds (cakv_decode_workspace_size > 32 MiB;
 * the million-token history with up to 16 new tokens needs ~25.6 MB).
 * Nothing in the array needs clearing: every entry a call reads was written
 * earlier in the same call. Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams, or threads)
 * race and must be ordered by the caller.
 */
cakv_status cakv_decode_noalloc(const void* q, const void* const* k_portions_host,
                                const void* const* v_portions_host, const int64_t* kv_len_host,
                                const int64_t* kv_off_host, int n_portions, int dtype, int B,
                                int Hq, int Hkv, int Tn, int D, int64_t q_off, int causal,
                                float scale, void* out, int out_dtype, float* lse, void* stream);

/*
 * Bytes of workspace cakv_decode needs for these sizes (written to the HOST
 * int64 *bytes_host; 0 when B or Tn is 0). Same argument checks as
 * cakv_decode.
 */
cakv_status cakv_decode_workspace_size(int B, int Hq, int Hkv, int Tn, int D,
                                       const int64_t* kv_len_host, int n_portions,
                                       int64_t* bytes_host);

#ifdef __cplusplus
}
#endif

#endif /* CAKV_H */
