/*
 * oracle.c -- plain, slow, fp64 CPU oracle for one rank's ring (context-
 * parallel) attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark may use it. It shares no code, header, table or helper
 * with the HIP path.
 *
 * Source: web page "Sequence parallelism -- splitting the token dimension
 * across GPUs" (llmdaily.org, day 58). Sections used:
 *   [ATTN]   "Attention wants keys and values from other tokens":
 *            Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V, and a causal
 *            token attends to every earlier token and to itself.
 *   [SMAX]   "But softmax seems to require all attention scores at once":
 *            p_i = e^{s_i} / sum_j e^{s_j}; running max m, normaliser l and
 *            value accumulator o; on a block with max m', m_new = max(m, m'),
 *            old terms rescaled by e^{m - m_new}, new ones by e^{m' - m_new}.
 *   [CAUSAL] "Causal attention gives us another optimization": the lower-
 *            triangular pattern and the blocks each GPU does / does not need.
 *   [RING]   "A better mental model: move blocks past the queries": queries
 *            stay, key/value blocks arrive one per round.
 *   [INFER]  "Training and inference stress this dimension differently":
 *            partial attention results over KV portions can be combined.
 *
 * Readings where the page is silent (all listed again in the design notes):
 *   - positions are 0-based; key j is allowed for query position p iff the
 *     attention is bidirectional or j <= p (diagonal allowed: [ATTN]);
 *   - a row with no allowed key has out = 0 and lse = -inf (empty sum);
 *   - lse = m + ln(l), natural log; o before finalisation is unnormalised;
 *   - combining two normalised partials (o_a, lse_a), (o_b, lse_b) is the
 *     [SMAX] rescale rule written for normalised pairs (log-sum-exp merge).
 *
 * Layouts (row-major, innermost last): Q [B, Tq, Hq, D]; K, V [B, Tk, Hkv, D];
 * outputs per requested row. Query head h reads key/value head h / (Hq/Hkv).
 * Inputs are either fp32 or bf16 bit patterns (uint16, upper half of an
 * IEEE fp32); every value is widened exactly to double before use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* exact widening of one stored input element to double */
static double load_elem(const void* base, int is_bf16, int64_t idx) {
    if (is_bf16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[idx];
}

static int64_t qk_index(int64_t b, int64_t t, int64_t h, int64_t c,
                        int64_t T, int64_t H, int64_t D) {
    return ((b * T + t) * H + h) * D + c;
}

/* score s_j = (q . k_j) / sqrt(d_k) in fp64, as in [ATTN] (scale passed in) */
static double score(const void* q, int q_bf16, const void* k, int kv_bf16,
                    int64_t b, int64_t i, int64_t h, int64_t j, int64_t g,
                    int64_t Tq, int64_t Hq, int64_t Tk, int64_t Hkv, int64_t D,
                    double scale) {
    double acc = 0.0;
    for (int64_t c = 0; c < D; ++c)
        acc += load_elem(q, q_bf16, qk_index(b, i, h, c, Tq, Hq, D)) *
               load_elem(k, kv_bf16, qk_index(b, j, g, c, Tk, Hkv, D));
    return acc * scale;
}

static int allowed(int causal, int64_t key_pos, int64_t query_pos) {
    return !causal || key_pos <= query_pos;
}

/*
 * O1: the plain definition. For each requested row (b, h, i) with global
 * query position q_off + i, every key j of [0, Tk) at global position
 * k_off + j that the mask allows takes part in
 *   out = sum_j e^{s_j - M} v_j / Z,  Z = sum_j e^{s_j - M},  M = max_j s_j,
 *   lse = M + ln Z.
 * Subtracting M changes nothing in exact arithmetic ([ATTN] softmax with the
 * [SMAX] maximum used for stability). weights (nullable) receives the
 * softmax weights p_j of each row over all Tk keys (0 where masked).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attention_rows(const void* q, int q_bf16, const void* k,
                          const void* v, int kv_bf16, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t Tq, int64_t Tk, int64_t D,
                          int64_t q_off, int64_t k_off, int causal,
                          double scale, int64_t n_rows, const int64_t* rows,
                          double* out, double* lse, double* weights) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Tq < 0 || Tk < 0 ||
        D <= 0 || n_rows < 0)
        return -1;
    const int64_t group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Tq) {
            bad = 1;
            continue;
        }
        const int64_t g = h / group;
        const int64_t qpos = q_off + i;
        double* s = (double*)malloc(sizeof(double) * (size_t)(Tk > 0 ? Tk : 1));
        double M = -INFINITY;
        for (int64_t j = 0; j < Tk; ++j) {
            if (allowed(causal, k_off + j, qpos)) {
                s[j] = score(q, q_bf16, k, kv_bf16, b, i, h, j, g, Tq, Hq, Tk,
                             Hkv, D, scale);
                if (s[j] > M) M = s[j];
            }
        }
        double* o = out + r * D;
        for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
        double Z = 0.0;
        if (M > -INFINITY) {
            for (int64_t j = 0; j < Tk; ++j) {
                if (!allowed(causal, k_off + j, qpos)) continue;
                const double e = exp(s[j] - M);
                Z += e;
                for (int64_t c = 0; c < D; ++c)
                    o[c] += e * load_elem(v, kv_bf16, qk_index(b, j, g, c, Tk, Hkv, D));
            }
            for (int64_t c = 0; c < D; ++c) o[c] /= Z;
            lse[r] = M + log(Z);
        } else {
            lse[r] = -INFINITY;
        }
        if (weights) {
            double* w = weights + r * Tk;
            for (int64_t j = 0; j < Tk; ++j)
                w[j] = (M > -INFINITY && allowed(causal, k_off + j, qpos))
                           ? exp(s[j] - M) / Z
                           : 0.0;
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * O2: the page's own algorithm, used only to cross-check O1. Key/value
 * blocks arrive one at a time ([RING]) in the given order; for each block
 * the row keeps (m, l, o) and applies the [SMAX] update literally:
 *   m' = max of the block's allowed scores, l' = sum e^{s - m'},
 *   o' = sum e^{s - m'} v;  m_new = max(m, m');
 *   l = l e^{m - m_new} + l' e^{m' - m_new}; o likewise.
 * A block with no allowed key for the row leaves the state unchanged. The
 * initial state is m = -inf, l = 0, o = 0 (the page implies an empty start).
 * K/V are one array [B, Tk, Hkv, D] over all positions; block t covers keys
 * [starts[t], starts[t] + lens[t]) at global positions k_off + key index.
 * Outputs: finalised out = o / l, lse = m + ln l (0 and -inf when l = 0), and
 * (nullable) the raw state m, l, o after the last block.
 */
int oracle_online_blockwise(const void* q, int q_bf16, const void* k,
                            const void* v, int kv_bf16, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Tq, int64_t Tk, int64_t D,
                            int64_t q_off, int64_t k_off, int causal,
                            double scale, int64_t n_blocks,
                            const int64_t* starts, const int64_t* lens,
                            const int64_t* order, int64_t n_rows,
                            const int64_t* rows, double* out, double* lse,
                            double* m_state, double* l_state, double* o_state) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Tq < 0 || Tk < 0 ||
        D <= 0 || n_rows < 0 || n_blocks < 0)
        return -1;
    for (int64_t t = 0; t < n_blocks; ++t) {
        const int64_t blk = order[t];
        if (blk < 0 || blk >= n_blocks || starts[blk] < 0 || lens[blk] < 0 ||
            starts[blk] + lens[blk] > Tk)
            return -1;
    }
    const int64_t group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Tq) {
            bad = 1;
            continue;
        }
        const int64_t g = h / group;
        const int64_t qpos = q_off + i;
        double m = -INFINITY, l = 0.0;
        double* o = (double*)calloc((size_t)D, sizeof(double));
        double* ob = (double*)malloc(sizeof(double) * (size_t)D);
        for (int64_t t = 0; t < n_blocks; ++t) {
            const int64_t blk = order[t];
            const int64_t j0 = starts[blk], j1 = starts[blk] + lens[blk];
            /* block maximum m' over the allowed scores */
            double mb = -INFINITY;
            for (int64_t j = j0; j < j1; ++j)
                if (allowed(causal, k_off + j, qpos)) {
                    double s = score(q, q_bf16, k, kv_bf16, b, i, h, j, g, Tq,
                                     Hq, Tk, Hkv, D, scale);
                    if (s > mb) mb = s;
                }
            if (mb == -INFINITY) continue; /* nothing allowed in this block */
            double lb = 0.0;
            for (int64_t c = 0; c < D; ++c) ob[c] = 0.0;
            for (int64_t j = j0; j < j1; ++j) {
                if (!allowed(causal, k_off + j, qpos)) continue;
                double s = score(q, q_bf16, k, kv_bf16, b, i, h, j, g, Tq, Hq,
                                 Tk, Hkv, D, scale);
                double e = exp(s - mb);
                lb += e;
                for (int64_t c = 0; c < D; ++c)
                    ob[c] += e * load_elem(v, kv_bf16, qk_index(b, j, g, c, Tk, Hkv, D));
            }
            const double m_new = m > mb ? m : mb;
            const double a_old = (m == -INFINITY) ? 0.0 : exp(m - m_new);
            const double a_new = exp(mb - m_new);
            l = l * a_old + lb * a_new;
            for (int64_t c = 0; c < D; ++c) o[c] = o[c] * a_old + ob[c] * a_new;
            m = m_new;
        }
        for (int64_t c = 0; c < D; ++c) out[r * D + c] = l > 0.0 ? o[c] / l : 0.0;
        lse[r] = l > 0.0 ? m + log(l) : -INFINITY;
        if (m_state) m_state[r] = m;
        if (l_state) l_state[r] = l;
        if (o_state)
            for (int64_t c = 0; c < D; ++c) o_state[r * D + c] = o[c];
        free(o);
        free(ob);
    }
    return bad ? -1 : 0;
}

/*
 * O3: brute-force schedule classification. For each key/value block t
 * (keys [starts[t], starts[t]+lens[t]), positions k_off + index) and the
 * query range [q_off, q_off + Tq) this counts the allowed (query, key) pairs
 * one by one ([CAUSAL]: a query never sees a later key) and classes the
 * block: 2 = SKIP (no pair allowed, or no pair at all), 0 = FULL (every pair
 * allowed), 1 = DIAG (some pairs). pairs_out (nullable) receives the count.
 * The same count is made for every tile of tile_q consecutive query rows by
 * tile_k consecutive keys of a block (rows from 0, keys from the block's
 * first key, the last tile of each clipped to what exists); tile_counts[3]
 * receives the number of FULL, partially masked and SKIP tiles, multiplied
 * by B * Hq (every batch row and query head has the same pattern).
 */
int oracle_classify(int64_t Tq, int64_t q_off, int64_t k_off, int causal,
                    int64_t n_blocks, const int64_t* starts,
                    const int64_t* lens, int64_t B, int64_t Hq,
                    int64_t tile_q, int64_t tile_k, int8_t* block_class,
                    int64_t* pairs_out, int64_t* tile_counts) {
    if (Tq < 0 || n_blocks < 0 || B < 0 || Hq < 0 || tile_q <= 0 || tile_k <= 0)
        return -1;
    int64_t tc[3] = {0, 0, 0};
    for (int64_t t = 0; t < n_blocks; ++t) {
        /* every pair is counted once, inside its tile; the block's count is
           the sum over its tiles (row tiles spread over threads) */
        int64_t pairs = 0, n_full = 0, n_part = 0, n_skip = 0;
        const int64_t n_row_tiles = (Tq + tile_q - 1) / tile_q;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : pairs, n_full, n_part, n_skip)
        for (int64_t it = 0; it < n_row_tiles; ++it) {
            const int64_t i0 = it * tile_q;
            const int64_t i1 = i0 + tile_q < Tq ? i0 + tile_q : Tq;
            for (int64_t j0 = 0; j0 < lens[t]; j0 += tile_k) {
                const int64_t j1 = j0 + tile_k < lens[t] ? j0 + tile_k : lens[t];
                int64_t p = 0;
                for (int64_t i = i0; i < i1; ++i)
                    for (int64_t j = j0; j < j1; ++j)
                        p += allowed(causal, k_off + starts[t] + j, q_off + i);
                pairs += p;
                if (p == 0) ++n_skip;
                else if (p == (i1 - i0) * (j1 - j0)) ++n_full;
                else ++n_part;
            }
        }
        const int64_t total = Tq * lens[t];
        if (block_class)
            block_class[t] = (pairs == 0) ? 2 : (pairs == total ? 0 : 1);
        if (pairs_out) pairs_out[t] = pairs;
        tc[0] += n_full;
        tc[1] += n_part;
        tc[2] += n_skip;
    }
    if (tile_counts)
        for (int c = 0; c < 3; ++c) tile_counts[c] = tc[c] * B * Hq;
    return 0;
}

/*
 * Combine two normalised partial results of the same rows over disjoint key
 * sets ([INFER] says they can be combined; the formula is the [SMAX] rescale
 * rule written for normalised pairs):
 *   M = max(lse_a, lse_b); lse = M + ln(e^{lse_a - M} + e^{lse_b - M});
 *   o = e^{lse_a - lse} o_a + e^{lse_b - lse} o_b.
 * Both -inf (neither side saw a key) gives o = 0, lse = -inf.
 */
void oracle_lse_merge(const double* o_a, const double* lse_a,
                      const double* o_b, const double* lse_b, int64_t rows,
                      int64_t D, double* o_out, double* lse_out) {
    for (int64_t r = 0; r < rows; ++r) {
        const double a = lse_a[r], b = lse_b[r];
        const double M = a > b ? a : b;
        if (M == -INFINITY) {
            for (int64_t c = 0; c < D; ++c) o_out[r * D + c] = 0.0;
            lse_out[r] = -INFINITY;
            continue;
        }
        const double lse = M + log(exp(a - M) + exp(b - M));
        const double wa = exp(a - lse), wb = exp(b - lse);
        for (int64_t c = 0; c < D; ++c)
            o_out[r * D + c] = wa * o_a[r * D + c] + wb * o_b[r * D + c];
        lse_out[r] = lse;
    }
}

/*
 * O4: gradients of the definition O1 (the pages give no backward formulas;
 * these are the chain rule applied to out_i = sum_j p_ij v_j with
 * p_ij = e^{s_ij} / sum_j' e^{s_ij'} over the allowed keys and
 * s_ij = scale q_i . k_j). With dout the gradient of a loss with respect to
 * out, for each query row i:
 *   dv_j  += p_ij dout_i                      (every allowed key j)
 *   dp_ij  = dout_i . v_j
 *   ds_ij  = p_ij (dp_ij - sum_j' p_ij' dp_ij')
 *   dq_i   = scale sum_j ds_ij k_j
 *   dk_j  += scale ds_ij q_i
 * Rows of the query heads that share a key/value head all add into that
 * head's dk, dv. dq: [B, Tq, Hq, D]; dk, dv: [B, Tk, Hkv, D]; all fp64,
 * overwritten. Parallel over (batch, key/value head) so that no two threads
 * add into the same dk, dv rows. Returns 0, or -1 on a bad argument.
 */
int oracle_attention_backward(const void* q, int q_bf16, const void* k,
                              const void* v, int kv_bf16, const void* dout,
                              int dout_bf16, int64_t B, int64_t Hq, int64_t Hkv,
                              int64_t Tq, int64_t Tk, int64_t D, int64_t q_off,
                              int64_t k_off, int causal, double scale,
                              double* dq, double* dk, double* dv) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Tq < 0 || Tk < 0 || D <= 0)
        return -1;
    const int64_t group = Hq / Hkv;
    memset(dq, 0, sizeof(double) * (size_t)(B * Tq * Hq * D));
    memset(dk, 0, sizeof(double) * (size_t)(B * Tk * Hkv * D));
    memset(dv, 0, sizeof(double) * (size_t)(B * Tk * Hkv * D));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < B * Hkv; ++bg) {
        const int64_t b = bg / Hkv, g = bg % Hkv;
        double* s = (double*)malloc(sizeof(double) * (size_t)(Tk > 0 ? Tk : 1));
        double* p = (double*)malloc(sizeof(double) * (size_t)(Tk > 0 ? Tk : 1));
        double* dp = (double*)malloc(sizeof(double) * (size_t)(Tk > 0 ? Tk : 1));
        for (int64_t h = g * group; h < (g + 1) * group; ++h) {
            for (int64_t i = 0; i < Tq; ++i) {
                const int64_t qpos = q_off + i;
                double M = -INFINITY;
                for (int64_t j = 0; j < Tk; ++j) {
                    if (allowed(causal, k_off + j, qpos)) {
                        s[j] = score(q, q_bf16, k, kv_bf16, b, i, h, j, g, Tq, Hq,
                                     Tk, Hkv, D, scale);
                        if (s[j] > M) M = s[j];
                    }
                }
                if (M == -INFINITY) continue;   /* no allowed key: no gradient */
                double Z = 0.0;
                for (int64_t j = 0; j < Tk; ++j) {
                    p[j] = allowed(causal, k_off + j, qpos) ? exp(s[j] - M) : 0.0;
                    Z += p[j];
                }
                double pdp = 0.0;
                for (int64_t j = 0; j < Tk; ++j) {
                    p[j] /= Z;
                    dp[j] = 0.0;
                    if (!allowed(causal, k_off + j, qpos)) continue;
                    for (int64_t c = 0; c < D; ++c)
                        dp[j] += load_elem(dout, dout_bf16, qk_index(b, i, h, c, Tq, Hq, D)) *
                                 load_elem(v, kv_bf16, qk_index(b, j, g, c, Tk, Hkv, D));
                    pdp += p[j] * dp[j];
                }
                double* dqi = dq + qk_index(b, i, h, 0, Tq, Hq, D);
                for (int64_t j = 0; j < Tk; ++j) {
                    if (!allowed(causal, k_off + j, qpos)) continue;
                    const double ds = p[j] * (dp[j] - pdp);
                    double* dkj = dk + qk_index(b, j, g, 0, Tk, Hkv, D);
                    double* dvj = dv + qk_index(b, j, g, 0, Tk, Hkv, D);
                    for (int64_t c = 0; c < D; ++c) {
                        dqi[c] += scale * ds * load_elem(k, kv_bf16, qk_index(b, j, g, c, Tk, Hkv, D));
                        dkj[c] += scale * ds * load_elem(q, q_bf16, qk_index(b, i, h, c, Tq, Hq, D));
                        dvj[c] += p[j] * load_elem(dout, dout_bf16, qk_index(b, i, h, c, Tq, Hq, D));
                    }
                }
            }
        }
        free(s);
        free(p);
        free(dp);
    }
    return 0;
}
