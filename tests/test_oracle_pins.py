"""Pins of the fp64 oracle against what the pages and the mathematics fix.

The oracle (oracle/oracle.c) is the definition the GPU path is judged by, so
it is checked here against things other than itself:
  * brute force written a second way (pure-Python math.exp loops, a bf16
    decoder of its own) on tiny inputs, covering offsets, GQA and bf16;
  * closed forms (one key, zero keys, two keys by hand, a dominant key);
  * invariants the page states or implies: weights sum to one, causal rows
    ignore later keys, the result does not depend on how the keys are cut into
    blocks or in which order the blocks arrive (page "Sequence parallelism --
    splitting the token dimension across GPUs", section "But softmax seems to
    require all attention scores at once");
  * softmax algebra: shift of every key, scaling of V, permutation of keys;
  * the log-sum-exp merge: identity, commutativity, associativity, and that
    merging per-block partials reproduces the whole.
"""
import itertools
import math
import struct

import numpy as np
import pytest

import oracle


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bits with round-to-nearest-even (test-local)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _brute(q, k, v, q_off, k_off, causal, scale):
    """softmax(q k^T * scale) v for every row, by pure-Python loops."""
    B, Tq, Hq, D = q.shape
    _, Tk, Hkv, _ = k.shape
    grp = Hq // Hkv
    val = (lambda a, idx: _bf16_value(a[idx])) if q.dtype == np.uint16 else (
        lambda a, idx: float(a[idx]))
    outs, lses = [], []
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for i in range(Tq):
                s = []
                for j in range(Tk):
                    if causal and k_off + j > q_off + i:
                        continue
                    dot = sum(val(q, (b, i, h, c)) * val(k, (b, j, g, c)) for c in range(D))
                    s.append((j, dot * scale))
                if not s:
                    outs.append([0.0] * D)
                    lses.append(-math.inf)
                    continue
                z = sum(math.exp(x) for _, x in s)
                outs.append([sum(math.exp(x) / z * val(v, (b, j, g, c)) for j, x in s)
                             for c in range(D)])
                lses.append(math.log(z))
    return np.array(outs), np.array(lses)


def _randn(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", [
    dict(B=1, Tq=5, Tk=5, Hq=1, Hkv=1, D=3, q_off=0, k_off=0),
    dict(B=2, Tq=3, Tk=8, Hq=4, Hkv=2, D=4, q_off=5, k_off=0),   # last chunk, GQA 2
    dict(B=1, Tq=4, Tk=3, Hq=2, Hkv=1, D=2, q_off=2, k_off=3),   # some rows see nothing
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_o1_matches_brute_force(case, causal, dtype):
    rng = np.random.default_rng(7)
    q = _randn(rng, (case["B"], case["Tq"], case["Hq"], case["D"]))
    k = _randn(rng, (case["B"], case["Tk"], case["Hkv"], case["D"]))
    v = _randn(rng, (case["B"], case["Tk"], case["Hkv"], case["D"]))
    if dtype == "bf16":
        q, k, v = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v)
    scale = 1.0 / math.sqrt(case["D"])
    out, lse = oracle.attention(q, k, v, q_off=case["q_off"], k_off=case["k_off"],
                                causal=causal, scale=scale)
    # brute force gives lse relative to no max: lse = ln sum e^{s}
    bo, bl = _brute(q, k, v, case["q_off"], case["k_off"], causal, scale)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-13)
    assert np.all(lse[~fin] == -np.inf) and np.all(out[~fin] == 0)


def test_single_key_closed_form():
    rng = np.random.default_rng(1)
    q = _randn(rng, (1, 1, 1, 8))
    k = _randn(rng, (1, 1, 1, 8))
    v = _randn(rng, (1, 1, 1, 8))
    out, lse = oracle.attention(q, k, v, causal=True)
    np.testing.assert_array_equal(out[0], v[0, 0, 0].astype(np.float64))
    s = float(np.dot(q[0, 0, 0].astype(np.float64), k[0, 0, 0].astype(np.float64))) / math.sqrt(8)
    assert abs(lse[0] - s) <= 1e-14 * max(1.0, abs(s))


@pytest.mark.parametrize("causal", [True, False])
def test_zero_keys_give_means(causal):
    """With K = 0 all scores are 0: row i averages the allowed values and
    lse = ln(number of allowed keys)."""
    rng = np.random.default_rng(2)
    T, D = 9, 4
    q = _randn(rng, (1, T, 1, D))
    k = np.zeros((1, T, 1, D), np.float32)
    v = _randn(rng, (1, T, 1, D))
    out, lse = oracle.attention(q, k, v, causal=causal)
    vv = v[0, :, 0].astype(np.float64)
    for i in range(T):
        n = i + 1 if causal else T
        np.testing.assert_allclose(out[i], vv[:n].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert abs(lse[i] - math.log(n)) < 1e-14


def test_two_keys_by_hand():
    """d_k = 1, q = 2, keys 0 and 1, scale 1/2: scores 0 and 1, weights
    1/(1+e) and e/(1+e), lse = ln(1+e)."""
    q = np.array([2.0], np.float32).reshape(1, 1, 1, 1)
    k = np.array([0.0, 1.0], np.float32).reshape(1, 2, 1, 1)
    v = np.array([3.0, -5.0], np.float32).reshape(1, 2, 1, 1)
    out, lse, w = oracle.attention(q, k, v, q_off=1, causal=True, scale=0.5,
                                   return_weights=True)
    e = math.e
    assert abs(w[0, 0] - 1 / (1 + e)) < 1e-15 and abs(w[0, 1] - e / (1 + e)) < 1e-15
    assert abs(out[0, 0] - (3.0 / (1 + e) - 5.0 * e / (1 + e))) < 1e-14
    assert abs(lse[0] - math.log(1 + e)) < 1e-15


def test_dominant_key():
    """One key 100 logits above every other: out = its value within e^-100."""
    D, T = 4, 6
    q = np.zeros((1, 1, 1, D), np.float32)
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, T, 1, D), np.float32)
    k[0, 3, 0, 0] = 200.0  # scale 1/2 -> score 100
    v = np.random.default_rng(3).standard_normal((1, T, 1, D)).astype(np.float32)
    out, lse = oracle.attention(q, k, v, q_off=T - 1, causal=True)
    np.testing.assert_allclose(out[0], v[0, 3, 0].astype(np.float64), atol=1e-40, rtol=1e-14)
    assert abs(lse[0] - 100.0) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_weights_are_a_distribution(causal):
    rng = np.random.default_rng(4)
    T, D = 33, 8
    q, k, v = (_randn(rng, (2, T, 2, D)) for _ in range(3))
    out, lse, w = oracle.attention(q, k, v, causal=causal, return_weights=True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-13)
    assert np.all(w >= 0)
    if causal:
        rows = oracle._rows_array(None, 2, 2, T)
        for r, (_, _, i) in enumerate(rows):
            assert np.all(w[r, i + 1:] == 0) and w[r, i] > 0


def test_causal_row_ignores_later_keys():
    rng = np.random.default_rng(5)
    T, D = 24, 8
    q, k, v = (_randn(rng, (1, T, 1, D)) for _ in range(3))
    out0, lse0 = oracle.attention(q, k, v, causal=True)
    for i in (0, 7, 16, 22):
        k2, v2 = k.copy(), v.copy()
        k2[0, i + 1:] = _randn(rng, k2[0, i + 1:].shape) * 9
        v2[0, i + 1:] = np.nan
        out1, lse1 = oracle.attention(q, k2, v2, causal=True, rows=[(0, 0, i)])
        assert np.array_equal(out1[0], out0[i]) and lse1[0] == lse0[i]


def test_value_scaling_and_key_shift():
    """out(aV) = a out(V); adding u to every key keeps out and moves lse_i by
    q_i.u * scale (softmax is shift-invariant). Values are multiples of 1/8
    so k + u is exact in fp32."""
    rng = np.random.default_rng(6)
    T, D = 17, 4
    q = (rng.integers(-16, 16, (1, T, 1, D)) / 8).astype(np.float32)
    k = (rng.integers(-16, 16, (1, T, 1, D)) / 8).astype(np.float32)
    v = _randn(rng, (1, T, 1, D))
    u = np.array([0.5, -0.25, 1.0, 0.125], np.float32)
    out, lse = oracle.attention(q, k, v, causal=True)
    out2, _ = oracle.attention(q, k, (2 * v).astype(np.float32), causal=True)
    np.testing.assert_allclose(out2, 2 * out, rtol=1e-14, atol=1e-15)
    out3, lse3 = oracle.attention(q, (k + u).astype(np.float32), v, causal=True)
    np.testing.assert_allclose(out3, out, rtol=1e-12, atol=1e-13)
    shift = q[0, :, 0].astype(np.float64) @ u.astype(np.float64) * 0.5
    np.testing.assert_allclose(lse3 - lse, shift, atol=1e-12)


def test_bidirectional_key_permutation():
    rng = np.random.default_rng(8)
    T, D = 20, 8
    q, k, v = (_randn(rng, (1, T, 1, D)) for _ in range(3))
    perm = rng.permutation(T)
    out, lse = oracle.attention(q, k, v, causal=False)
    outp, lsep = oracle.attention(q, k[:, perm], v[:, perm], causal=False)
    np.testing.assert_allclose(outp, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lsep, lse, rtol=1e-13, atol=1e-13)


def _chunks(T, n):
    c = T // n
    return np.arange(n) * c, np.full(n, c)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_blockwise_equals_plain_for_any_chunk_count(n, causal):
    """Page section 'But softmax seems to require all attention scores at
    once': tiling does not change the result. O2 over N blocks in ring order
    r, r-1, ... equals O1 for every rank of N."""
    rng = np.random.default_rng(9)
    T, D = 64, 8
    q, k, v = (_randn(rng, (2, T, 2, D)) for _ in range(3))
    k[:, :, 1] *= 8  # sharp head: larger rescale factors
    starts, lens = _chunks(T, n)
    C = T // n
    for r in range(n):
        ql = np.ascontiguousarray(q[:, r * C:(r + 1) * C])
        order = [(r - t) % n for t in range(n)]
        o1, l1 = oracle.attention(ql, k, v, q_off=r * C, causal=causal)
        o2, l2 = oracle.online_blockwise(ql, k, v, starts, lens, order, q_off=r * C,
                                         causal=causal)
        np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)


def test_blockwise_any_block_order():
    rng = np.random.default_rng(10)
    T, D, n = 32, 4, 4
    q, k, v = (_randn(rng, (1, T, 1, D)) for _ in range(3))
    starts, lens = _chunks(T, n)
    ql = np.ascontiguousarray(q[:, 24:])
    o1, l1 = oracle.attention(ql, k, v, q_off=24, causal=True)
    for order in itertools.permutations(range(n)):
        o2, l2 = oracle.online_blockwise(ql, k, v, starts, lens, order, q_off=24)
        np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)


def test_blockwise_state_is_running_statistics():
    """After the blocks the state is m = max score, l = sum e^{s-m},
    o = sum e^{s-m} v (unnormalised), so o / l = out and m + ln l = lse."""
    rng = np.random.default_rng(11)
    T, D = 16, 4
    q, k, v = (_randn(rng, (1, T, 1, D)) for _ in range(3))
    starts, lens = _chunks(T, 4)
    out, lse, (m, l_, o) = oracle.online_blockwise(q, k, v, starts, lens, [0, 1, 2, 3],
                                                   causal=True, return_state=True)
    _, _, w = oracle.attention(q, k, v, causal=True, return_weights=True)
    s = (q[0, :, 0].astype(np.float64) @ k[0, :, 0].astype(np.float64).T) / 2.0
    for i in range(T):
        assert m[i] == pytest.approx(s[i, :i + 1].max(), abs=1e-14)
    np.testing.assert_allclose(o / l_[:, None], out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(m + np.log(l_), lse, rtol=1e-13, atol=1e-14)


def test_blockwise_empty_rows_are_zero_and_minus_inf():
    rng = np.random.default_rng(12)
    q, k, v = (_randn(rng, (1, 4, 1, 4)) for _ in range(3))
    # keys at positions 10.., queries at 0..3: nothing allowed
    out, lse = oracle.online_blockwise(q, k, v, [0], [4], [0], k_off=10, causal=True)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_merge_algebra_and_recombination():
    rng = np.random.default_rng(13)
    T, D, n = 48, 8, 4
    q, k, v = (_randn(rng, (1, T, 1, D)) for _ in range(3))
    k *= 3
    C = T // n
    ql = np.ascontiguousarray(q[:, 3 * C:])
    full_o, full_l = oracle.attention(ql, k, v, q_off=3 * C, causal=True)
    parts = [oracle.attention(ql, np.ascontiguousarray(k[:, j * C:(j + 1) * C]),
                              np.ascontiguousarray(v[:, j * C:(j + 1) * C]),
                              q_off=3 * C, k_off=j * C, causal=True) for j in range(n)]
    # identity (0, -inf)
    zero_o = np.zeros_like(full_o)
    ninf = np.full_like(full_l, -np.inf)
    o, l_ = oracle.lse_merge(parts[0][0], parts[0][1], zero_o, ninf)
    np.testing.assert_array_equal(o, parts[0][0])
    np.testing.assert_array_equal(l_, parts[0][1])
    o, l_ = oracle.lse_merge(zero_o, ninf, zero_o, ninf)
    assert np.all(o == 0) and np.all(l_ == -np.inf)
    # commutative
    a = oracle.lse_merge(*parts[1], *parts[2])
    b = oracle.lse_merge(*parts[2], *parts[1])
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-15, atol=1e-15)
    # associative and recombines to the whole, in ring order and as a tree
    seq = parts[3]
    for j in (2, 1, 0):
        seq = oracle.lse_merge(*seq, *parts[j])
    tree = oracle.lse_merge(*oracle.lse_merge(*parts[0], *parts[1]),
                            *oracle.lse_merge(*parts[2], *parts[3]))
    for got in (seq, tree):
        np.testing.assert_allclose(got[0], full_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got[1], full_l, rtol=1e-13, atol=1e-13)


def test_classify_matches_page_causal_needs():
    """Page section 'Causal attention gives us another optimization'."""
    rows = [l.split() for l in open(_golden("page_causal_needs_n4.txt"))
            if l.strip() and not l.startswith("#")]
    C, n = 8, 4
    starts, lens = _chunks(C * n, n)
    for gpu in range(n):
        cls, pairs, _ = oracle.classify(C, gpu * C, starts, lens, causal=True)
        for g, j, need, _src in rows:
            if int(g) == gpu:
                assert (pairs[int(j)] > 0) == bool(int(need))
                assert cls[int(j)] == (2 if not int(need) else (1 if int(j) == gpu else 0))


def test_classify_pair_counts_closed_form():
    """Rank r of N equal chunks of C under a causal mask sees r*C*C + C(C+1)/2
    pairs; bidirectional sees N*C*C. Tiles: brute-force counts add up."""
    for C, n in ((8, 4), (37, 3), (64, 2)):
        starts, lens = _chunks(C * n, n)
        for r in range(n):
            _, pairs, tiles = oracle.classify(C, r * C, starts, lens, causal=True,
                                              tile_q=32, tile_k=64)
            assert pairs.sum() == r * C * C + C * (C + 1) // 2
            nt = -(-C // 32) * -(-C // 64) * n
            assert tiles.sum() == nt
            _, pairs, tiles = oracle.classify(C, r * C, starts, lens, causal=False)
            assert pairs.sum() == n * C * C and tiles[1] == 0 and tiles[2] == 0


def test_classify_tile_counts_small_by_hand():
    """C=64, tiles 32x64, rank 1 of 2: block 0 is all FULL (2 tiles), block 1
    (diagonal) has two row tiles, both partially masked."""
    starts, lens = _chunks(128, 2)
    cls, _, tiles = oracle.classify(64, 64, starts, lens, causal=True, tile_q=32, tile_k=64)
    assert list(cls) == [0, 1] and list(tiles) == [2, 2, 0]
    # tile_k = 16: diagonal block rows 0..31 see key tiles 0,1 partly/fully
    cls, _, tiles = oracle.classify(64, 64, starts, lens, causal=True, tile_q=32, tile_k=16)
    # block 0: 2x4 FULL; block 1: row tile 0 -> keys 0-15 masked, 16-31 masked,
    # 32-63 skip; row tile 1 -> 0-15, 16-31 full, 32-47, 48-63 masked
    assert list(tiles) == [8 + 2, 4, 2]


def _golden(name):
    import os
    return os.path.join(os.path.dirname(__file__), "golden", name)


def test_classify_respects_key_offset():
    """Only position differences matter: moving the keys by one chunk equals
    moving the queries back by one; keys entirely after the queries are SKIP."""
    C, n = 16, 4
    starts, lens = _chunks(C * n, n)
    cls, pairs, _ = oracle.classify(C, 0, starts, lens, k_off=C, causal=True)
    assert list(cls) == [2, 2, 2, 2] and pairs.sum() == 0
    for r in range(1, n):
        a = oracle.classify(C, r * C, starts, lens, k_off=C, causal=True)
        b = oracle.classify(C, (r - 1) * C, starts, lens, k_off=0, causal=True)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


# ---- O4: gradients of the definition --------------------------------------

def _loss(q, k, v, dout, q_off, causal, k_off=0):
    """sum(out * dout) with out from O1 (fp64 on the stored inputs)."""
    B, Tq, Hq, D = q.shape
    o, _ = oracle.attention(q, k, v, q_off=q_off, k_off=k_off, causal=causal)
    # O1 rows come b-major, then head, then position
    o = o.reshape(B, Hq, Tq, D).transpose(0, 2, 1, 3)
    return float((o * dout.astype(np.float64)).sum())


@pytest.mark.parametrize("causal,k_off", [(True, 0), (False, 0), (True, 4)])
def test_o4_matches_finite_differences(causal, k_off):
    """Central differences of sum(out * dout) through O1, element by element
    on a sample of q, k and v entries (perturbations taken exactly as the
    difference of the two stored fp32 values). With k_off = 4 the keys sit
    at positions 4..10, so the causal rule compares global positions: the
    query at 3 sees no key (no gradient), the one at 7 sees four."""
    rng = np.random.default_rng(41 + causal + k_off)
    B, Tq, Tk, Hq, Hkv, D = 1, 5, 7, 4, 2, 8
    q = rng.standard_normal((B, Tq, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Tk, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, Tk, Hkv, D)).astype(np.float32)
    dout = rng.standard_normal((B, Tq, Hq, D)).astype(np.float32)
    q_off = 3   # queries at 3..7 see keys up to their own position when causal
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, q_off=q_off, k_off=k_off,
                                           causal=causal)
    eps = 1.0 / 512
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        idx = list(np.ndindex(x.shape))
        pick = [idx[i] for i in rng.choice(len(idx), 24, replace=False)]
        for e in pick:
            xp, xm = x.copy(), x.copy()
            xp[e] = np.float32(x[e] + eps)
            xm[e] = np.float32(x[e] - eps)
            h = float(xp[e]) - float(xm[e])
            args = {"q": q, "k": k, "v": v}
            lp = _loss(*[xp if n == name else args[n] for n in ("q", "k", "v")], dout, q_off,
                       causal, k_off)
            lm = _loss(*[xm if n == name else args[n] for n in ("q", "k", "v")], dout, q_off,
                       causal, k_off)
            fd = (lp - lm) / h
            assert abs(fd - g[e]) <= 2e-5 * max(1.0, abs(fd)), (name, e, fd, g[e])


def test_o4_single_key_closed_form():
    """One key: p = 1, so dv = the sum of dout over the query heads that read
    it, and dq = dk = 0."""
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 1, 2, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, 1, 8)).astype(np.float32)
    v = rng.standard_normal((1, 1, 1, 8)).astype(np.float32)
    dout = rng.standard_normal((1, 1, 2, 8)).astype(np.float32)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=False)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0, 0, 0], dout[0, 0].astype(np.float64).sum(axis=0), rtol=0,
                               atol=1e-12)


def test_o4_invariants_bidirectional():
    """Every row sees every key: shifting all keys by one vector leaves the
    output unchanged, so the key gradients of each head sum to zero; the
    weights of a row sum to 1, so the value gradients sum to the rows' dout."""
    rng = np.random.default_rng(44)
    B, Tq, Tk, Hq, Hkv, D = 2, 6, 9, 4, 2, 16
    q = rng.standard_normal((B, Tq, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Tk, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, Tk, Hkv, D)).astype(np.float32)
    dout = rng.standard_normal((B, Tq, Hq, D)).astype(np.float32)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=False)
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    G = Hq // Hkv
    want = dout.astype(np.float64).reshape(B, Tq, Hkv, G, D).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=0, atol=1e-11)


def test_o4_causal_future_keys_get_nothing():
    """Causal: keys after every query get zero gradients, and a query's
    gradient does not move when a later key changes."""
    rng = np.random.default_rng(45)
    q = rng.standard_normal((1, 4, 2, 8)).astype(np.float32)
    k = rng.standard_normal((1, 10, 2, 8)).astype(np.float32)
    v = rng.standard_normal((1, 10, 2, 8)).astype(np.float32)
    dout = rng.standard_normal((1, 4, 2, 8)).astype(np.float32)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, q_off=2, causal=True)
    assert not dk[0, 6:].any() and not dv[0, 6:].any()      # keys 6..9 follow queries 2..5
    k2 = k.copy()
    k2[0, 5] += 1.0                                           # key 5: seen by query 5 only
    dq2, _, _ = oracle.attention_backward(q, k2, v, dout, q_off=2, causal=True)
    assert np.array_equal(dq[0, :3], dq2[0, :3]) and not np.array_equal(dq[0, 3], dq2[0, 3])


def test_o4_bf16_inputs_read_as_their_values():
    """O4 on bf16 bit patterns (the GPU tests' inputs: q, k, v and dout all
    bf16) equals O4 on fp32 arrays holding the same values, decoded by this
    file's own bf16 decoder; also with the dtypes mixed, so each operand's
    dtype flag is honoured on its own."""
    rng = np.random.default_rng(46)
    B, Tq, Tk, Hq, Hkv, D = 1, 5, 9, 4, 2, 8
    bits = {n: _bf16_bits(rng.standard_normal(s).astype(np.float32))
            for n, s in (("q", (B, Tq, Hq, D)), ("k", (B, Tk, Hkv, D)),
                         ("v", (B, Tk, Hkv, D)), ("dout", (B, Tq, Hq, D)))}
    vals = {n: np.vectorize(_bf16_value)(b).astype(np.float32) for n, b in bits.items()}
    want = oracle.attention_backward(vals["q"], vals["k"], vals["v"], vals["dout"], q_off=4,
                                     causal=True)
    for mix in (("q", "k", "v", "dout"), ("q",), ("k", "v"), ("dout",)):
        args = {n: (bits[n] if n in mix else vals[n]) for n in bits}
        got = oracle.attention_backward(args["q"], args["k"], args["v"], args["dout"], q_off=4,
                                        causal=True)
        for g, w in zip(got, want):
            assert np.array_equal(g, w), mix
