"""Seeded inputs and the sizes the page prints.

* The generator is SplitMix64 (Steele, Lea, Flood 2014); its first outputs for
  seed 0 are published with the reference implementation and checked here,
  then slices of a tensor must equal the same slice of the whole tensor.
* Page "Sequence parallelism -- splitting the token dimension across GPUs":
  section "Start with the hidden-state tensor" (B=8, T=32,768, d=8192 bf16 is
  4,294,967,296 bytes), section "Split tokens across four GPUs" (token ranges
  and roughly 1 GiB per GPU), section "Attention wants keys and values from
  other tokens" (token 30,000 lives on GPU 3). The hidden-state workload
  (8 x 32768 tokens, 64 heads x 128) is that tensor cut by heads.
"""
import os

import numpy as np

import cakv_synth as syn


def _golden(name):
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    out = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            out[k] = [int(x) for x in v]
    return out


def test_splitmix64_reference_values():
    # SplitMix64 seeded with state 0: the first outputs of the published
    # algorithm (state += GAMMA; mix) are these well-known constants.
    lib = syn._load()
    assert lib.synth_raw(0, 0) == 0xE220A8397B1DCDAF
    assert lib.synth_raw(0, 1) == 0x6E789E6AA1B965F4
    assert lib.synth_raw(0, 2) == 0x06C45D188009454F


def test_slices_match_whole_tensor():
    w = syn.scaled(syn.WORKLOADS[2], T=256, N=4)
    q_full = syn.make_q_full(w)
    for r in range(w.N):
        ql = syn.make_q_local(w, r)
        np.testing.assert_array_equal(ql, q_full[:, r * w.C:(r + 1) * w.C])
    a = syn.make_kv_full(w, "k")
    b = syn.make_kv_full(w, "k")
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, syn.make_kv_full(w, "v"))


def test_distributions():
    x = np.empty(1 << 20, np.float32)
    syn.fill(x, seed=5, tensor=0)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    syn.fill(x, seed=5, tensor=0, dist=syn.UNIFORM)
    assert x.min() >= -1 and x.max() < 1 and abs(x.mean()) < 5e-3
    assert abs(x.var() - 1 / 3) < 5e-3


def test_head_multiplier_is_exact_times_eight():
    w = syn.scaled(syn.WORKLOADS[2], T=64, N=4)
    k = syn.bf16_to_f32(syn.make_kv_full(w, "k"))
    w1 = syn.scaled(w, k_head_mul=None)
    k1 = syn.bf16_to_f32(syn.make_kv_full(w1, "k"))
    np.testing.assert_array_equal(k[:, :, 4:], 8 * k1[:, :, 4:])
    np.testing.assert_array_equal(k[:, :, :4], k1[:, :, :4])


def test_hidden_state_size_pin():
    g = _golden("page_sizes.txt")
    w = syn.WORKLOADS[4]
    assert g["hidden_B"] == [w.B] and g["hidden_T"] == [w.T]
    assert g["hidden_d"] == [w.Hq * w.D]
    bytes_per = g["hidden_bytes_per_elem"][0]
    assert w.B * w.T * w.Hq * w.D * bytes_per == g["hidden_bytes"][0] == 4294967296
    # the full K (or V) of that workload is exactly one such tensor
    assert w.B * w.T * w.Hkv * w.D * 2 == 4294967296


def test_local_shard_pins():
    g = _golden("page_sizes.txt")
    w = syn.WORKLOADS[4]
    assert g["gpus"] == [w.N]
    C = w.C
    for r in range(w.N):
        lo, hi = g[f"range_gpu{r}"]           # 1-based, inclusive
        assert (lo - 1, hi) == (r * C, (r + 1) * C)
    # local query shard = a quarter of the hidden state = 1 GiB
    assert w.B * C * w.Hq * w.D * 2 == g["local_portion_bytes_approx"][0]
    tok = g["causal_example_token"][0] - 1   # 0-based position
    assert tok // C == g["causal_example_owner"][0] == 3


def test_sample_rows_are_valid_and_seeded():
    w = syn.scaled(syn.WORKLOADS[4], B=2, Hq=3, Hkv=3, T=4096)
    r1 = syn.sample_rows(w, per_head=12)
    r2 = syn.sample_rows(w, per_head=12)
    np.testing.assert_array_equal(r1, r2)
    assert len(r1) == 2 * 3 * 12
    assert r1[:, 2].min() >= 0 and r1[:, 2].max() < w.C
    for req in (0, 1, 127, 128, 255, 256, w.C // 2, w.C - 2, w.C - 1):
        assert np.sum(r1[:, 2] == req) == 6
