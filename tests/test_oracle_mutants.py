"""The oracle's pins can fail: each plausible mistake below, planted in a
copy of oracle/oracle.c, must make at least one CPU pin test fail.

The mistakes cover every oracle function: the exact bf16 widening, the
causal rule of web page "Sequence parallelism -- splitting the token
dimension across GPUs" (section "Causal attention gives us another
optimization": a query sees keys at or before its own global position), the
softmax and scale of section "Attention wants keys and values from other
tokens", the running (m, l, o) update of section "But softmax seems to
require all attention scores at once", the tile and block classes (O3), the
log-sum-exp merge (section "Training and inference stress this dimension
differently") and the chain-rule gradients (O4). Each mutant is compiled
with the oracle's own gcc flags into a temporary library that the pin
tests load through CAKV_ORACLE_LIB.

Not listed: changing which scores feed the stabilising maximum M alone,
which leaves every result unchanged in exact arithmetic (M cancels in
e^{s - M} / sum e^{s - M}), so no test of results can or should catch it.
"""
import os
import pathlib
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = (ROOT / "oracle" / "oracle.c").read_text()
PIN_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_tiles.py",
             "tests/test_inputs_and_sizes.py", "tests/test_tolerances.py"]

# (name, text in oracle.c, replacement): each text occurs exactly once
MUTANTS = [
    ("bf16 widening shifted by 15", "<< 16;\n        float f;", "<< 15;\n        float f;"),
    ("diagonal excluded", "return !causal || key_pos <= query_pos;",
     "return !causal || key_pos < query_pos;"),
    ("mask reversed", "return !causal || key_pos <= query_pos;",
     "return !causal || key_pos >= query_pos;"),
    ("scale dropped", "return acc * scale;", "return acc;"),
    ("K read from the query head",
     "load_elem(k, kv_bf16, qk_index(b, j, g, c, Tk, Hkv, D));\n    return",
     "load_elem(k, kv_bf16, qk_index(b, j, h % Hkv, c, Tk, Hkv, D));\n    return"),
    ("O1 grouped heads by modulo",
     "const int64_t g = h / group;\n        const int64_t qpos = q_off + i;\n        double* s =",
     "const int64_t g = h % Hkv;\n        const int64_t qpos = q_off + i;\n        double* s ="),
    ("O1 query offset ignored", "const int64_t qpos = q_off + i;\n        double* s =",
     "const int64_t qpos = i;\n        double* s ="),
    ("O1 key offset ignored", "if (allowed(causal, k_off + j, qpos)) {\n                s[j] = score",
     "if (allowed(causal, j, qpos)) {\n                s[j] = score"),
    ("O1 lse without the maximum", "lse[r] = M + log(Z);", "lse[r] = log(Z);"),
    ("O1 output not normalised", "for (int64_t c = 0; c < D; ++c) o[c] /= Z;", ""),
    ("O1 exponent sign", "const double e = exp(s[j] - M);", "const double e = exp(M - s[j]);"),
    ("O1 empty row lse 0", "        } else {\n            lse[r] = -INFINITY;\n        }",
     "        } else {\n            lse[r] = 0.0;\n        }"),
    ("O1 weights not normalised", "? exp(s[j] - M) / Z", "? exp(s[j] - M)"),
    ("O2 old terms rescaled the wrong way", "exp(m - m_new);\n            const double a_new",
     "exp(m_new - m);\n            const double a_new"),
    ("O2 new l terms not rescaled", "l = l * a_old + lb * a_new;", "l = l * a_old + lb;"),
    ("O2 new o terms not rescaled", "o[c] = o[c] * a_old + ob[c] * a_new;",
     "o[c] = o[c] * a_old + ob[c];"),
    ("O2 running maximum not updated", "            m = m_new;\n        }", "        }"),
    ("O2 last key of a block dropped",
     "const int64_t j0 = starts[blk], j1 = starts[blk] + lens[blk];",
     "const int64_t j0 = starts[blk], j1 = starts[blk] + lens[blk] - 1;"),
    ("O2 lse without the maximum", "lse[r] = l > 0.0 ? m + log(l) : -INFINITY;",
     "lse[r] = l > 0.0 ? log(l) : -INFINITY;"),
    ("O3 one masked pair counts as full", "else if (p == (i1 - i0) * (j1 - j0)) ++n_full;",
     "else if (p >= (i1 - i0) * (j1 - j0) - 1) ++n_full;"),
    ("O3 last tile not clipped",
     "const int64_t j1 = j0 + tile_k < lens[t] ? j0 + tile_k : lens[t];",
     "const int64_t j1 = j0 + tile_k;"),
    ("O3 query offset ignored", "p += allowed(causal, k_off + starts[t] + j, q_off + i);",
     "p += allowed(causal, k_off + starts[t] + j, i);"),
    ("O3 block start ignored", "p += allowed(causal, k_off + starts[t] + j, q_off + i);",
     "p += allowed(causal, k_off + j, q_off + i);"),
    ("O3 block class off by one",
     "block_class[t] = (pairs == 0) ? 2 : (pairs == total ? 0 : 1);",
     "block_class[t] = (pairs == 0) ? 2 : (pairs >= total - 1 ? 0 : 1);"),
    ("O3 counts not scaled by heads", "tile_counts[c] = tc[c] * B * Hq;",
     "tile_counts[c] = tc[c] * B;"),
    ("O3 skipped tile counted as masked", "if (p == 0) ++n_skip;", "if (p == 0) ++n_part;"),
    ("merge weights swapped",
     "o_out[r * D + c] = wa * o_a[r * D + c] + wb * o_b[r * D + c];",
     "o_out[r * D + c] = wb * o_a[r * D + c] + wa * o_b[r * D + c];"),
    ("merge lse without the maximum", "const double lse = M + log(exp(a - M) + exp(b - M));",
     "const double lse = log(exp(a - M) + exp(b - M));"),
    ("merge of two empty rows gives lse 0",
     "            lse_out[r] = -INFINITY;\n            continue;",
     "            lse_out[r] = 0.0;\n            continue;"),
    ("O4 dk without the scale", "dkj[c] += scale * ds *", "dkj[c] += ds *"),
    ("O4 delta dropped", "const double ds = p[j] * (dp[j] - pdp);", "const double ds = p[j] * dp[j];"),
    ("O4 dv from ds", "dvj[c] += p[j] * load_elem(dout", "dvj[c] += ds * load_elem(dout"),
    ("O4 dq from q",
     "dqi[c] += scale * ds * load_elem(k, kv_bf16, qk_index(b, j, g, c, Tk, Hkv, D));",
     "dqi[c] += scale * ds * load_elem(q, q_bf16, qk_index(b, i, h, c, Tq, Hq, D));"),
    ("O4 grouped heads by modulo", "for (int64_t h = g * group; h < (g + 1) * group; ++h) {",
     "for (int64_t h = g; h < Hq; h += Hkv) {"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, old, new, tmp_path):
    assert SRC.count(old) == 1, f"{name}: the text to replace must occur once in oracle.c"
    c_file = tmp_path / "oracle_mutant.c"
    lib = tmp_path / "liboracle_mutant.so"
    c_file.write_text(SRC.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                    "-o", str(lib), str(c_file), "-lm"], check=True)
    env = dict(os.environ, CAKV_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", *PIN_TESTS, "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 1, f"{name}: no pin failed\n{r.stdout[-2000:]}"


def test_pins_pass_on_the_committed_oracle():
    """The same pin run passes on the committed oracle, so a mutant's failure
    is the mutant's doing."""
    env = dict(os.environ, OMP_NUM_THREADS="4")
    env.pop("CAKV_ORACLE_LIB", None)
    r = subprocess.run([sys.executable, "-m", "pytest", *PIN_TESTS, "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
