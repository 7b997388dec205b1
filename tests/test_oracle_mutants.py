"""Pin strength: every plausible mistake planted in a copy of the oracle must fail some pin.

Each mutant is a one-line textual change to a copy of oracle/oracle.c (a dropped term, a wrong
sign, index or operand, an off-by-one in a mask). The copy is compiled into a temporary
directory and the whole pin suite runs against it in a child process (a broken build may crash,
which also counts as caught). The shipped oracle is never modified.
"""
import concurrent.futures
import json
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = [
    ("gqa head map", "const int64_t hkv = hq / G;", "const int64_t hkv = hq % P->num_kv_heads;"),
    ("causal off by one", "if (P->causal && j > pos) return 0;", "if (P->causal && j >= pos) return 0;"),
    ("window off by one", "pos - j >= P->window", "pos - j > P->window"),
    ("query position", "int64_t pos = L - q_tokens(P, b) + t;", "int64_t pos = L - 1 - t;"),
    ("varlen query position", "int64_t pos = L - q_tokens(P, b) + t;", "int64_t pos = L - P->q_len + t;"),
    ("varlen query rows", "if (P->q_starts) return q_row(P, b, t) * st[1] + hq * st[2];",
     "if (P->q_starts) return (b * P->q_len + t) * st[1] + hq * st[2];"),
    ("varlen sequence lookup", "if (P->q_starts[c] <= n && n < P->q_starts[c + 1]) b = c;",
     "if (P->q_starts[c] < n && n <= P->q_starts[c + 1]) b = c;"),
    ("tree bit order", ">> (i % 32)) & 1u);", ">> (31 - i % 32)) & 1u);"),
    ("tree first draft", "const int64_t first_draft = L - q_tokens(P, b);", "const int64_t first_draft = L - P->q_len;"),
    ("tree row pitch", "q_row(P, b, t) * words + i / 32", "q_row(P, b, t) + i / 32"),
    ("tree prefix bound", "if (j < first_draft) return 1;", "if (j <= first_draft) return 1;"),
    ("int4 field order", ">> (4 * (d % 8))) & 15u;", ">> (4 * (7 - d % 8))) & 15u;"),
    ("int4 scale and shift swapped", "(double)field * half_value(coef & 0xFFFFu) + half_value(coef >> 16)",
     "(double)field * half_value(coef >> 16) + half_value(coef & 0xFFFFu)"),
    ("int4 group of a dimension", "const uint32_t coef = w[d / (dim / n_groups)];",
     "const uint32_t coef = w[d % n_groups];"),
    ("int4 values after the coefficients", "(w[n_groups + d / 8] >>", "(w[d / 8] >>"),
    ("half exponent bias", "mag = ldexp(1.0 + m / 1024.0, e - 15);", "mag = ldexp(1.0 + m / 1024.0, e - 14);"),
    ("half subnormal scale", "mag = ldexp((double)m, -24);", "mag = ldexp((double)m, -25);"),
    ("second score part dropped",
     "acc += widen(P->q2, P->q_type, qo2 + d) * widen(P->k2, P->kv_type, ko2 + d);", "acc += 0.0;"),
    ("scale dropped", "return P->scale * acc;", "return acc;"),
    ("softmax sign", "double w = exp(s[j] - m);", "double w = exp(m - s[j]);"),
    ("lse without max", "lse[i] = m + log(l);", "lse[i] = log(l);"),
    ("no normalisation", "for (int64_t d = 0; d < P->dim_v; d++) o[d] /= l;", ""),
    ("page slot index", "(j % P->page_size) * st[1]", "(j / P->page_size) * st[1]"),
    ("page table index", "P->block_table[b * P->bt_stride + j / P->page_size]",
     "P->block_table[b * P->bt_stride + j % P->page_size]"),
    ("values read from keys", ": widen(P->v, P->kv_type, vo + d) * vs;",
     ": widen(P->k, P->kv_type, vo + d) * vs;"),
    ("bf16 widening", "<< 16;", "<< 15;"),
    ("block id off by one", "+ i * P->idx_stride[2]] == blk)", "+ i * P->idx_stride[2]] == blk + 1)"),
    ("block of key", "int64_t blk = j / P->block_size;", "int64_t blk = j % P->block_size;"),
    ("merge weight sign", "double w = exp(ls[s] - M);", "double w = exp(M - ls[s]);"),
    ("merge lse without max", "lse[r] = M + log(W);", "lse[r] = log(W);"),
    ("merge empty guard", "if (M == -INFINITY) {", "if (0) {"),
    ("empty row lse", "lse[i] = -INFINITY;\n            free(s);", "lse[i] = 0.0;\n            free(s);"),
    ("key range end", "j >= P->key_hi", "j > P->key_hi"),
    ("sequence length of row", "P->seq_lens[b] : P->kv_len", "P->seq_lens[0] : P->kv_len"),
    ("query token of row", "int64_t b = n / P->q_len, t = n % P->q_len;",
     "int64_t b = n / P->q_len, t = r % P->q_len;"),
    ("q token stride", "return b * st[0] + t * st[1] + hq * st[2];", "return b * st[0] + t * st[2] + hq * st[2];"),
    ("running max", "if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    ("merge normalisation", "for (int32_t d = 0; d < dim_v; d++) o[d] /= W;", ""),
    ("e4m3 exponent bias", "mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    ("e4m3 subnormal scale", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    ("e4m3 mantissa step", "1.0 + m / 8.0", "1.0 + m / 16.0"),
    ("e4m3 sign dropped", "        mag = ldexp(1.0 + m / 8.0, e - 7);\n    return sign ? -mag : mag;",
     "        mag = ldexp(1.0 + m / 8.0, e - 7);\n    return mag;"),
    ("half sign dropped", "        mag = ldexp(1.0 + m / 1024.0, e - 15);\n    return sign ? -mag : mag;",
     "        mag = ldexp(1.0 + m / 1024.0, e - 15);\n    return mag;"),
    ("e4m3 nan code", "if (e == 15 && m == 7)", "if (e == 15)"),
    ("key scale dropped", ": widen(P->k, P->kv_type, ko + d) * ks;", ": widen(P->k, P->kv_type, ko + d);"),
    ("value scale dropped", ": widen(P->v, P->kv_type, vo + d) * vs;", ": widen(P->v, P->kv_type, vo + d);"),
    ("key scale from value scales", "(double)P->k_scale[kv_row(P, P->ks_stride, b, hkv, j)]",
     "(double)P->v_scale[kv_row(P, P->ks_stride, b, hkv, j)]"),
    ("key scale strides", "P->k_scale[kv_row(P, P->ks_stride, b, hkv, j)]",
     "P->k_scale[kv_row(P, P->vs_stride, b, hkv, j)]"),
]

_CHILD = """
import json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins
failed = oracle_pins.run_all(oracle.Oracle({lib!r}))
print(json.dumps(failed))
"""


def _run_mutant(tmp, idx, find, repl):
    src = open(oracle.SOURCE).read()
    assert src.count(find) == 1, f"mutant anchor not found exactly once: {find!r}"
    path = os.path.join(tmp, f"m{idx}.c")
    with open(path, "w") as f:
        f.write(src.replace(find, repl))
    lib = os.path.join(tmp, f"libm{idx}.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", path, "-o", lib, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, tests=HERE, lib=lib)],
                       capture_output=True, text=True, timeout=300, env=env)
    if r.returncode != 0:
        return ["child exited with status %d" % r.returncode]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            futs = {name: ex.submit(_run_mutant, tmp, i, f, r) for i, (name, f, r) in enumerate(MUTANTS)}
            survivors = [name for name, fut in futs.items() if not fut.result()]
    assert not survivors, f"mutants no pin caught: {survivors}"


@pytest.mark.parametrize("name,find,repl", MUTANTS[:1])
def test_unmutated_copy_passes(name, find, repl):
    """Control: the same child-process harness on an unmodified copy reports no failure."""
    with tempfile.TemporaryDirectory() as tmp:
        assert _run_mutant(tmp, 0, find, find) == []
