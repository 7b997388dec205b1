"""Helpers for the GPU parity tests: run a workload through the HIP library and through the
oracle on the same seeded inputs, and compare to the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances (max absolute error against the fp64 oracle): fp32 inputs 1e-5 on out and lse;
# bf16 inputs with fp32 accumulation 1e-2 on out and 1e-3 on lse.
TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (1e-2, 1e-3)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_available():
    return torch.cuda.is_available()


def oracle_of(orc, w, rows=None, key_range=None):
    """Oracle result for a CPU workload (all rows, or the flat row indices given)."""
    kw = dict(scale=w.scale, seq_lens=w.seq_lens, causal=w.causal, window=w.window, rows=rows,
              key_range=key_range)
    if w.kv_format == "fp8":
        kw.update(k_scale=w.k_scale, v_scale=w.v_scale)
    if w.kv_format == "int4":
        kw.update(int4_groups=w.kv_groups)
    if w.q_starts is not None:
        kw.update(q_starts=w.q_starts, q_len=w.q_len)
    if w.tree_mask is not None:
        kw.update(tree_mask=w.tree_mask)
    if w.kind == "contiguous":
        if w.num_blocks is not None:
            kw.update(num_blocks=w.num_blocks, block_idx=w.block_idx, block_size=w.block_size)
        return orc.attend(w.q, w.k, w.v, **kw)
    kw.update(block_table=w.block_table, page_size=w.page_size)
    if w.kind == "paged":
        return orc.attend(w.q, w.k, w.v, **kw)
    return orc.attend(w.q, w.k, w.k, q2=w.q_pe, k2=w.kpe, **kw)


def errors(out, lse, ref_o, ref_l):
    """(max |out - ref|, max |lse - ref| over rows with finite lse, rows where exactly one side is
    -inf, max |ref out|)."""
    o = out.double().cpu().numpy().reshape(ref_o.shape)
    l_ = lse.double().cpu().numpy().reshape(ref_l.shape)
    e_out = float(np.max(np.abs(o - ref_o), initial=0.0))
    both = np.isfinite(ref_l) & np.isfinite(l_)
    e_lse = float(np.max(np.abs(l_[both] - ref_l[both]), initial=0.0))
    inf_mismatch = int(np.sum(np.isneginf(ref_l) != np.isneginf(l_)))
    return e_out, e_lse, inf_mismatch, float(np.max(np.abs(ref_o), initial=0.0))


def assert_matches(out, lse, ref_o, ref_l, dtype, what=""):
    tol_o, tol_l = TOL[dtype]
    assert torch.isfinite(out).all(), f"{what}: non-finite output"
    e_out, e_lse, mism, ref_max = errors(out, lse, ref_o, ref_l)
    say(f"  {what}: max|dout| {e_out:.3e} (tol {tol_o:g}, max|out| {ref_max:.3f}), "
        f"max|dlse| {e_lse:.3e} (tol {tol_l:g}), -inf mismatches {mism}")
    assert mism == 0, f"{what}: rows with no visible key disagree"
    assert e_out <= tol_o, f"{what}: out error {e_out} > {tol_o}"
    assert e_lse <= tol_l, f"{what}: lse error {e_lse} > {tol_l}"
