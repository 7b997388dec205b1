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


def assert_matches_beyond_rounding(out, lse, ref_o, ref_l, dtype, what=""):
    """assert_matches for outputs of large magnitude: above |out| of about 2.5 the output's own
    bf16 rounding alone (half a spacing, 2^-9 relative) exceeds the absolute tolerance, so the
    tolerance applies to the error beyond that rounding."""
    tol_o, tol_l = TOL[dtype]
    assert torch.isfinite(out).all(), f"{what}: non-finite output"
    e_out, e_lse, mism, ref_max = errors(out, lse, ref_o, ref_l)
    o = out.double().cpu().numpy().reshape(ref_o.shape)
    half = bf16_half_ulp(ref_o) if dtype == torch.bfloat16 else np.zeros_like(ref_o)
    excess = float(np.max(np.abs(o - ref_o) - half, initial=0.0))
    say(f"  {what}: max|dout| {e_out:.3e} (max|out| {ref_max:.3f}), beyond output rounding {excess:.3e} "
        f"(tol {tol_o:g}), max|dlse| {e_lse:.3e} (tol {tol_l:g}), -inf mismatches {mism}")
    assert mism == 0, f"{what}: rows with no visible key disagree"
    assert excess <= tol_o, f"{what}: out error beyond rounding {excess} > {tol_o}"
    assert e_lse <= tol_l, f"{what}: lse error {e_lse} > {tol_l}"


def bf16_half_ulp(x):
    """Half the spacing of bf16 numbers at |x| (the most that rounding x to bf16 can move it)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))   # a = m * 2^e with m in [0.5, 1)
    return np.ldexp(1.0, e - 9)                     # ulp 2^(e - 8), half of it


# Regression bounds of the full-size workloads, next to the contract tolerances above: what the
# kernels reach, with room for box-to-box noise. lse: a key dropped from a 4096-key softmax moves
# the LSE by about 2.4e-4, which these bounds catch. out: the error beyond the output's own bf16
# rounding (at most half a bf16 spacing of the reference value), as a maximum, and the mean error
# against the mean of that half spacing: rounding to nearest even averages about half of it plus
# the rounding of P, truncation about all of it, so a bias shows in the mean.
TIGHT = {torch.float32: dict(lse=2e-6, excess=2e-6, mean_abs=1e-7),
         torch.bfloat16: dict(lse=1e-4, excess=2e-3, mean_rel=1.2, mean_abs=2e-5)}


def assert_tight(out, lse, ref_o, ref_l, dtype, what=""):
    """Contract tolerances (assert_matches), then the tighter regression bounds of TIGHT."""
    assert_matches(out, lse, ref_o, ref_l, dtype, what)
    o = out.double().cpu().numpy().reshape(ref_o.shape)
    l_ = lse.double().cpu().numpy().reshape(ref_l.shape)
    fin = np.isfinite(ref_l)
    e_lse = float(np.max(np.abs(l_[fin] - ref_l[fin]), initial=0.0))
    d = np.abs(o - ref_o)
    half = bf16_half_ulp(ref_o) if dtype == torch.bfloat16 else np.zeros_like(ref_o)
    excess = float(np.max(d - half, initial=0.0))
    mean = float(np.mean(d)) if d.size else 0.0
    b = TIGHT[dtype]
    mean_bound = b.get("mean_rel", 0.0) * (float(np.mean(half)) if d.size else 0.0) + b["mean_abs"]
    say(f"  {what} regression: max|dlse| {e_lse:.2e} (bound {b['lse']:g}), max error beyond output "
        f"rounding {excess:.2e} (bound {b['excess']:g}), mean|dout| {mean:.2e} (bound {mean_bound:.2e}; "
        f"mean half bf16 spacing {float(np.mean(half)) if d.size else 0.0:.2e})")
    assert e_lse <= b["lse"], f"{what}: lse error {e_lse} above the regression bound"
    assert excess <= b["excess"], f"{what}: out error beyond rounding {excess} above the regression bound"
    assert mean <= mean_bound, f"{what}: mean out error {mean} above the regression bound {mean_bound}"
