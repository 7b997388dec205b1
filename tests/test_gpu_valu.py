"""GPU parity of the VALU split-KV path (<= 8 query rows per KV head) and the merge kernel,
against the fp64 oracle on the same seeded inputs, through the C ABI."""
import math

import numpy as np
import pytest
import torch

from attention_decode_amd import _abi, inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run(w_cpu, num_splits=None):
    wg = w_cpu.to("cuda")
    step = DecodeStep(wg, num_splits=num_splits)
    out, lse = step()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), step


# ------------------------------------------------------------------------------ full workloads
@pytest.mark.parametrize("config", [1, 2, 3])
def test_workload_full(orc, config):
    say(f"[gpu] workload {config}: full size, every row")
    w = inputs.make(config)
    out, lse, step = run(w)
    say(f"  splits {step.splits}")
    ref_o, ref_l = oracle_of(orc, w)
    assert_tight(out, lse, ref_o, ref_l, w.dtype, f"workload {config}")


def test_workload1_partials(orc):
    """The tiny fp32 workload forces 4 splits of 128 keys: every partial (o_s, lse_s) equals the
    oracle restricted to that key range."""
    say("[gpu] workload 1 partials")
    w = inputs.make(1)
    wg = w.to("cuda")
    step = DecodeStep(wg, fused=False)
    assert step.splits == 4
    step()
    torch.cuda.synchronize()
    po, pl = step.part_o.cpu(), step.part_lse.cpu()
    for s in range(4):
        ref_o, ref_l = oracle_of(orc, w, key_range=(128 * s, 128 * (s + 1)))
        assert_matches(po[:, :, :, s], pl[:, :, :, s], ref_o, ref_l, w.dtype, f"split {s}")


# ------------------------------------------------------------------------------ small cases
SMALL = []
for dtype in (torch.float32, torch.bfloat16):
    for D in (64, 128):
        for G, Q in ((1, 1), (2, 1), (4, 1), (8, 1), (2, 2), (4, 2), (1, 3)):
            SMALL.append((dtype, D, G, Q))


@pytest.mark.parametrize("dtype,D,G,Q", SMALL, ids=lambda x: str(x).replace("torch.", ""))
@pytest.mark.parametrize("mask", ["none", "causal", "causal_window", "window"])
def test_contiguous_small(orc, dtype, D, G, Q, mask):
    causal = mask.startswith("causal")
    window = 37 if "window" in mask else 0
    lens = [300, 1, 37, 0, 129]
    say(f"[gpu] contiguous {dtype} D={D} G={G} Q={Q} mask={mask} lens={lens}")
    Hkv = 2
    w = inputs.contiguous(batch=len(lens), num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, kv_len=300,
                          q_len=Q, dtype=dtype, seed=D * 100 + G * 10 + Q, seq_lens=lens, causal=causal,
                          window=window)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3, 7):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, dtype, f"S={S}")


@pytest.mark.parametrize("page_size", [16, 32, 64])
@pytest.mark.parametrize("dtype,G", [(torch.bfloat16, 4), (torch.float32, 1), (torch.bfloat16, 8)])
def test_paged_small(orc, page_size, dtype, G):
    lens = [1, 15, 16, 17, 250, 700, 0, 33]
    say(f"[gpu] paged page={page_size} {dtype} G={G} lens={lens}")
    w = inputs.paged(seq_lens=lens, num_q_heads=2 * G, num_kv_heads=2, head_dim=128, page_size=page_size,
                     dtype=dtype, seed=page_size + G)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (0, 1, 5):
        out, lse, step = run(w, num_splits=S or None)
        assert_matches(out, lse, ref_o, ref_l, dtype, f"S={step.splits}")


def test_paged_causal_window_two_queries(orc):
    lens = [64, 1000, 513]
    say(f"[gpu] paged Q=2 causal window lens={lens}")
    w = inputs.paged(seq_lens=lens, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, q_len=2,
                     dtype=torch.bfloat16, seed=5, causal=True, window=100)
    ref_o, ref_l = oracle_of(orc, w)
    out, lse, _ = run(w, num_splits=3)
    assert_matches(out, lse, ref_o, ref_l, w.dtype, "paged causal window")


# ------------------------------------------------------------------------------ structure
def test_split_invariance():
    """Different split counts agree with each other (and the oracle) on the GPU workload shape."""
    say("[gpu] split invariance, GQA contiguous 4 x 2048")
    w = inputs.contiguous(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_len=2048, seed=77)
    outs = []
    for S in (1, 2, 3, 4, 7, 16):
        out, lse, _ = run(w, num_splits=S)
        outs.append((S, out.double(), lse.double()))
    o0, l0 = outs[0][1], outs[0][2]
    for S, o, l_ in outs[1:]:
        assert (o - o0).abs().max() <= 2e-3, f"S={S}"
        assert (l_ - l0).abs().max() <= 1e-4, f"S={S}"


def test_poisoned_pool_is_bit_identical():
    """Unreferenced pages, tail slots past each sequence and table padding hold NaN, and the pool is
    permuted differently: the result must be finite and bit-identical to the clean run (the work
    decomposition depends only on logical positions)."""
    lens = [5, 16, 250, 1000, 4097, 31]
    say("[gpu] poisoned paged pool")
    clean = inputs.paged(seq_lens=lens, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, seed=9)
    dirty = inputs.paged(seq_lens=lens, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, seed=9,
                         poison=True)
    assert torch.isnan(dirty.k).any()
    a = run(clean, num_splits=4)
    b = run(dirty, num_splits=4)
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_workload3_poisoned_bit_identical():
    say("[gpu] workload 3 clean vs poisoned")
    a = run(inputs.make(3))
    b = run(inputs.make(3, poison=True))
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_deterministic():
    say("[gpu] determinism, workload 2")
    w = inputs.make(2).to("cuda")
    step = DecodeStep(w)
    o1, l1 = (t.clone() for t in step())
    o2, l2 = step()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_and_degenerate(orc):
    say("[gpu] empty sequences, kv_len_max 0, batch 0")
    w = inputs.contiguous(batch=3, num_q_heads=4, num_kv_heads=1, head_dim=64, kv_len=8, seed=3,
                          seq_lens=[0, 0, 0])
    out, lse, _ = run(w, num_splits=2)
    assert torch.all(out == 0) and torch.all(lse == -math.inf)
    wp = inputs.paged(seq_lens=[0, 3], num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=16, seed=4)
    out, lse, _ = run(wp)
    ref_o, ref_l = oracle_of(orc, wp)
    assert_matches(out, lse, ref_o, ref_l, wp.dtype, "paged with an empty sequence")
    # kv_len_max = 0: every row is empty
    q = torch.randn(2, 1, 4, 128, device="cuda").to(torch.bfloat16)
    kv = torch.zeros(2, 1, 1, 128, device="cuda", dtype=torch.bfloat16)
    out = torch.full((2, 1, 4, 128), 7.0, device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros(2, 1, 4, device="cuda")
    a = _abi.make_args(q, kv, kv, scale=0.1, kv_len_max=0, out=out, lse=lse)
    po = torch.empty(2, 1, 4, 2, 128, device="cuda")
    pl = torch.empty(2, 1, 4, 2, device="cuda")
    _abi.attn_decode_splitkv(a, None, None, 2, po, pl)
    _abi.attn_decode_merge(po, pl, 2, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == -math.inf)
    # batch 0: nothing enqueued, success
    a0 = _abi.make_args(q[:0], kv[:0], kv[:0], scale=0.1, kv_len_max=1, out=out[:0], lse=lse[:0])
    _abi.attn_decode_splitkv(a0, None, None, 2, po, pl)


def test_merge_kernel_against_oracle(orc):
    """The merge alone on random partials with -inf slots, fp32 and bf16 outputs, strided out."""
    say("[gpu] merge kernel")
    g = torch.Generator().manual_seed(31)
    B, Q, Hq, S, Dv = 3, 2, 4, 6, 128
    po = torch.randn(B, Q, Hq, S, Dv, generator=g)
    pl = torch.randn(B, Q, Hq, S, generator=g) * 3
    pl[0, 0, 0, :] = -math.inf
    pl[1, :, :, 2] = -math.inf
    po[1, :, :, 2] = 0
    ref_o, ref_l = orc.merge(po.reshape(-1, S, Dv).double().numpy(), pl.reshape(-1, S).double().numpy())
    for dt in (torch.float32, torch.bfloat16):
        big = torch.zeros(B, Q, Hq + 4, Dv, device="cuda", dtype=dt)
        out = big[:, :, 2:2 + Hq]
        lse = torch.empty(B, Q, Hq, device="cuda")
        _abi.attn_decode_merge(po.cuda(), pl.cuda(), S, out, lse)
        torch.cuda.synchronize()
        tol = 1e-6 if dt == torch.float32 else 1e-2
        o = out.double().cpu().numpy().reshape(-1, Dv)
        assert np.max(np.abs(o - ref_o)) <= tol
        lr = lse.double().cpu().numpy().reshape(-1)
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isneginf(lr), np.isneginf(ref_l))
        assert np.max(np.abs(lr[fin] - ref_l[fin])) <= 1e-5
        assert torch.all(big[:, :, :2] == 0) and torch.all(big[:, :, 2 + Hq:] == 0)
