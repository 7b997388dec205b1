"""GPU tests of the C ABI's entry points as a caller uses them: attn_decode_paged called directly,
the split planner's choice per workload (plan only, no launch), caches whose lengths are not
given (seq_lens = NULL), and the public merge with per-sequence split counts. Every result is
compared with the fp64 oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

from attention_decode_amd import _abi, inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def test_paged_entry_point_workload3(orc):
    """attn_decode_paged on the full paged workload (64 ragged sequences, page 16): every row
    against the oracle, and bit for bit what attn_decode gives for the same arguments."""
    say("[gpu] attn_decode_paged, workload 3 full size")
    w = inputs.make(3).to("cuda")
    step = DecodeStep(w)
    ws = torch.zeros(_abi.attn_decode_workspace_size(step.args, step.paged, 0), dtype=torch.uint8, device="cuda")
    _abi.attn_decode_paged(step.args, step.paged, 0, ws)
    torch.cuda.synchronize()
    out, lse = step.out.cpu().clone(), step.lse.cpu().clone()
    assert int(ws[:1 << 20].count_nonzero()) == 0, "arrival counters not left at zero"
    step()
    torch.cuda.synchronize()
    assert torch.equal(out, step.out.cpu()) and torch.equal(lse, step.lse.cpu())
    ref_o, ref_l = oracle_of(orc, inputs.make(3))
    assert_tight(out, lse, ref_o, ref_l, w.dtype, "attn_decode_paged workload 3")


@pytest.mark.parametrize("S", [1, 3])
def test_paged_entry_point_small(orc, S):
    lens = [1, 15, 16, 17, 250, 0, 33]
    say(f"[gpu] attn_decode_paged small, S={S}")
    w = inputs.paged(seq_lens=lens, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, seed=41)
    wg = w.to("cuda")
    step = DecodeStep(wg, num_splits=S)
    ws = torch.zeros(_abi.attn_decode_workspace_size(step.args, step.paged, S), dtype=torch.uint8, device="cuda")
    _abi.attn_decode_paged(step.args, step.paged, S, ws)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_of(orc, w)
    assert_matches(step.out.cpu(), step.lse.cpu(), ref_o, ref_l, w.dtype, f"paged entry S={S}")


# The planner's choice (splits, keys per split) for the workloads on a 256-compute-unit MI355X.
PLANS = {1: (4, 128), 2: (2, 2048), 3: (5, 1648), 4: (4, 1056), 5: (4, 2048), 6: (3, 2736),
         7: (2, 4096), 8: (3, 2736)}


@pytest.mark.parametrize("config", sorted(PLANS))
def test_planner_choice(config):
    """attn_decode_plan gives the same (splits, chunk) as when the bounds of its heuristic were
    measured; a change to the heuristic shows up here."""
    w = inputs.make(config).to("cuda")
    step = DecodeStep(w)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"the plans are those of a 256-compute-unit part ({cus} here)")
    S, chunk = _abi.attn_decode_plan(step.args, step.paged, step.sparse)
    if w.num_splits:
        S = w.num_splits
        chunk = -(-(-(-w.kv_len_max // S)) // 16) * 16
    say(f"[gpu] plan of workload {config}: {S} x {chunk}")
    assert (S, chunk) == PLANS[config]


def test_planner_long_paged_cache_without_lengths():
    """seq_lens = NULL on a long cache of small pages: the planner raises the split count until a
    split's pages fit the map it stages (plan only; no kernel runs)."""
    B, Hq, Hkv, D, page, L = 16, 32, 8, 128, 16, 65536
    q = torch.zeros(B, 1, Hq, D, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(8, Hkv, page, D, dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    bt = torch.zeros(B, L // page, dtype=torch.int32, device="cuda")
    a = _abi.make_args(q, pool, pool, scale=0.1, kv_len_max=L, out=torch.zeros_like(q))
    pg = _abi.make_paged(bt, page)
    S, chunk = _abi.attn_decode_plan(a, pg, None)
    say(f"[gpu] plan for {B} x {L} keys, page {page}, no lengths: {S} x {chunk}")
    assert -(-chunk // page) + 2 <= 1040 and S * chunk >= L
    assert _abi.attn_decode_workspace_size(a, pg, 0) > 0


@pytest.mark.parametrize("kind", ["contiguous", "paged"])
@pytest.mark.parametrize("S", [0, 1, 3])
def test_lengths_not_given(orc, kind, S):
    """seq_lens = NULL: every sequence has kv_len_max keys, and the result equals the oracle's with
    those lengths."""
    say(f"[gpu] seq_lens NULL, {kind}, S={S}")
    if kind == "contiguous":
        w = inputs.contiguous(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128, kv_len=700, q_len=2,
                              seed=51, causal=True)
    else:
        w = inputs.paged(seq_lens=[640, 640, 640], num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=32,
                         seed=52)
    w.lens_given = False
    ref_o, ref_l = oracle_of(orc, w)
    step = DecodeStep(w.to("cuda"), num_splits=S or None)
    out, lse = step()
    torch.cuda.synchronize()
    assert_matches(out.cpu(), lse.cpu(), ref_o, ref_l, w.dtype, f"{kind} without lengths, S={step.splits}")


def test_merge_with_splits_per_batch(orc):
    """The public merge with a count of splits per sequence: slots past a sequence's count hold NaN
    and are never read; each row equals the oracle's merge of its leading slots; a count of 0 gives
    (0, -inf); counts above num_splits are clamped."""
    say("[gpu] merge with splits_per_batch")
    g = torch.Generator().manual_seed(61)
    B, Q, Hq, S, Dv = 5, 2, 4, 6, 128
    po = torch.randn(B, Q, Hq, S, Dv, generator=g)
    pl = torch.randn(B, Q, Hq, S, generator=g) * 3
    counts = [0, 1, 3, 6, 9]
    for b, c in enumerate(counts):
        po[b, :, :, min(c, S):] = float("nan")
        pl[b, :, :, min(c, S):] = float("nan")
    ref_o = np.zeros((B, Q, Hq, Dv))
    ref_l = np.full((B, Q, Hq), -math.inf)
    for b, c in enumerate(counts):
        c = min(c, S)
        if c:
            o, l_ = orc.merge(po[b, :, :, :c].reshape(-1, c, Dv).double().numpy(),
                              pl[b, :, :, :c].reshape(-1, c).double().numpy())
            ref_o[b], ref_l[b] = o.reshape(Q, Hq, Dv), l_.reshape(Q, Hq)
    spb = torch.tensor(counts, dtype=torch.int32, device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        out = torch.full((B, Q, Hq, Dv), 7.0, device="cuda", dtype=dt)
        lse = torch.empty(B, Q, Hq, device="cuda")
        _abi.attn_decode_merge(po.cuda(), pl.cuda(), S, out, lse, splits_per_batch=spb)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        tol = 1e-6 if dt == torch.float32 else 1e-2
        assert np.max(np.abs(out.double().cpu().numpy() - ref_o)) <= tol
        lr = lse.double().cpu().numpy()
        assert np.array_equal(np.isneginf(lr), np.isneginf(ref_l))
        fin = np.isfinite(ref_l)
        assert np.max(np.abs(lr[fin] - ref_l[fin])) <= 1e-5


def test_public_two_pass_ragged_merge(orc):
    """The public two-pass path on a ragged paged batch: attn_decode_splitkv writes every slot, the
    slots past each sequence's last non-empty split are then overwritten with NaN, and
    attn_decode_merge with splits_per_batch = ceil(L_b / chunk) reproduces the oracle."""
    lens = [5, 700, 33, 1500, 0]
    S = 4
    say(f"[gpu] two-pass ragged merge, lens {lens}, S={S}")
    w = inputs.paged(seq_lens=lens, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, seed=62)
    wg = w.to("cuda")
    step = DecodeStep(wg, num_splits=S, fused=False)
    _abi.attn_decode_splitkv(step.args, step.paged, None, S, step.part_o, step.part_lse)
    chunk = -(-(-(-w.kv_len_max // S)) // 16) * 16
    counts = [-(-L // chunk) for L in lens]
    for b, c in enumerate(counts):
        step.part_o[b, :, :, c:] = float("nan")
        step.part_lse[b, :, :, c:] = float("nan")
    spb = torch.tensor(counts, dtype=torch.int32, device="cuda")
    _abi.attn_decode_merge(step.part_o, step.part_lse, S, step.out, step.lse, splits_per_batch=spb)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_of(orc, w)
    assert_matches(step.out.cpu(), step.lse.cpu(), ref_o, ref_l, w.dtype, "ragged two-pass")


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 64 << 20])
def test_read_probe_reads_every_word_once(nbytes):
    """The streaming probe reads each 16-byte piece exactly once: the XOR of the words it writes
    equals the XOR of every 32-bit word of the buffer."""
    say(f"[gpu] read probe over {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes % 1000)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    sink = torch.zeros(_abi.AD_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    _abi.attn_decode_read_probe(src.cuda(), sink)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(src.numpy().view(np.uint32)))
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    assert got == want
