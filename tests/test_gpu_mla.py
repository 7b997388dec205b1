"""GPU parity of multi-head latent attention (shared latent KV head: 512 latent + 64 rotary
dims, values = the latent row) against the fp64 oracle on the same seeded inputs, through the
C ABI entry point attn_decode_mla."""
import numpy as np
import pytest
import torch

from attention_decode_amd import _abi, inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_matches_beyond_rounding, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run(w_cpu, num_splits=None):
    wg = w_cpu.to("cuda")
    step = DecodeStep(wg, num_splits=num_splits)
    out, lse = step()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), step


def flat_rows(w):
    return w.batch * w.q_len * w.num_q_heads


def test_workload5_every_row(orc):
    """Full size (32 sequences x 128 heads x 8192 keys, page 64): all 4096 rows against the oracle."""
    say("[gpu] workload 5 (MLA) full size, every row")
    w = inputs.make(5)
    out, lse, step = run(w)
    say(f"  splits {step.splits}")
    ref_o, ref_l = oracle_of(orc, w)
    assert_tight(out, lse, ref_o, ref_l, w.dtype, f"workload 5, {flat_rows(w)} rows")


def chunk_of(w, S):
    """Keys per split of a forced split count: ceil(kv_len_max / S) rounded up to 16."""
    return -(-(-(-w.kv_len_max // S)) // 16) * 16


def mla_partials(w_cpu, S):
    wg = w_cpu.to("cuda")
    step = DecodeStep(wg, num_splits=S)
    B, Q, H = w_cpu.batch, w_cpu.q_len, w_cpu.num_q_heads
    po = torch.full((B, Q, H, S, 512), float("nan"), device="cuda")
    pl = torch.full((B, Q, H, S), float("nan"), device="cuda")
    _abi.attn_decode_mla_splitkv(step.args, wg.kpe, wg.q_pe, step.paged, S, po, pl)
    torch.cuda.synchronize()
    return po.cpu(), pl.cpu()


def test_mla_splitkv_partials_small(orc):
    """attn_decode_mla_splitkv writes every (row, split) slot: each equals the oracle restricted to
    the split's key range, and splits past a short sequence's end hold (0, -inf)."""
    lens = [1, 700, 64, 333]
    S = 3
    say(f"[gpu] mla split partials, lens {lens}, S={S}")
    w = inputs.mla(batch=len(lens), num_heads=64, kv_len=max(lens), page_size=16, seq_lens=lens, q_len=2,
                   causal=True, seed=81)
    po, pl = mla_partials(w, S)
    c = chunk_of(w, S)
    for s in range(S):
        ref_o, ref_l = oracle_of(orc, w, key_range=(s * c, (s + 1) * c))
        assert_matches(po[:, :, :, s], pl[:, :, :, s], ref_o, ref_l, w.dtype, f"split {s} of {c} keys")


def test_workload5_partials_sampled_rows(orc):
    """Workload 5 in 8 splits of 1024 keys (twice the planner's count, so more split boundaries),
    written by attn_decode_mla_splitkv: every split of the heads of sequences 0 and 31 and 64
    random rows, against the oracle on each key range."""
    say("[gpu] workload 5 split partials, sampled rows")
    w = inputs.make(5)
    S = 8
    po, pl = mla_partials(w, S)
    c = chunk_of(w, S)
    H = w.num_q_heads
    g = torch.Generator().manual_seed(82)
    rows = sorted(set(list(range(H)) + list(range(31 * H, 32 * H)) +
                      torch.randint(0, flat_rows(w), (64,), generator=g).tolist()))
    for s in range(S):
        ref_o, ref_l = oracle_of(orc, w, rows=rows, key_range=(s * c, (s + 1) * c))
        o = po[:, :, :, s].reshape(-1, 512)[rows]
        l_ = pl[:, :, :, s].reshape(-1)[rows]
        assert_matches(o, l_, ref_o, ref_l, w.dtype, f"split {s}")


def test_workload5_poisoned_bit_identical():
    say("[gpu] workload 5 clean vs poisoned pool")
    a = run(inputs.make(5))
    b = run(inputs.make(5, poison=True))
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


CASES = [  # (heads, page, lens, q_len, causal, window)
    (128, 64, [1, 31, 33, 700], 1, False, 0),
    (128, 16, [64, 1000, 5], 1, False, 0),
    (16, 32, [300, 2], 1, False, 0),
    (160, 64, [257, 90], 1, False, 0),       # two row blocks, the second partly empty
    (64, 16, [500, 77], 2, True, 0),         # two query tokens, causal
    (32, 64, [640, 129], 3, True, 200),      # three query tokens, causal + window
]


@pytest.mark.parametrize("H,page,lens,Q,causal,window", CASES, ids=lambda x: str(x))
def test_mla_small(orc, H, page, lens, Q, causal, window):
    say(f"[gpu] mla H={H} page={page} lens={lens} Q={Q} causal={causal} window={window}")
    w = inputs.mla(batch=len(lens), num_heads=H, kv_len=max(lens), page_size=page, seq_lens=lens, q_len=Q,
                   causal=causal, window=window, seed=700 + H + page + Q)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, w.dtype, f"S={S}")


def test_mla_poisoned_small_bit_identical():
    lens = [5, 64, 250, 1000, 31]
    say("[gpu] mla poisoned small pool")
    kw = dict(batch=len(lens), num_heads=128, kv_len=1000, page_size=16, seq_lens=lens, seed=9)
    a = run(inputs.mla(**kw), num_splits=4)
    b = run(inputs.mla(**kw, poison=True), num_splits=4)
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_mla_score_far_above_first_tile(orc):
    """A late key scores ~110 (natural log units) above the rest: far beyond what a reference max
    fixed at the first tile may absorb, so the unit is recomputed exactly with each row's true
    max. The result still equals the oracle (dominated by that key)."""
    say("[gpu] mla: score far above the first tile's max")
    lens = [300, 300]
    w = inputs.mla(batch=2, num_heads=32, kv_len=300, page_size=16, seq_lens=lens, seed=11)
    u = w.storage["q"][0, 0, 0].clone()
    w.storage["q"][0, 0, :] = u                      # every head of sequence 0 queries along u
    j0 = 250
    page = int(w.block_table[0, j0 // 16])
    w.storage["ckv"][page, j0 % 16, 0] = (3.0 * u.float()).to(w.dtype)
    ref_o, ref_l = oracle_of(orc, w)
    assert np.min(ref_l.reshape(2, 32)[0]) > 60       # the key really dominates sequence 0
    out, lse, _ = run(w, num_splits=1)
    assert_matches(out, lse, ref_o, ref_l, w.dtype, "far score")


@pytest.mark.parametrize("head", [5, 27])
def test_mla_score_far_above_first_tile_one_row(orc, head):
    """As above, but only one query head sees the far key: the work group must still notice that a
    single row (held by lanes other than the first of its waves) went past its reference max, and
    recompute (a vote taken by one lane alone left that row's output NaN). Other heads see the
    far key's large value row with moderate weight, so outputs reach about 8.3, where bf16's own
    rounding is 0.03: the tolerance applies beyond that rounding."""
    say(f"[gpu] mla: one row ({head}) far above its first tile's max")
    lens = [300, 300]
    w = inputs.mla(batch=2, num_heads=32, kv_len=300, page_size=16, seq_lens=lens, seed=12)
    u = w.storage["q"][0, 0, head].clone()
    j0 = 250
    page = int(w.block_table[0, j0 // 16])
    w.storage["ckv"][page, j0 % 16, 0] = (3.0 * u.float()).to(w.dtype)
    ref_o, ref_l = oracle_of(orc, w)
    lse0 = ref_l.reshape(2, 32)[0]
    assert lse0[head] > 60 and np.delete(lse0, head).max() < 30  # only that row is dominated
    out, lse, _ = run(w, num_splits=1)
    assert_matches_beyond_rounding(out, lse, ref_o, ref_l, w.dtype, f"far score on head {head}")


def test_mla_far_score_with_masks_and_splits(orc):
    """The exact recompute under a causal sliding window with two query tokens and three splits:
    one head of the first token sees the far key (in the last split, inside both tokens' windows);
    the split holding it recomputes, with the rows the window hides from part of the split kept
    at probability 0, and the merge weighs it against the other splits."""
    say("[gpu] mla: far score under causal + window, 2 tokens, 3 splits")
    lens = [300, 260]
    w = inputs.mla(batch=2, num_heads=32, kv_len=300, page_size=16, seq_lens=lens, q_len=2, causal=True,
                   window=200, seed=14)
    head = 9
    u = w.storage["q"][0, 0, head].clone()
    j0 = 250
    page = int(w.block_table[0, j0 // 16])
    w.storage["ckv"][page, j0 % 16, 0] = (3.0 * u.float()).to(w.dtype)
    ref_o, ref_l = oracle_of(orc, w)
    lse = ref_l.reshape(2, 2, 32)
    assert lse[0, 0, head] > 60 and np.delete(lse[0, 0], head).max() < 30
    out, lse_, _ = run(w, num_splits=3)
    assert_matches_beyond_rounding(out, lse_, ref_o, ref_l, w.dtype, "far score, masked, 3 splits")


def test_mla_split_invariance():
    say("[gpu] mla split invariance")
    w = inputs.mla(batch=2, num_heads=128, kv_len=3000, page_size=64, seq_lens=[3000, 1777], seed=13)
    outs = [(S,) + run(w, num_splits=S)[:2] for S in (1, 2, 5, 8)]
    o0, l0 = outs[0][1].double(), outs[0][2].double()
    # Each result carries bf16 rounding of P (2^-9 relative on every weight) and of the output; the
    # worst element of either stays inside the oracle tolerance, and the mean difference is
    # rounding noise (a systematic error, e.g. a mishandled split boundary, moves the mean).
    for S, o, l_ in outs[1:]:
        d = (o.double() - o0).abs()
        assert float(d.max()) <= 1e-2 and float(d.mean()) <= 3e-4, f"S={S}: max {float(d.max())} mean {float(d.mean())}"
        assert (l_.double() - l0).abs().max() <= 1e-4, f"S={S}"
