"""GPU tests of the longest-piece-first placement of the GQA partial passes (decode_unit_lpt).

Each work group ranks the (sequence, split) pieces from the lengths and takes the piece of its
rank, so the placement changes which group computes a piece, never what it computes: with the
placement forced on (AD_LPT=1) every output, LSE and partial slot must equal the grid order's
(AD_LPT=0) bit for bit, on all three GQA partial kernels, in one launch (merge inside, with the
arrival counters back at zero) and in two (every partial slot, empty ones included), and match
the oracle. The lengths cover empty sequences, one key, exact multiples of the split length, the
full key range and remainders of every size; the planner turns it on by itself only for grids of
more work groups than compute units, which the full-size ragged workloads are (their parity tests
run with it)."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KERNELS = {  # name: (AD_PARTIAL_KERNEL, AD_MFMA_TILE)
    "valu": ("valu", "16"),
    "mfma16": ("mfma", "16"),
    "mfma32": ("mfma", "32"),
}


def run(wg, S, fused, monkeypatch, lpt):
    monkeypatch.setenv("AD_LPT", "1" if lpt else "0")
    step = DecodeStep(wg, num_splits=S, fused=fused)
    out, lse = step()
    torch.cuda.synchronize()
    parts = None if fused else (step.part_o.cpu(), step.part_lse.cpu())
    counters = int(step.workspace[:1 << 20].count_nonzero()) if fused else 0
    return out.cpu(), lse.cpu(), parts, counters


def bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


LENS = [0, 1, 512, 300, 1024, 513, 37, 0, 1023, 777, 256, 1000]  # kv_len_max 1024


@pytest.mark.parametrize("kernel", sorted(KERNELS))
@pytest.mark.parametrize("kind", ["contiguous", "paged"])
@pytest.mark.parametrize("S", [1, 2, 3, 4, 7])
def test_placement_changes_nothing(orc, monkeypatch, kernel, kind, S):
    monkeypatch.setenv("AD_PARTIAL_KERNEL", KERNELS[kernel][0])
    monkeypatch.setenv("AD_MFMA_TILE", KERNELS[kernel][1])
    say(f"[gpu] placement {kernel} {kind} S={S}")
    common = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, seed=2100 + S, causal=True, window=700)
    if kind == "contiguous":
        w = inputs.contiguous(batch=len(LENS), kv_len=1024, seq_lens=LENS, **common)
    else:
        w = inputs.paged(seq_lens=LENS, page_size=16, poison=True, **common)
    wg = w.to("cuda")
    ref_o, ref_l = oracle_of(orc, w)
    for fused in (True, False):
        o0, l0, p0, c0 = run(wg, S, fused, monkeypatch, lpt=False)
        o1, l1, p1, c1 = run(wg, S, fused, monkeypatch, lpt=True)
        assert torch.equal(bits(o0), bits(o1)) and torch.equal(l0, l1), f"fused={fused}: outputs differ"
        if fused:
            assert c0 == 0 and c1 == 0, "arrival counters not back to zero"
        else:
            assert torch.equal(p0[0], p1[0]) and torch.equal(p0[1], p1[1]), "partial slots differ"
        assert_matches(o1, l1, ref_o, ref_l, w.dtype, f"fused={fused}")


@pytest.mark.parametrize("kernel", ["valu", "mfma16", "mfma16rows"])
def test_placement_fp8_int4_and_drafts(orc, monkeypatch, kernel):
    """Quantised caches and packed draft tokens with tree masks, placement forced on and off."""
    monkeypatch.setenv("AD_PARTIAL_KERNEL", KERNELS[kernel[:6]][0])
    monkeypatch.setenv("AD_MFMA_TILE", KERNELS[kernel[:6]][1])
    monkeypatch.setenv("AD_MFMA_ROWS", "1" if kernel.endswith("rows") else "0")
    lens = [300, 45, 0, 129, 1024, 1, 640]
    for fmt in ("fp8", "int4"):
        say(f"[gpu] placement {kernel} {fmt}")
        w = inputs.paged(seq_lens=lens, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, seed=2200,
                         kv_format=fmt, poison=True)
        wg = w.to("cuda")
        ref_o, ref_l = oracle_of(orc, w)
        o0, l0, _, _ = run(wg, 3, True, monkeypatch, lpt=False)
        o1, l1, _, c1 = run(wg, 3, True, monkeypatch, lpt=True)
        assert torch.equal(bits(o0), bits(o1)) and torch.equal(l0, l1) and c1 == 0
        assert_matches(o1, l1, ref_o, ref_l, torch.bfloat16, fmt)
    base = inputs.paged(seq_lens=lens, num_q_heads=8, num_kv_heads=2, head_dim=128, q_len=5, page_size=16,
                        seed=2201, poison=True)
    w = inputs.with_spec(base, counts=[5, 2, 0, 4, 1, 3, 5], tree=True, seed=8)
    wg = w.to("cuda")
    ref_o, ref_l = oracle_of(orc, w)
    o0, l0, _, _ = run(wg, 2, True, monkeypatch, lpt=False)
    o1, l1, _, c1 = run(wg, 2, True, monkeypatch, lpt=True)
    assert torch.equal(bits(o0), bits(o1)) and torch.equal(l0, l1) and c1 == 0
    assert_matches(o1, l1, ref_o, ref_l, torch.bfloat16, "drafts")


@pytest.mark.parametrize("batch", [256, 257])
def test_placement_at_the_batch_limit(orc, monkeypatch, batch):
    """256 sequences is the most the placement ranks (one thread per sequence); 257 runs in grid
    order even when asked. Both match the oracle on sampled rows."""
    g = torch.Generator().manual_seed(batch)
    lens = torch.randint(0, 300, (batch,), generator=g).tolist()
    say(f"[gpu] placement with {batch} sequences")
    w = inputs.paged(seq_lens=lens, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, seed=2300)
    wg = w.to("cuda")
    o0, l0, _, _ = run(wg, 2, True, monkeypatch, lpt=False)
    o1, l1, _, c1 = run(wg, 2, True, monkeypatch, lpt=True)
    assert torch.equal(bits(o0), bits(o1)) and torch.equal(l0, l1) and c1 == 0
    rows = list(range(0, batch * 4, 37))
    ref_o, ref_l = oracle_of(orc, w, rows=rows)
    assert_matches(o1.reshape(-1, 64)[rows], l1.reshape(-1)[rows], ref_o, ref_l, w.dtype, "sampled rows")
