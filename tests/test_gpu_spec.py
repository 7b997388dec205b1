"""GPU parity of speculative decoding -- packed variable-length queries (q_starts) and tree masks
over each sequence's draft tokens -- against the fp64 oracle on the same seeded inputs, through
the C ABI: contiguous, paged and block-sparse caches, both partial kernels, one or two words of
mask per token row, sequences without queries, and the identities a mask must satisfy."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# mfma: 32-row matrix-core units, mfma_rows: their whole-row load form, mfma16: 16-row units
KERNELS = ["valu", "mfma", "mfma_rows", "mfma16"]


def force(monkeypatch, kernel):
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "valu" if kernel == "valu" else "mfma")
    monkeypatch.setenv("AD_MFMA_ROWS", "1" if kernel == "mfma_rows" else "0")
    monkeypatch.setenv("AD_MFMA_TILE", "16" if kernel == "mfma16" else "32")


def run(w, num_splits=None):
    step = DecodeStep(w.to("cuda"), num_splits=num_splits)
    out, lse = step()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), step


def bits_equal(a, b):
    return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_workload7_full(orc):
    say("[gpu] workload 7 (paged, 1-8 drafts per sequence, token trees): full size, every row")
    w = inputs.make(7)
    out, lse, step = run(w)
    say(f"  splits {step.splits}, tokens {w.q.shape[0]}")
    ref_o, ref_l = oracle_of(orc, w)
    assert_tight(out, lse, ref_o, ref_l, torch.bfloat16, "workload 7")


def test_workload7_poisoned_bit_identical():
    """NaN in unreferenced pages and tail slots changes nothing, bit for bit."""
    say("[gpu] workload 7 poisoned pool")
    a = run(inputs.make(7))
    b = run(inputs.make(7, poison=True))
    assert bits_equal(a, b)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("kind", ["contiguous", "paged", "sparse"])
@pytest.mark.parametrize("G,Q", [(1, 3), (4, 2), (8, 4), (2, 40)])
@pytest.mark.parametrize("mask", ["tree", "tree_causal_window", "none_causal"])
def test_small(orc, monkeypatch, kernel, kind, G, Q, mask):
    force(monkeypatch, kernel)
    lens = [300, 45, 70, 0, 129, 64]
    counts = [Q, 1, min(Q, 3), 0, 0, Q - 1]  # includes sequences without queries (one of them empty)
    causal = "causal" in mask
    window = 37 if "window" in mask else 0
    say(f"[gpu] spec {kind} {kernel} G={G} Q={Q} {mask}")
    common = dict(num_q_heads=G * 2, num_kv_heads=2, head_dim=128, q_len=Q, seed=1200 + G * 50 + Q,
                  causal=causal, window=window)
    if kind == "contiguous":
        w = inputs.contiguous(batch=len(lens), kv_len=300, seq_lens=lens, **common)
    elif kind == "paged":
        w = inputs.paged(seq_lens=lens, page_size=16, poison=True, **common)
    else:
        w = inputs.sparse(batch=len(lens), kv_len=384, block_size=64, poison=True,
                          blocks=[[[0, 2, 4], [1, 4]], [[0], [0]], [[0, 1], [1]], [[], [0]], [[2], []], [[0], [0, 1]]],
                          seq_lens=lens, **common)
    w = inputs.with_spec(w, counts=counts, tree=mask.startswith("tree"), seed=7 + Q)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"S={S}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_one_launch_equals_two_launches(monkeypatch, kernel):
    """The in-pass merge and the merge kernel write the same bits to the packed rows."""
    force(monkeypatch, kernel)
    w = inputs.with_spec(inputs.paged(seq_lens=[300, 45, 0, 129], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                      q_len=5, page_size=16, seed=3),
                         counts=[5, 2, 0, 4], tree=True, seed=9)
    for S in (1, 3):
        monkeypatch.setenv("AD_FUSED_MERGE", "1")
        a = run(w, num_splits=S)
        monkeypatch.setenv("AD_FUSED_MERGE", "0")
        b = run(w, num_splits=S)
        assert bits_equal(a, b), f"S={S}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_mask_identities(monkeypatch, kernel):
    """A mask with every bit set is no mask; a chain-shaped tree is the bottom-right causal mask;
    packed queries with every count at q_len are the [B, q_len] layout -- all bit for bit."""
    force(monkeypatch, kernel)
    Q = 6
    base = inputs.paged(seq_lens=[300, 6, 129, 40], num_q_heads=8, num_kv_heads=2, head_dim=128, q_len=Q,
                        page_size=16, seed=21)
    plain = run(base)
    ones = inputs.with_spec(base)
    ones.tree_mask = torch.full((base.batch * Q, 1), -1, dtype=torch.int32)
    assert bits_equal(run(ones), plain)
    chain = inputs.with_spec(base)
    chain.tree_mask = torch.tensor([(1 << (t + 1)) - 1 for t in range(Q)] * base.batch, dtype=torch.int32)[:, None]
    causal = inputs.with_spec(base)
    causal.causal = True
    assert bits_equal(run(chain), run(causal))
    packed = inputs.with_spec(base, counts=[Q] * base.batch)
    po, pl, _ = run(packed)
    assert bits_equal((po.reshape(plain[0].shape), pl.reshape(plain[1].shape)), plain)


def test_rows_outside_the_sequences_untouched(monkeypatch):
    """Only the packed rows of existing tokens are written: rows past the last one keep their
    contents."""
    monkeypatch.delenv("AD_PARTIAL_KERNEL", raising=False)
    w = inputs.with_spec(inputs.paged(seq_lens=[200, 31, 77], num_q_heads=16, num_kv_heads=2, head_dim=128,
                                      q_len=4, page_size=16, seed=5), counts=[4, 0, 2], tree=True, seed=1)
    g = w.to("cuda")
    T, Hq = g.q.shape[0], w.num_q_heads
    out = torch.full((T + 3, Hq, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T + 3, Hq), 7.0, dtype=torch.float32, device="cuda")
    step = DecodeStep(g, out=out[:T], lse=lse[:T])
    step()
    torch.cuda.synchronize()
    assert torch.all(out[T:] == 7.0) and torch.all(lse[T:] == 7.0)
    assert torch.isfinite(out[:T]).all() and torch.isfinite(lse[:T]).all()



@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("kind", ["paged", "sparse"])
def test_fp8_cache_with_drafts(orc, monkeypatch, kernel, kind):
    """Packed draft tokens with tree masks over an E4M3 cache with row scales."""
    force(monkeypatch, kernel)
    lens = [300, 45, 0, 129]
    say(f"[gpu] spec + fp8 {kind} {kernel}")
    common = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, q_len=5, seed=1500, causal=False, window=0,
                  kv_format="fp8", poison=True)
    if kind == "paged":
        w = inputs.paged(seq_lens=lens, page_size=16, **common)
    else:
        w = inputs.sparse(batch=4, kv_len=384, block_size=64, seq_lens=lens,
                          blocks=[[[0, 2, 4], [1, 4]], [[0], [0]], [[], [0]], [[0, 1], [2]]], **common)
    w = inputs.with_spec(w, counts=[5, 2, 0, 4], tree=True, seed=4)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"S={S}")
