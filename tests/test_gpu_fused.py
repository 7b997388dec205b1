"""GPU tests of the whole-step entry attn_decode. With the in-pass merge forced (one launch), the
last split of each work unit merges the unit's partials: the result must equal the two-pass path
(attn_decode_splitkv + attn_decode_merge) bit for bit, since both merge the same partials in the
same order; the arrival counters must be zero again after every call; and a workspace must be
reusable across calls with different split counts. With two launches forced, attn_decode must
give the same result too. Parity against the oracle runs in the other GPU tests, which call
attn_decode with its own choice of one or two launches."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(autouse=True)
def one_launch(monkeypatch):
    """attn_decode picks one or two launches by shape; these tests force the one-launch merge."""
    monkeypatch.setenv("AD_FUSED_MERGE", "1")


def both(wg, S):
    fused = DecodeStep(wg, num_splits=S, fused=True)
    two = DecodeStep(wg, num_splits=S, fused=False)
    o1, l1 = fused()
    o2, l2 = two()
    torch.cuda.synchronize()
    return fused, (o1.cpu(), l1.cpu()), (o2.cpu(), l2.cpu())


def counters_of(step):
    """The arrival counters: the fixed region at the start of the workspace."""
    return step.workspace[:1 << 20].cpu()


def same(x, y):
    return torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                       y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_fused_equals_two_pass(config):
    w = inputs.make(config)
    wg = w.to("cuda")
    S = DecodeStep(wg).splits
    for s in sorted({S, 1, 3}):
        say(f"[gpu] workload {config}: one launch vs two passes, {s} splits")
        step, (o1, l1), (o2, l2) = both(wg, s)
        assert same(o1, o2), f"S={s}: out differs from the two-pass result"
        assert same(l1, l2), f"S={s}: lse differs from the two-pass result"
        assert int(counters_of(step).count_nonzero()) == 0, "arrival counters not back to zero"


def test_fused_small_cases_equal_two_pass():
    """Ragged and empty sequences, masks, fp32 and bf16, both head dims, VALU and matrix-core row
    counts, contiguous and block-sparse."""
    lens = [300, 1, 37, 0, 129]
    for dtype, D, G, Q, mask in ((torch.float32, 128, 8, 1, "causal"), (torch.bfloat16, 64, 4, 2, "window"),
                                 (torch.bfloat16, 128, 8, 4, "causal_window"), (torch.bfloat16, 128, 16, 1, "none")):
        causal, window = mask.startswith("causal"), 37 if "window" in mask else 0
        w = inputs.contiguous(batch=len(lens), num_q_heads=G * 2, num_kv_heads=2, head_dim=D, kv_len=300, q_len=Q,
                              dtype=dtype, seed=7, seq_lens=lens, causal=causal, window=window)
        wg = w.to("cuda")
        for S in (1, 2, 7):
            say(f"[gpu] one launch vs two passes: {dtype} D={D} G={G} Q={Q} {mask} S={S}")
            step, (o1, l1), (o2, l2) = both(wg, S)
            assert same(o1, o2) and same(l1, l2), f"{dtype} D={D} G={G} Q={Q} {mask} S={S}"
            assert int(counters_of(step).count_nonzero()) == 0
            assert torch.all(o1[3] == 0) and torch.all(torch.isneginf(l1[3])), "empty sequence: out 0, lse -inf"
    # block-sparse: some (b, h) list no block at all
    w = inputs.sparse(batch=3, num_q_heads=16, num_kv_heads=2, head_dim=128, kv_len=2048, q_len=2,
                      dtype=torch.bfloat16, seed=3, block_size=128, blocks=[[[0, 3, 5], []], [[1], [2, 4, 6, 8]],
                                                                              [[], []]], causal=True, window=0)
    wg = w.to("cuda")
    for S in (1, 2, 5):
        say(f"[gpu] one launch vs two passes: block-sparse S={S}")
        step, (o1, l1), (o2, l2) = both(wg, S)
        assert same(o1, o2) and same(l1, l2), f"block-sparse S={S}"
        assert int(counters_of(step).count_nonzero()) == 0


def test_fused_workspace_reuse_across_calls_and_split_counts():
    """One zero-filled workspace, many calls with different split counts: every call matches the
    two-pass result, and the counters stay clean between calls."""
    w = inputs.make(3)
    wg = w.to("cuda")
    big = DecodeStep(wg, num_splits=8, fused=True)  # workspace sized for 8 splits
    for S in (8, 3, 1, 5, 8, 2):
        step = DecodeStep(wg, num_splits=S, fused=True)
        step.workspace = big.workspace  # large enough for every S <= 8
        o1, l1 = step()
        ref = DecodeStep(wg, num_splits=S, fused=False)
        o2, l2 = ref()
        torch.cuda.synchronize()
        say(f"[gpu] workload 3, shared workspace, {S} splits")
        assert same(o1.cpu(), o2.cpu()) and same(l1.cpu(), l2.cpu()), f"S={S}"
        assert int(counters_of(big).count_nonzero()) == 0


def test_two_launch_choice_equals_two_pass(monkeypatch):
    """attn_decode's two-launch form (partial pass + merge kernel in its workspace) for contiguous,
    paged and block-sparse caches."""
    monkeypatch.setenv("AD_FUSED_MERGE", "0")
    cases = [inputs.make(3), inputs.make(4),
             inputs.contiguous(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=128, kv_len=300, q_len=1,
                               dtype=torch.bfloat16, seed=9, seq_lens=[300, 1, 37, 0, 129])]
    for w in cases:
        wg = w.to("cuda")
        for S in (1, 3):
            say(f"[gpu] attn_decode two launches vs splitkv + merge: {w.name} S={S}")
            step, (o1, l1), (o2, l2) = both(wg, S)
            assert same(o1, o2) and same(l1, l2), f"{w.name} S={S}"
            assert int(counters_of(step).count_nonzero()) == 0
