"""attn_decode_noalloc, the whole decode step in the library's own static workspace, against
attn_decode with a caller workspace on the same inputs: two calls in a row (the second smaller,
so it runs in what the first left behind), one that merges in two launches and one that merges
inside its single launch. The library runs the same kernels with the same plan, so the results
must agree bit for bit; each is also checked against the fp64 oracle."""
import pytest
import torch

from attention_decode_amd import _abi, inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def both(w_cpu, num_splits=0):
    wg = w_cpu.to("cuda")
    step = DecodeStep(wg, num_splits=num_splits or None)
    ref_out, ref_lse = (t.cpu().clone() for t in step())
    step.out.fill_(7.0)
    step.lse.fill_(7.0)
    _abi.attn_decode_noalloc(step.args, step.paged, step.sparse, num_splits)
    torch.cuda.synchronize()
    return step, (ref_out, ref_lse), (step.out.cpu(), step.lse.cpu())


def test_noalloc_two_calls_shrinking(orc):
    cases = [
        ("workload 3 (paged, ragged, two launches)", inputs.make(3), 0),
        ("small paged, forced 3 splits", inputs.paged(seq_lens=[7, 300, 0, 64], num_q_heads=8, num_kv_heads=2,
                                                     head_dim=128, page_size=16, seed=91), 3),
    ]
    for what, w, S in cases:
        say(f"[gpu] noalloc: {what}")
        step, (o1, l1), (o2, l2) = both(w, S)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{what}: differs from attn_decode"
        ref_o, ref_l = oracle_of(orc, w)
        assert_matches(o2, l2, ref_o, ref_l, w.dtype, what)


def test_noalloc_single_launch_twice(orc, monkeypatch):
    """The merge inside the single launch counts arrivals in the library's array: two calls in a
    row, the second smaller, both bit-identical to attn_decode (the counters came back to zero)."""
    monkeypatch.setenv("AD_FUSED_MERGE", "1")
    for what, w in (("workload 2 (one launch)", inputs.make(2)),
                    ("small contiguous (one launch)", inputs.contiguous(batch=3, num_q_heads=8, num_kv_heads=2,
                                                                        head_dim=64, kv_len=500, seed=92,
                                                                        seq_lens=[500, 1, 250]))):
        say(f"[gpu] noalloc: {what}")
        step, (o1, l1), (o2, l2) = both(w)
        assert _abi.attn_decode_launches(step.args, step.paged, step.sparse, step.splits) == 1
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{what}: differs from attn_decode"
        ref_o, ref_l = oracle_of(orc, w)
        assert_matches(o2, l2, ref_o, ref_l, w.dtype, what)
