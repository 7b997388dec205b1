"""Repeatability: every workload's step gives the same bits each time it runs, also with the
other workloads' steps (their own workspaces, arrival counters and merges) launched in between.
The split count, the in-pass merge's election of the last arrival and the exact recompute of the
MLA kernel change nothing: each result depends only on its inputs."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import gpu_available, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def test_every_workload_repeats_bit_for_bit():
    configs = list(range(1, 9))
    say(f"[gpu] determinism over workloads {configs}")
    steps = {c: DecodeStep(inputs.make(c).to("cuda")) for c in configs}
    first = {}
    for c in configs:
        out, lse = steps[c]()
        first[c] = (out.clone(), lse.clone())
    torch.cuda.synchronize()
    for rep in range(2):
        for c in reversed(configs):
            out, lse = steps[c]()
            torch.cuda.synchronize()
            assert torch.equal(out, first[c][0]) and torch.equal(lse, first[c][1]), f"workload {c}, repeat {rep}"
    say("  all repeats bit-identical")
