"""GPU parity of the E4M3 (fp8) cache path against the fp64 oracle on the same seeded inputs,
through the C ABI: contiguous, paged and block-sparse caches, row and tensor scales, ragged and
empty sequences, masks, grouped and speculative query rows, split counts, and NaN codes in every
cache slot that must not be read."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# the matrix-core kernel in its 16-row units (operands straight from the loads, and whole-row
# loads with K through LDS: AD_MFMA_ROWS) and 32-row units (AD_MFMA_TILE), and the vector form
# (AD_PARTIAL_KERNEL=valu)
KERNELS = ["mfma16", "mfma16rows", "mfma32", "valu"]


def force(monkeypatch, kernel):
    if kernel == "valu":
        monkeypatch.setenv("AD_PARTIAL_KERNEL", "valu")
    else:
        monkeypatch.delenv("AD_PARTIAL_KERNEL", raising=False)
        monkeypatch.setenv("AD_MFMA_TILE", kernel[4:6])
        monkeypatch.setenv("AD_MFMA_ROWS", "1" if kernel.endswith("rows") else "0")


def run(w, num_splits=None, fused=True):
    step = DecodeStep(w.to("cuda"), num_splits=num_splits, fused=fused)
    out, lse = step()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), step


@pytest.mark.parametrize("tile", ["default", "16rows", "16regs", "32"])
def test_workload6_full(orc, monkeypatch, tile):
    """The planner's choice, both load forms of the 16-row units, and the 32-row units, every row."""
    if tile != "default":
        monkeypatch.setenv("AD_MFMA_TILE", tile[:2])
        monkeypatch.setenv("AD_MFMA_ROWS", "1" if tile == "16rows" else "0")
    say(f"[gpu] workload 6 (fp8 paged ragged): full size, every row, tile {tile}")
    w = inputs.make(6)
    out, lse, step = run(w)
    say(f"  splits {step.splits}")
    ref_o, ref_l = oracle_of(orc, w)
    assert_tight(out, lse, ref_o, ref_l, torch.bfloat16, "workload 6")


@pytest.mark.parametrize("kernel", KERNELS)
def test_workload6_poisoned_bit_identical(monkeypatch, kernel):
    """NaN codes and NaN scales in unreferenced pages and tail slots change nothing, bit for bit."""
    force(monkeypatch, kernel)
    say(f"[gpu] workload 6 poisoned pool, {kernel}")
    a, la, _ = run(inputs.make(6))
    b, lb, _ = run(inputs.make(6, poison=True))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("scales", ["token", "tensor"])
@pytest.mark.parametrize("G,Q", [(1, 1), (2, 1), (4, 1), (8, 1), (4, 2), (1, 3), (16, 1), (8, 5)])
@pytest.mark.parametrize("mask", ["none", "causal_window"])
def test_contiguous_small(orc, monkeypatch, kernel, scales, G, Q, mask):
    force(monkeypatch, kernel)
    causal = mask.startswith("causal")
    window = 37 if "window" in mask else 0
    lens = [300, 1, 37, 0, 129]
    say(f"[gpu] fp8 contiguous {kernel} G={G} Q={Q} {mask} scales={scales}")
    w = inputs.contiguous(batch=len(lens), num_q_heads=G * 2, num_kv_heads=2, head_dim=128, kv_len=300, q_len=Q,
                          seed=800 + G * 10 + Q, seq_lens=lens, causal=causal, window=window, kv_format="fp8",
                          kv_scales=scales)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3, 7):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"S={S}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("page_size", [16, 32, 64])
def test_paged_small(orc, monkeypatch, kernel, page_size):
    force(monkeypatch, kernel)
    lens = [1, 15, 16, 17, 300, 0, 77]
    say(f"[gpu] fp8 paged {kernel} page={page_size}")
    w = inputs.paged(seq_lens=lens, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=page_size,
                     seed=900 + page_size, kv_format="fp8", poison=True)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 2, 5):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"page {page_size} S={S}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_block_sparse(orc, monkeypatch, kernel):
    force(monkeypatch, kernel)
    say(f"[gpu] fp8 block-sparse {kernel}, causal, poisoned unlisted blocks")
    w = inputs.sparse(batch=3, num_q_heads=16, num_kv_heads=2, head_dim=128, kv_len=2048, q_len=2,
                      block_size=128, blocks=[[[0, 3, 5], []], [[1], [2, 4, 6, 8]], [[7, 9], [15]]],
                      seed=5, causal=True, window=0, kv_format="fp8", poison=True)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 2, 5):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"S={S}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_one_launch_equals_two_launches(monkeypatch, kernel):
    """The in-pass merge and the merge kernel give the same bits on an fp8 cache."""
    force(monkeypatch, kernel)
    w = inputs.contiguous(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=128, kv_len=300, q_len=1, seed=4,
                          seq_lens=[300, 1, 37, 0, 129], kv_format="fp8")
    for S in (1, 3):
        monkeypatch.setenv("AD_FUSED_MERGE", "1")
        o1, l1, _ = run(w, num_splits=S)
        o2, l2, _ = run(w, num_splits=S, fused=False)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), f"S={S}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_every_value_code_decodes_exactly(monkeypatch, kernel):
    """With one key per sequence the output is that key's value row times its scale (1 here), and
    every E4M3 value is a bf16 value: each of the 252 nonzero finite codes (and +0) must come out bit-exact as
    PyTorch's float8_e4m3fn decodes it (sequence 0 carries codes 0x00-0x7E, sequence 1 0x80-0xFE;
    the two NaN codes are replaced by 0, and so is -0, 0x80: a weighted sum that starts from +0
    returns +0 for it, which attention cannot tell apart)."""
    force(monkeypatch, kernel)
    say(f"[gpu] fp8 value codes, {kernel}")
    w = inputs.contiguous(batch=2, num_q_heads=1, num_kv_heads=1, head_dim=128, kv_len=1, seed=11,
                          kv_format="fp8")
    codes = torch.arange(256, dtype=torch.int32).reshape(2, 128)
    codes[(codes % 128 == 127) | (codes == 128)] = 0
    w.storage["v"].copy_(codes.to(torch.uint8).reshape(2, 1, 1, 128))
    w.storage["v_scale"].fill_(1.0)
    out, lse, _ = run(w)
    want = codes.to(torch.uint8).view(torch.float8_e4m3fn).to(torch.bfloat16).reshape(2, 1, 1, 128)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
