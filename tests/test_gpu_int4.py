"""GPU parity of the int4 cache path (4-bit fields with fp16 scale / shift per group, rows of
32-bit words) against the fp64 oracle on the same seeded inputs, through the C ABI: contiguous,
paged and block-sparse caches, 1 to 8 groups, ragged and empty sequences, masks, grouped and
speculative query rows, split counts, and NaN coefficients in every row that must not be read.
Rows of one group run on the 16-row matrix-core kernel by default and on the vector kernel with
AD_PARTIAL_KERNEL=valu; rows of 2, 4 or 8 groups always on the vector kernel."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


KERNELS = ["default", "valu"]


def force(monkeypatch, kernel):
    if kernel == "valu":
        monkeypatch.setenv("AD_PARTIAL_KERNEL", "valu")
    else:
        monkeypatch.delenv("AD_PARTIAL_KERNEL", raising=False)


def run(w, num_splits=None, fused=True):
    step = DecodeStep(w.to("cuda"), num_splits=num_splits, fused=fused)
    out, lse = step()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), step


@pytest.mark.parametrize("kernel", KERNELS)
def test_workload8_full(orc, monkeypatch, kernel):
    force(monkeypatch, kernel)
    say(f"[gpu] workload 8 (int4 paged ragged): full size, every row, {kernel}")
    w = inputs.make(8)
    out, lse, step = run(w)
    say(f"  splits {step.splits}")
    ref_o, ref_l = oracle_of(orc, w)
    assert_tight(out, lse, ref_o, ref_l, torch.bfloat16, "workload 8")


@pytest.mark.parametrize("kernel", KERNELS)
def test_workload8_poisoned_bit_identical(monkeypatch, kernel):
    """NaN coefficients in unreferenced pages and tail slots change nothing, bit for bit."""
    force(monkeypatch, kernel)
    say(f"[gpu] workload 8 poisoned pool, {kernel}")
    a, la, _ = run(inputs.make(8))
    b, lb, _ = run(inputs.make(8, poison=True))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


# (groups, kernel): one group on both kernels, more groups on the vector kernel only
GROUPS = [(1, "default"), (1, "valu"), (2, "default"), (4, "default"), (8, "default")]


@pytest.mark.parametrize("groups,kernel", GROUPS)
@pytest.mark.parametrize("G,Q", [(1, 1), (2, 1), (4, 1), (8, 1), (4, 2), (1, 3), (16, 1), (4, 5)])
@pytest.mark.parametrize("mask", ["none", "causal_window"])
def test_contiguous_small(orc, monkeypatch, groups, kernel, G, Q, mask):
    force(monkeypatch, kernel)
    causal = mask.startswith("causal")
    window = 37 if "window" in mask else 0
    lens = [300, 1, 37, 0, 129]
    say(f"[gpu] int4 contiguous groups={groups} {kernel} G={G} Q={Q} {mask}")
    w = inputs.contiguous(batch=len(lens), num_q_heads=G * 2, num_kv_heads=2, head_dim=128, kv_len=300, q_len=Q,
                          seed=1300 + G * 10 + Q, seq_lens=lens, causal=causal, window=window, kv_format="int4",
                          kv_groups=groups)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3, 7):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"S={S}")


@pytest.mark.parametrize("page_size", [16, 32, 64])
@pytest.mark.parametrize("groups,kernel", [(1, "default"), (1, "valu"), (4, "default")])
def test_paged_small(orc, monkeypatch, page_size, groups, kernel):
    force(monkeypatch, kernel)
    lens = [1, 15, 16, 17, 300, 0, 77]
    say(f"[gpu] int4 paged page={page_size} groups={groups} {kernel}")
    w = inputs.paged(seq_lens=lens, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=page_size,
                     seed=1400 + page_size, kv_format="int4", kv_groups=groups, poison=True)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 2, 5):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"page {page_size} S={S}")


@pytest.mark.parametrize("groups", [1, 2])
def test_block_sparse(orc, groups):
    say(f"[gpu] int4 block-sparse, causal, poisoned unlisted blocks, groups={groups}")
    w = inputs.sparse(batch=3, num_q_heads=16, num_kv_heads=2, head_dim=128, kv_len=2048, q_len=2,
                      block_size=128, blocks=[[[0, 3, 5], []], [[1], [2, 4, 6, 8]], [[7, 9], [15]]],
                      seed=15, causal=True, window=0, kv_format="int4", kv_groups=groups, poison=True)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 2, 5):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"S={S}")


@pytest.mark.parametrize("groups", [1, 4])
def test_speculative_rows(orc, groups):
    """Packed variable-length queries with tree masks over an int4 cache."""
    say(f"[gpu] int4 paged, variable query lengths + tree masks, groups={groups}")
    base = inputs.paged(seq_lens=[300, 45, 0, 129], num_q_heads=8, num_kv_heads=2, head_dim=128, q_len=5,
                        page_size=16, seed=17, kv_format="int4", kv_groups=groups, poison=True)
    w = inputs.with_spec(base, counts=[5, 2, 0, 4], tree=True, seed=3)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, torch.bfloat16, f"S={S}")


@pytest.mark.parametrize("groups", [1, 2])
def test_one_launch_equals_two_launches(monkeypatch, groups):
    """The in-pass merge and the merge kernel give the same bits on an int4 cache."""
    w = inputs.contiguous(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=128, kv_len=300, q_len=1, seed=4,
                          seq_lens=[300, 1, 37, 0, 129], kv_format="int4", kv_groups=groups)
    for S in (1, 3):
        monkeypatch.setenv("AD_FUSED_MERGE", "1")
        o1, l1, _ = run(w, num_splits=S)
        o2, l2, _ = run(w, num_splits=S, fused=False)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2), f"S={S}"


@pytest.mark.parametrize("groups,kernel", [(4, "default"), (1, "default"), (1, "valu")])
def test_fields_decode_exactly(monkeypatch, groups, kernel):
    """One key per sequence: the output is its value row. With scale 1 and shift 0 every field
    0..15 comes out as that integer; with scale 2^-3 and shift -1 as field/8 - 1 (all exact in
    bf16). Field d % 8 of word d / 8 is dimension d, and group g's coefficient word applies to
    dimensions 128 g / groups .. 128 (g + 1) / groups - 1."""
    force(monkeypatch, kernel)
    say(f"[gpu] int4 fields, exact, groups={groups} {kernel}")
    w = inputs.contiguous(batch=2, num_q_heads=1, num_kv_heads=1, head_dim=128, kv_len=1, seed=12,
                          kv_format="int4", kv_groups=groups)
    f0 = torch.arange(128) % 16
    f1 = f0.flip(0)
    fields = torch.stack([f0, f1])                                      # [2, 128]
    packed = torch.zeros(2, 16, dtype=torch.int64)
    for j in range(8):
        packed |= fields.reshape(2, 16, 8)[:, :, j].long() << (4 * j)
    one = 0x3C00                                                        # fp16 1.0
    eighth, minus_one = 0x3000, 0xBC00                                  # fp16 2^-3, -1.0
    coef = torch.tensor([[one] * groups, [eighth | (minus_one << 16)] * groups], dtype=torch.int64)
    words = torch.cat([coef, packed], dim=1)
    words = torch.where(words >= 2 ** 31, words - 2 ** 32, words).to(torch.int32)
    w.storage["v"].copy_(words.reshape(2, 1, 1, 16 + groups))
    out, _, _ = run(w)
    want = torch.stack([f0.float(), f1.float() / 8 - 1]).to(torch.bfloat16).reshape(2, 1, 1, 128)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
