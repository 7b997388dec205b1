"""GPU parity of the matrix-core split-KV path (bf16, more than 8 query rows per KV head: grouped
heads times speculative query tokens), and of the vector path's row blocking, against the fp64
oracle on the same seeded inputs, through the C ABI."""
import contextlib
import os

import numpy as np
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@contextlib.contextmanager
def kernel(name):
    """Force the partial kernel choice (AD_PARTIAL_KERNEL is read at every call)."""
    old = os.environ.get("AD_PARTIAL_KERNEL")
    os.environ["AD_PARTIAL_KERNEL"] = name
    try:
        yield
    finally:
        if old is None:
            del os.environ["AD_PARTIAL_KERNEL"]
        else:
            os.environ["AD_PARTIAL_KERNEL"] = old


@pytest.fixture(autouse=True, params=["cols", "rows", "tile16"])
def load_form(request, monkeypatch):
    """Every test runs in the three forms of the bf16 matrix-core pass: 32-row units whose lane
    pairs read K as the matrix operand straight from HBM (cols) or whose waves read whole rows and
    stage them through LDS (rows), and 16-row units (tile16; a KV head with more rows takes several
    units)."""
    monkeypatch.setenv("AD_MFMA_TILE", "16" if request.param == "tile16" else "32")
    monkeypatch.setenv("AD_MFMA_ROWS", "1" if request.param == "rows" else "0")
    return request.param


def run(w_cpu, num_splits=None):
    wg = w_cpu.to("cuda")
    step = DecodeStep(wg, num_splits=num_splits)
    out, lse = step()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), step


# ------------------------------------------------------------------------------ workload 4
def test_workload4_full(orc):
    """Block-sparse + causal + sliding window, 4 speculative tokens x 8 heads = 32 rows per KV head,
    every row compared."""
    say("[gpu] workload 4: full size, every row")
    w = inputs.make(4)
    out, lse, step = run(w)
    say(f"  splits {step.splits}")
    ref_o, ref_l = oracle_of(orc, w)
    assert_tight(out, lse, ref_o, ref_l, w.dtype, "workload 4")


def test_workload4_poisoned_bit_identical():
    """Unlisted blocks hold NaN: the result is finite and bit-identical to the clean cache."""
    say("[gpu] workload 4 clean vs poisoned")
    a = run(inputs.make(4))
    b = run(inputs.make(4, poison=True))
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------------------ small cases
MASKS = {"none": (False, 0), "causal": (True, 0), "window": (False, 45), "causal_window": (True, 70)}
SHAPES = [  # (D, G, Q): rows per KV head = G * Q
    (128, 16, 1), (128, 8, 2), (128, 4, 3), (128, 8, 4), (64, 8, 4), (128, 16, 3), (64, 32, 2),
    (128, 5, 2), (64, 9, 1),
]


@pytest.mark.parametrize("D,G,Q", SHAPES, ids=lambda x: str(x))
@pytest.mark.parametrize("mask", list(MASKS))
def test_contiguous_small(orc, D, G, Q, mask):
    causal, window = MASKS[mask]
    say(f"[gpu] mfma contiguous D={D} G={G} Q={Q} {mask}")
    Hkv = 2
    # ragged lengths: shorter than a tile, not a multiple of 32, longer than several splits
    w = inputs.contiguous(batch=4, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, kv_len=700, q_len=Q,
                          seq_lens=[Q + 3, 33, 700, 415], seed=100 + D + G * 7 + Q, causal=causal, window=window)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3):
        out, lse, _ = run(w, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, w.dtype, f"S={S}")


@pytest.mark.parametrize("page_size", [16, 32, 64])
@pytest.mark.parametrize("G,Q", [(16, 1), (8, 4)])
def test_paged_small(orc, page_size, G, Q):
    say(f"[gpu] mfma paged page={page_size} G={G} Q={Q}")
    w = inputs.paged(seq_lens=[1 + Q, 40, 1111, 300], num_q_heads=G * 2, num_kv_heads=2, head_dim=128,
                     page_size=page_size, q_len=Q, seed=200 + page_size + G, causal=True, window=300)
    ref_o, ref_l = oracle_of(orc, w)
    out, lse, _ = run(w, num_splits=3)
    assert_matches(out, lse, ref_o, ref_l, w.dtype, "paged")


def test_paged_poisoned_bit_identical():
    lens = [5, 16, 250, 1000, 4097, 31]
    say("[gpu] mfma poisoned paged pool")
    kw = dict(seq_lens=lens, num_q_heads=32, num_kv_heads=2, head_dim=128, page_size=16, q_len=2, seed=9)
    a = run(inputs.paged(**kw), num_splits=4)
    b = run(inputs.paged(**kw, poison=True), num_splits=4)
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("block_size", [16, 32, 128])
def test_sparse_small(orc, block_size):
    """Per-(b, KV head) block lists of different lengths and orders, blocks partly past the end of
    short sequences, causal + window, poisoned unlisted blocks."""
    say(f"[gpu] mfma sparse block={block_size}")
    B, Hkv, Lmax, Q = 3, 2, 1024, 4
    nblk = Lmax // block_size
    g = torch.Generator().manual_seed(block_size)
    lists = []
    for b in range(B):
        row = []
        for h in range(Hkv):
            k = int(torch.randint(0, nblk + 1, (1,), generator=g))
            row.append(torch.randperm(nblk, generator=g)[:k].tolist())
        lists.append(row)
    lists[0][0] = []                      # no listed block at all
    lists[1][1] = list(range(nblk))       # every block
    kw = dict(batch=B, num_q_heads=8 * Hkv, num_kv_heads=Hkv, head_dim=128, kv_len=Lmax, q_len=Q,
              block_size=block_size, blocks=lists, seed=300 + block_size, causal=True, window=333,
              seq_lens=[1024, 517, 1000])
    w = inputs.sparse(**kw)
    ref_o, ref_l = oracle_of(orc, w)
    out, lse, _ = run(w, num_splits=2)
    assert_matches(out, lse, ref_o, ref_l, w.dtype, "sparse")
    wp = inputs.sparse(**kw, poison=True)
    out2, lse2, _ = run(wp, num_splits=2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_split_invariance():
    say("[gpu] mfma split invariance, 32 rows per KV head")
    w = inputs.contiguous(batch=2, num_q_heads=32, num_kv_heads=4, head_dim=128, kv_len=3000, q_len=4,
                          seed=77, causal=True)
    outs = []
    for S in (1, 2, 3, 5, 8, 16):
        out, lse, _ = run(w, num_splits=S)
        outs.append((S, out.double(), lse.double()))
    o0, l0 = outs[0][1], outs[0][2]
    for S, o, l_ in outs[1:]:
        assert (o - o0).abs().max() <= 2e-3, f"S={S}"
        assert (l_ - l0).abs().max() <= 1e-4, f"S={S}"


# ------------------------------------------------------------------------------ forced kernel choice
@pytest.mark.parametrize("G,Q", [(1, 1), (4, 1), (8, 1), (2, 3)])
def test_mfma_forced_on_few_rows(orc, G, Q):
    """The matrix-core kernels also serve 1..8 rows (padded to 32 or 16)."""
    say(f"[gpu] forced mfma G={G} Q={Q}")
    w = inputs.contiguous(batch=3, num_q_heads=G * 2, num_kv_heads=2, head_dim=128, kv_len=600, q_len=Q,
                          seq_lens=[600, 77, 5], seed=400 + G + Q, causal=True, window=200)
    ref_o, ref_l = oracle_of(orc, w)
    with kernel("mfma"):
        out, lse, _ = run(w, num_splits=2)
    assert_matches(out, lse, ref_o, ref_l, w.dtype, "forced mfma")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_valu_row_blocks(orc, dtype):
    """More than 8 rows on the vector kernel: 8-row blocks per KV head (fp32 always takes this path)."""
    say(f"[gpu] valu row blocks {dtype}")
    w = inputs.contiguous(batch=2, num_q_heads=24, num_kv_heads=2, head_dim=64, kv_len=500, q_len=2,
                          seq_lens=[500, 123], seed=500, causal=True, window=100, dtype=dtype)
    ref_o, ref_l = oracle_of(orc, w)
    with kernel("valu"):
        out, lse, _ = run(w, num_splits=3)
    assert_matches(out, lse, ref_o, ref_l, w.dtype, "valu row blocks")


def test_mfma_matches_valu_closely():
    """Both kernels on the same 32-row problem agree to rounding (they round P differently)."""
    say("[gpu] mfma vs valu")
    w = inputs.contiguous(batch=2, num_q_heads=32, num_kv_heads=4, head_dim=128, kv_len=2000, q_len=4,
                          seed=600, causal=True, window=1500)
    with kernel("valu"):
        ov, lv, _ = run(w, num_splits=2)
    om, lm, _ = run(w, num_splits=2)
    assert float((ov.double() - om.double()).abs().max()) <= 2e-3
    assert float((lv.double() - lm.double()).abs().max()) <= 2e-4
    assert not np.isnan(om.float().numpy()).any()


@pytest.mark.parametrize("kind", ["contiguous", "paged", "sparse", "spec"])
def test_load_forms_bit_identical(monkeypatch, kind):
    """The two load forms feed the matrix cores the same operands in the same order: the results
    agree bit for bit."""
    say(f"[gpu] mfma load forms {kind}")
    common = dict(num_q_heads=16, num_kv_heads=2, head_dim=128, q_len=4, seed=700, causal=True, window=900)
    if kind == "contiguous":
        w = inputs.contiguous(batch=3, kv_len=1500, seq_lens=[1500, 31, 777], **common)
    elif kind == "sparse":
        w = inputs.sparse(batch=2, kv_len=1024, block_size=64, seq_lens=[1024, 600], poison=True,
                          blocks=[[[0, 3, 9, 15], [2]], [[1, 4, 8], []]], **common)
    else:
        w = inputs.paged(seq_lens=[1500, 31, 777, 4], page_size=16, poison=True, **common)
        if kind == "spec":
            w = inputs.with_spec(w, counts=[4, 2, 0, 3], tree=True, seed=2)
    res = []
    for form in ("0", "1"):
        monkeypatch.setenv("AD_MFMA_ROWS", form)
        for S in (1, 3):
            out, lse, _ = run(w, num_splits=S)
            res.append((out.view(torch.int16), lse))
    for S_i in (0, 1):
        a, b = res[S_i], res[2 + S_i]
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), f"split set {S_i}"
