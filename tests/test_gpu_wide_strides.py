"""GPU parity with cache strides too wide for the kernels' 32-bit address fast paths, which then
take their general 64-bit address arithmetic: the MLA copy issue (pool byte strides below 2^32:
two 32 x 32-bit multiply-adds per row) and the 16-row matrix-core kernel's whole-row fp8 loads
(slot strides below 2^26 elements: one multiply-add per lane and block). The wide pools are built
on the device with the same values at wide offsets; each result must equal the compact pool's
bit for bit (the arithmetic order depends only on logical positions) and the fp64 oracle's."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def run(wg, num_splits=None):
    out, lse = DecodeStep(wg, num_splits=num_splits)()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def widen(t, dim, stride):
    """A view with t's values in a fresh zeroed device buffer: the dimensions after `dim` packed,
    dimension `dim` stepping `stride` elements, the dimensions before it packed around that."""
    shape = list(t.shape)
    strides = [0] * len(shape)
    s = 1
    for d in range(len(shape) - 1, dim, -1):
        strides[d] = s
        s *= shape[d]
    assert stride >= s
    strides[dim] = stride
    s = stride * shape[dim]
    for d in range(dim - 1, -1, -1):
        strides[d] = s
        s *= shape[d]
    size = 1 + sum((n - 1) * st for n, st in zip(shape, strides))
    buf = torch.zeros(size, dtype=t.dtype, device="cuda")
    view = torch.as_strided(buf, shape, strides)
    view.copy_(t)
    return view


def test_mla_page_stride_past_4gb(orc):
    """The ckv pool's pages 2^31 + 32768 elements apart: byte strides past 2^32 (4.3 GB of pool)."""
    lens = [100]
    say("[gpu] mla with a ckv page stride of 2^31 + 32768 elements")
    w = inputs.mla(batch=1, num_heads=32, kv_len=100, page_size=64, seq_lens=lens, seed=23)
    ref_o, ref_l = oracle_of(orc, w)
    wg = w.to("cuda")
    o0, l0 = run(wg, num_splits=2)
    stride = 2 ** 31 + 64 * 512
    wide = widen(wg.k, 0, stride)
    assert wide.stride(0) == stride and 2 * wide.stride(0) >= 2 ** 32
    wg.k = wg.v = wide
    o1, l1 = run(wg, num_splits=2)
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "wide and compact pools differ"
    assert_matches(o1, l1, ref_o, ref_l, w.dtype, "mla, wide page stride")
    del wide, wg
    torch.cuda.empty_cache()


def test_fp8_whole_rows_slot_stride_past_2_26(orc, monkeypatch):
    """The paged fp8 pool's slots 2^26 + 256 bytes apart, on the 16-row kernel's whole-row form."""
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "mfma")
    monkeypatch.setenv("AD_MFMA_TILE", "16")
    monkeypatch.setenv("AD_MFMA_ROWS", "1")
    say("[gpu] fp8 whole rows with a slot stride of 2^26 + 256 bytes")
    w = inputs.paged(seq_lens=[16, 9], num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, seed=24,
                     kv_format="fp8")
    ref_o, ref_l = oracle_of(orc, w)
    wg = w.to("cuda")
    o0, l0 = run(wg)
    stride = 2 ** 26 + 256
    for name in ("k", "v"):  # [pages, page_size, Hkv, D]: widen the slot dimension
        t = getattr(wg, name).contiguous()
        wide = widen(t, 1, stride)
        assert wide.stride(1) == stride
        setattr(wg, name, wide)
    o1, l1 = run(wg)
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "wide and compact pools differ"
    assert_matches(o1, l1, ref_o, ref_l, torch.bfloat16, "fp8 whole rows, wide slot stride")
    del wg
    torch.cuda.empty_cache()
