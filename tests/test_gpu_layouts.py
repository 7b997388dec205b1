"""GPU parity on token-major caches: the contiguous cache stored [B, L, Hkv, D] and the paged pool
stored [pages, page_size, Hkv, D] (every key's KV heads side by side, so the stride between two
keys of one head is Hkv * D), at the full sizes of the contiguous GQA workload and the paged ragged
workload, on both GQA partial kernels (the vector kernel, and the matrix-core kernel in both of
its load forms). Each result is compared with the fp64 oracle, and with the head-major cache of the
same values bit for bit (the kernels' arithmetic order depends only on logical positions)."""
import functools

import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, assert_tight, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KERNELS = ["valu", "mfma_cols", "mfma_rows"]


@pytest.fixture(params=KERNELS)
def kernel(request, monkeypatch):
    k = request.param
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "valu" if k == "valu" else "mfma")
    monkeypatch.setenv("AD_MFMA_ROWS", "1" if k == "mfma_rows" else "0")
    return k


def run(w_cpu, num_splits=None):
    step = DecodeStep(w_cpu.to("cuda"), num_splits=num_splits)
    out, lse = step()
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@functools.lru_cache(maxsize=None)
def reference(config):
    import oracle

    w = inputs.make(config)
    return oracle_of(oracle.load(), w)


@pytest.mark.parametrize("config", [2, 3])
def test_token_major_full_size(kernel, config):
    say(f"[gpu] workload {config} token-major, kernel {kernel}")
    w = inputs.make(config)
    t = inputs.token_major(w)
    assert t.k.stride(1) == w.num_kv_heads * w.head_dim_qk and t.k.is_contiguous()
    out, lse = run(t)
    ref_o, ref_l = reference(config)
    assert_tight(out, lse, ref_o, ref_l, w.dtype, f"workload {config} token-major ({kernel})")
    o2, l2 = run(w)
    assert torch.equal(out, o2) and torch.equal(lse, l2), "token-major and head-major results differ"


def test_token_major_poisoned_pool(kernel):
    """The paged workload with NaN in every unreferenced page and tail slot, stored token-major:
    finite and bit-identical to the clean token-major pool."""
    say(f"[gpu] workload 3 token-major poisoned, kernel {kernel}")
    a = run(inputs.token_major(inputs.make(3)))
    b = run(inputs.token_major(inputs.make(3, poison=True)))
    assert torch.isfinite(b[0]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("case", ["contig_causal_window", "paged_32", "sparse_poison"])
def test_token_major_small(orc, kernel, case):
    """Ragged and masked small caches in token-major storage, several split counts."""
    say(f"[gpu] token-major small {case}, kernel {kernel}")
    if case == "contig_causal_window":
        w = inputs.contiguous(batch=4, num_q_heads=32, num_kv_heads=4, head_dim=128, kv_len=900, q_len=2,
                              seed=71, seq_lens=[900, 3, 517, 0], causal=True, window=300)
    elif case == "paged_32":
        w = inputs.paged(seq_lens=[1, 31, 32, 33, 800, 0], num_q_heads=16, num_kv_heads=2, head_dim=64,
                         page_size=32, seed=72, poison=True)
    else:
        w = inputs.sparse(batch=2, num_q_heads=16, num_kv_heads=2, head_dim=128, kv_len=1024, q_len=4,
                          block_size=128, blocks=[[[0, 3, 7], [7]], [[], [1, 2, 3, 4, 5, 6, 7]]], seed=73,
                          causal=True, window=500, poison=True)
    t = inputs.token_major(w)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 3):
        out, lse = run(t, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, w.dtype, f"{case} S={S}")
        o2, l2 = run(w, num_splits=S)
        assert torch.equal(torch.nan_to_num(out), torch.nan_to_num(o2)) and torch.equal(lse, l2)


@pytest.mark.parametrize("fp8_kernel", ["mfma", "valu"])
def test_token_major_fp8(orc, monkeypatch, fp8_kernel):
    """An fp8 pool with per-row scales, cache and scales stored token-major."""
    monkeypatch.setenv("AD_PARTIAL_KERNEL", fp8_kernel)
    say(f"[gpu] token-major fp8 pool, kernel {fp8_kernel}")
    w = inputs.paged(seq_lens=[5, 300, 1000, 17], num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                     seed=74, kv_format="fp8", poison=True)
    t = inputs.token_major(w)
    assert t.k_scale.stride(1) == 4
    ref_o, ref_l = oracle_of(orc, w)
    out, lse = run(t, num_splits=2)
    assert_matches(out, lse, ref_o, ref_l, w.dtype, "fp8 token-major")


@pytest.mark.parametrize("config,rows", [(6, "1"), (6, "0"), (8, None)], ids=["fp8_whole_rows", "fp8_half_rows", "int4"])
def test_token_major_quantised_full_size(monkeypatch, config, rows):
    """The ragged fp8 and int4 workloads at full size, cache (and fp8 row scales) stored
    token-major, on the 16-row kernel (fp8 in both load forms; the whole-row form addresses a block
    from one page lookup and the row stride, here Hkv rows): the oracle's result, and the
    head-major result bit for bit."""
    monkeypatch.delenv("AD_PARTIAL_KERNEL", raising=False)
    if rows is not None:
        monkeypatch.setenv("AD_MFMA_ROWS", rows)
    say(f"[gpu] workload {config} token-major, AD_MFMA_ROWS={rows}")
    w = inputs.make(config)
    t = inputs.token_major(w)
    out, lse = run(t)
    ref_o, ref_l = reference(config)
    assert_tight(out, lse, ref_o, ref_l, torch.bfloat16, f"workload {config} token-major")
    o2, l2 = run(w)
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2), \
        "token-major and head-major results differ"


@pytest.mark.parametrize("groups", [1, 4])
def test_token_major_int4(orc, monkeypatch, groups):
    """An int4 pool (one coefficient group per row on the 16-row kernel, four on the vector kernel),
    stored token-major, NaN coefficients in every unreferenced row."""
    monkeypatch.delenv("AD_PARTIAL_KERNEL", raising=False)
    say(f"[gpu] token-major int4 pool, groups {groups}")
    w = inputs.paged(seq_lens=[5, 300, 1000, 17], num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                     seed=75, kv_format="int4", kv_groups=groups, poison=True)
    t = inputs.token_major(w)
    ref_o, ref_l = oracle_of(orc, w)
    for S in (1, 2):
        out, lse = run(t, num_splits=S)
        assert_matches(out, lse, ref_o, ref_l, w.dtype, f"int4 token-major S={S}")
        o2, l2 = run(w, num_splits=S)
        assert torch.equal(out.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
