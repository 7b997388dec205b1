"""The C-ABI library on the CPU: it loads, exports every symbol the header declares, and rejects
malformed arguments with the documented code before making any HIP call (none of these tests
needs a GPU; valid calls are exercised by the GPU tests)."""
import ctypes
import os
import re

import pytest
import torch

import attention_decode_amd as ad
from attention_decode_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_decode(?:_\w+)?)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_decode", "attn_decode_launches", "attn_decode_kernel", "attn_decode_splitkv", "attn_decode_merge", "attn_decode_paged", "attn_decode_mla",
              "attn_decode_workspace_size", "attn_decode_plan", "attn_decode_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_abi.LIBRARY)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (AD_\w+) \(?(-?\d+)\)?", text)}
    for code, name in _abi.STATUS.items():
        assert codes[name] == code
    assert codes["AD_F32"] == _abi.AD_F32 and codes["AD_BF16"] == _abi.AD_BF16
    assert codes["AD_MAX_SPLITS"] == _abi.AD_MAX_SPLITS


def test_struct_layouts_match_header_sizes():
    """The ctypes mirrors have the size and field offsets the C compiler gives the header's
    structs (a C program built against include/attn_decode.h prints them)."""
    import subprocess
    import tempfile

    structs = {"ad_decode_args": _abi.DecodeArgs, "ad_paged": _abi.Paged, "ad_sparse": _abi.Sparse}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "attn_decode.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'    printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'    printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["    return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        open(src, "w").write("\n".join(lines) + "\n")
        subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(x.split()[:2]): int(x.split()[2]) for x in out if x}
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, f"{cname}.{fname}"


# ------------------------------------------------------------------------------ rejection paths
def _tensors(dtype=torch.bfloat16, B=2, Q=1, Hq=8, Hkv=2, D=128, L=64):
    q = torch.zeros(B, Q, Hq, D, dtype=dtype)
    k = torch.zeros(B, Hkv, L, D, dtype=dtype).permute(0, 2, 1, 3)
    v = torch.zeros(B, Hkv, L, D, dtype=dtype).permute(0, 2, 1, 3)
    out = torch.zeros(B, Q, Hq, D, dtype=dtype)
    return q, k, v, out


def _args(**over):
    q, k, v, out = _tensors()
    a = _abi.make_args(q, k, v, scale=0.1, out=out)
    for key, val in over.items():
        setattr(a, key, val)
    return a, (q, k, v, out)


def _splitkv(a, sparse=None, S=2):
    po = torch.zeros(64, dtype=torch.float32)
    pl = torch.zeros(64, dtype=torch.float32)
    return _abi.lib().attn_decode_splitkv(ctypes.byref(a), None, ctypes.byref(sparse) if sparse else None, S,
                                          po.data_ptr(), pl.data_ptr(), None)


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 7, -2),
    ("num_q_heads", 7, -3),
    ("q_len", 0, -3),
    ("batch", -1, -3),
    ("head_dim_qk", 96, -5),
    ("head_dim_v", 64, -5),
    ("kv_len_max", -5, -7),
    ("window", -1, -7),
    ("causal", 2, -7),
    ("q", None, -1),
    ("k", None, -1),
    ("v", None, -1),
])
def test_splitkv_rejects(field, value, code):
    a, keep = _args(**{field: value})
    assert _splitkv(a) == code
    assert ad.attn_decode_last_error() != ""


def test_many_rows_per_kv_head_pass_validation():
    """32 and 128 query rows per KV head (grouped heads x speculative tokens) are accepted, bf16 and
    fp32 alike: the workspace query gets past every host check and sizes the partials."""
    for dtype, Hq, Q in ((torch.bfloat16, 32, 1), (torch.bfloat16, 32, 4), (torch.float32, 16, 2)):
        q, k, v, out = _tensors(dtype=dtype, Hq=Hq, Hkv=1, Q=Q)
        a = _abi.make_args(q, k, v, scale=0.1, out=out)
        rows = 2 * Q * Hq
        # the fixed arrival-counter region, then partial outputs and partial LSEs
        expect = (1 << 20) + -(-rows * 2 * 128 * 4 // 256) * 256 + -(-rows * 2 * 4 // 256) * 256
        assert _abi.lib().attn_decode_workspace_size(ctypes.byref(a), None, None, 2) == expect


def test_splitkv_rejects_misaligned_rows():
    q, k, v, out = _tensors()
    a = _abi.make_args(q, k, v, scale=0.1)
    a.q = a.q + 2  # one bf16 element off a 16-byte boundary
    assert _splitkv(a) == -4
    a, keep = _args()
    a.k_stride[1] = 129  # odd row pitch
    assert _splitkv(a) == -4


def test_splitkv_rejects_split_counts():
    a, keep = _args()
    assert _splitkv(a, S=-1) == -7
    assert _splitkv(a, S=_abi.AD_MAX_SPLITS + 1) == -7
    assert _splitkv(a, S=0 + 0, sparse=None) not in (-1, -2, -3, -4, -5, -6)  # 0 = plan (needs a GPU)


def test_splitkv_rejects_null_partials():
    a, keep = _args()
    assert _abi.lib().attn_decode_splitkv(ctypes.byref(a), None, None, 2, None, None, None) == -1


def test_splitkv_rejects_bad_block_lists():
    a, keep = _args()
    nb = torch.zeros(2, 2, dtype=torch.int32)
    ix = torch.zeros(2, 2, 4, dtype=torch.int32)
    for bs, code in ((24, -7), (8, -7), (8192, -7)):
        sp = _abi.make_sparse(nb, ix, bs)
        assert _splitkv(a, sparse=sp) == code
    sp = _abi.make_sparse(nb, ix, 128)
    sp.block_idx = None
    assert _splitkv(a, sparse=sp) == -1


def _paged_call(a, pg, ws_bytes=1 << 21, ws_ptr=None, S=2):
    ws = torch.zeros(ws_bytes + 256, dtype=torch.uint8)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    return _abi.lib().attn_decode_paged(ctypes.byref(a), ctypes.byref(pg) if pg else None, S,
                                        base if ws_ptr is None else ws_ptr, ws_bytes, None), ws


def test_paged_rejections():
    q, _, _, out = _tensors()
    pool = torch.zeros(10, 2, 16, 128, dtype=torch.bfloat16).permute(0, 2, 1, 3)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    a = _abi.make_args(q, pool, pool, scale=0.1, kv_len_max=64, out=out)
    assert _paged_call(a, None)[0] == -1
    for ps in (8, 48, 128):
        assert _paged_call(a, _abi.make_paged(bt, ps))[0] == -7
    short = torch.zeros(2, 3, dtype=torch.int32)  # 3 pages < ceil(64 / 16)
    assert _paged_call(a, _abi.make_paged(short, 16))[0] == -7
    pg = _abi.make_paged(bt, 16)
    assert _paged_call(a, pg, ws_ptr=0)[0] == -6
    ws = torch.zeros((1 << 20) + 512, dtype=torch.uint8)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    assert _abi.lib().attn_decode_paged(ctypes.byref(a), ctypes.byref(pg), 2, base + 16, 1 << 20, None) == -4
    a.out = None
    assert _paged_call(a, pg)[0] == -1
    # a block list over a paged cache
    po = torch.zeros(64)
    sp = _abi.make_sparse(torch.zeros(2, 2, dtype=torch.int32), torch.zeros(2, 2, 4, dtype=torch.int32), 16)
    assert _abi.lib().attn_decode_splitkv(ctypes.byref(a), ctypes.byref(pg), ctypes.byref(sp), 2, po.data_ptr(),
                                          po.data_ptr(), None) == -5


def test_paged_rejects_small_workspace():
    q, _, _, out = _tensors()
    pool = torch.zeros(10, 2, 16, 128, dtype=torch.bfloat16).permute(0, 2, 1, 3)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    a = _abi.make_args(q, pool, pool, scale=0.1, kv_len_max=64, out=out)
    pg = _abi.make_paged(bt, 16)
    # 2 splits: the 1 MiB arrival-counter region, then rows 16 * 2 * 128 * 4 = 16 KiB of partial
    # outputs + 256 B of LSEs
    need = (1 << 20) + 16384 + 256
    assert _abi.lib().attn_decode_workspace_size(ctypes.byref(a), ctypes.byref(pg), None, 2) == need
    assert _paged_call(a, pg, ws_bytes=need - 1)[0] == -6


def _decode_call(a, pg=None, sp=None, ws_bytes=1 << 21, ws_ptr=None, S=2):
    ws = torch.zeros(ws_bytes + 256, dtype=torch.uint8)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    return _abi.lib().attn_decode(ctypes.byref(a), ctypes.byref(pg) if pg else None, ctypes.byref(sp) if sp else None,
                                  S, base if ws_ptr is None else ws_ptr, ws_bytes, None), ws


def test_decode_rejections():
    """The one-launch entry checks its workspace, split count, output and cache arguments on the host."""
    a, keep = _args()
    assert _decode_call(a, ws_ptr=0)[0] == -6
    ws = torch.zeros((1 << 21) + 512, dtype=torch.uint8)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    assert _abi.lib().attn_decode(ctypes.byref(a), None, None, 2, base + 16, 1 << 21, None) == -4
    need = _abi.lib().attn_decode_workspace_size(ctypes.byref(a), None, None, 2)
    assert need > 0
    assert _decode_call(a, ws_bytes=need - 256)[0] == -6
    assert _decode_call(a, S=-1)[0] == -7
    assert _decode_call(a, S=_abi.AD_MAX_SPLITS + 1)[0] == -7
    nb = torch.zeros(2, 2, dtype=torch.int32)
    sp = _abi.make_sparse(nb, torch.zeros(2, 2, 4, dtype=torch.int32), 24)
    assert _decode_call(a, sp=sp)[0] == -7
    pg = _abi.make_paged(torch.zeros(2, 4, dtype=torch.int32), 16)
    sp = _abi.make_sparse(nb, torch.zeros(2, 2, 4, dtype=torch.int32), 16)
    assert _decode_call(a, pg=pg, sp=sp)[0] == -5
    a.out = None
    assert _decode_call(a)[0] == -1
    assert ad.attn_decode_last_error() != ""


def test_merge_rejections():
    L = _abi.lib()
    po = torch.zeros(4096, dtype=torch.float32)
    out = torch.zeros(2, 1, 8, 128, dtype=torch.bfloat16)
    s3 = _abi.I64x3(*out.stride()[:3])
    args = [po.data_ptr(), po.data_ptr(), None, 2, 2, 1, 8, 128, 1, out.data_ptr(), s3, None, None]

    def call(**kw):
        a = list(args)
        names = ["po", "pl", "spb", "S", "B", "Q", "Hq", "Dv", "dt", "out", "stride", "lse", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.attn_decode_merge(*a)

    assert call(po=None) == -1
    assert call(out=None) == -1
    assert call(dt=5) == -2
    assert call(S=0) == -7
    assert call(S=_abi.AD_MAX_SPLITS + 1) == -7
    assert call(Dv=96) == -5
    assert call(Q=0) == -3
    assert call(out=out.data_ptr() + 2) == -4
    assert call(spb=po.data_ptr() + 2) == -4   # splits_per_batch must be 4-byte aligned
    assert call(B=0) == 0  # nothing to merge: no launch, success


def test_mla_rejections():
    qn = torch.zeros(2, 1, 16, 512, dtype=torch.bfloat16)
    ckv = torch.zeros(8, 64, 1, 512, dtype=torch.bfloat16)
    kpe = torch.zeros(8, 64, 1, 64, dtype=torch.bfloat16)
    qpe = torch.zeros(2, 1, 16, 64, dtype=torch.bfloat16)
    out = torch.zeros(2, 1, 16, 512, dtype=torch.bfloat16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    a = _abi.make_args(qn, ckv, None, scale=0.1, kv_len_max=256, out=out, head_dim_qk=576)
    pg = _abi.make_paged(bt, 64)
    L = _abi.lib()
    ws = torch.zeros(1 << 20, dtype=torch.uint8)

    def call(args, kpe_p=kpe.data_ptr(), qpe_p=qpe.data_ptr()):
        return L.attn_decode_mla(ctypes.byref(args), kpe_p, _abi._s3(kpe), qpe_p, _abi._s3(qpe), ctypes.byref(pg),
                                 2, ws.data_ptr(), ws.numel(), None)

    assert call(a, kpe_p=None) == -1
    a.v = ckv.data_ptr() + 1024
    assert call(a) == -5  # values must be the latent rows themselves
    a.v = None
    a.head_dim_qk = 192
    assert call(a) == -5
    a.head_dim_qk = 576
    a.dtype = _abi.AD_F32
    assert call(a) == -5
    a.dtype = _abi.AD_BF16
    # the partial-pass-only entry point: same checks, then its own partial buffers
    po = torch.zeros(4096, dtype=torch.float32)

    def call_split(args, part_o=po.data_ptr(), part_lse=po.data_ptr(), kpe_p=kpe.data_ptr()):
        return L.attn_decode_mla_splitkv(ctypes.byref(args), kpe_p, _abi._s3(kpe), qpe.data_ptr(), _abi._s3(qpe),
                                         ctypes.byref(pg), 2, part_o, part_lse, None)

    assert call_split(a, kpe_p=None) == -1
    assert call_split(a, part_o=None) == -1
    assert call_split(a, part_o=po.data_ptr() + 4) == -4
    assert call_split(a, part_lse=po.data_ptr() + 2) == -4
    a.head_dim_v = 256
    assert call_split(a) == -5


def test_errors_raise_in_python():
    a, keep = _args(num_q_heads=7)
    with pytest.raises(_abi.ADError) as e:
        _abi.attn_decode_splitkv(a, None, None, 2, torch.zeros(16), torch.zeros(16))
    assert e.value.code == -3 and "multiple" in str(e.value)


def test_launch_count_query(monkeypatch):
    """attn_decode_launches reports one launch (merge inside the partial pass) or two (merge kernel
    after it), as AD_FUSED_MERGE forces here (no device query is made then), 0 for an empty batch,
    and checks its arguments like attn_decode."""
    a, keep = _args()
    monkeypatch.setenv("AD_FUSED_MERGE", "1")
    assert ad.attn_decode_launches(a, None, None, 2) == 1
    monkeypatch.setenv("AD_FUSED_MERGE", "0")
    assert ad.attn_decode_launches(a, None, None, 2) == 2
    b, keep2 = _args(batch=0)
    assert ad.attn_decode_launches(b, None, None, 2) == 0
    assert _abi.lib().attn_decode_launches(ctypes.byref(a), None, None, 2, None) == -1
    a.head_dim_qk = 96
    with pytest.raises(_abi.ADError):
        ad.attn_decode_launches(a, None, None, 2)


def test_fp8_cache_rejections():
    """An E4M3 cache: bf16 queries, head dim 128, both scale arrays, 4-byte aligned, not with MLA,
    and a known kv_format."""
    q, _, _, out = _tensors()
    kb = torch.zeros(2, 2, 64, 128, dtype=torch.uint8).permute(0, 2, 1, 3)
    ks = torch.ones(2, 2, 64, dtype=torch.float32).permute(0, 2, 1)
    a = _abi.make_args(q, kb, kb, scale=0.1, out=out, k_scale=ks, v_scale=ks)
    assert a.kv_format == _abi.AD_KV_FP8_E4M3
    ws = torch.zeros((1 << 21) + 256, dtype=torch.uint8)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256

    def call(args):
        return _abi.lib().attn_decode(ctypes.byref(args), None, None, 2, base, 1 << 21, None)

    b = _abi.make_args(q, kb, kb, scale=0.1, out=out, k_scale=ks, v_scale=ks)
    b.v_scale = None
    assert call(b) == -1
    b = _abi.make_args(q, kb, kb, scale=0.1, out=out, k_scale=ks, v_scale=ks)
    b.k_scale = b.k_scale + 2
    assert call(b) == -4
    b = _abi.make_args(q, kb, kb, scale=0.1, out=out, k_scale=ks, v_scale=ks)
    b.kv_format = 7
    assert call(b) == -2
    b = _abi.make_args(q, kb, kb, scale=0.1, out=out, k_scale=ks, v_scale=ks)
    b.head_dim_qk = b.head_dim_v = 64
    assert call(b) == -5
    q32, _, _, out32 = _tensors(dtype=torch.float32)
    b = _abi.make_args(q32, kb, kb, scale=0.1, out=out32, k_scale=ks, v_scale=ks)
    assert call(b) == -5
    b = _abi.make_args(q, kb, kb, scale=0.1, out=out, k_scale=ks, v_scale=ks)
    b.k_stride[1] = 136  # a byte row pitch that breaks 16-byte alignment
    assert call(b) == -4


def test_testing_aids_need_the_switch(monkeypatch):
    """Without AD_TEST_KNOBS=1 the testing aids are ignored: a kernel override changes nothing."""
    q, k, v, out = _tensors(Hq=2, Hkv=2)   # one query row per KV head: the vector kernel
    a = _abi.make_args(q, k, v, scale=0.1, out=out)
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "mfma")
    assert _abi.attn_decode_kernel(a) == _abi.AD_KERNEL_MATRIX16
    monkeypatch.setenv("AD_MFMA_TILE", "32")
    assert _abi.attn_decode_kernel(a) == _abi.AD_KERNEL_MATRIX
    monkeypatch.setenv("AD_TEST_KNOBS", "0")
    assert _abi.attn_decode_kernel(a) == _abi.AD_KERNEL_VECTOR
    monkeypatch.delenv("AD_TEST_KNOBS")
    assert _abi.attn_decode_kernel(a) == _abi.AD_KERNEL_VECTOR


def test_workspace_size_takes_the_block_list():
    """The workspace query plans with the block list the call will carry, and rejects what the
    calls reject (a block list over a paged cache) with a message."""
    a, keep = _args()
    nb = torch.zeros(2, 2, dtype=torch.int32)
    sp = _abi.make_sparse(nb, torch.zeros(2, 2, 4, dtype=torch.int32), 16)
    L = _abi.lib()
    assert L.attn_decode_workspace_size(ctypes.byref(a), None, ctypes.byref(sp), 2) == \
        L.attn_decode_workspace_size(ctypes.byref(a), None, None, 2)
    pg = _abi.make_paged(torch.zeros(2, 4, dtype=torch.int32), 16)
    assert L.attn_decode_workspace_size(ctypes.byref(a), ctypes.byref(pg), ctypes.byref(sp), 2) == 0
    assert "block list" in ad.attn_decode_last_error()
    bad = _abi.make_sparse(nb, torch.zeros(2, 2, 4, dtype=torch.int32), 24)
    assert L.attn_decode_workspace_size(ctypes.byref(a), None, ctypes.byref(bad), 2) == 0


def test_kernel_query(monkeypatch):
    """attn_decode_kernel names the partial-pass kernel: vector ALUs for up to 8 rows per KV head
    and for fp32, matrix cores for more bf16 rows and for every fp8 cache (16-row units up to 16
    rows per KV head, 32-row units above), the MLA kernel for the 576 / 512 head dims;
    AD_PARTIAL_KERNEL overrides the bf16 choice and AD_MFMA_TILE the matrix-core units."""
    monkeypatch.delenv("AD_PARTIAL_KERNEL", raising=False)
    monkeypatch.delenv("AD_MFMA_TILE", raising=False)
    a, keep = _args()  # 8 / 2 heads: 4 rows per KV head
    assert ad.attn_decode_kernel(a) == ad.AD_KERNEL_VECTOR
    q, k, v, out = _tensors(Hq=64, Hkv=2)
    assert ad.attn_decode_kernel(_abi.make_args(q, k, v, scale=0.1, out=out)) == ad.AD_KERNEL_MATRIX
    for Hq, kind in ((18, ad.AD_KERNEL_MATRIX16), (32, ad.AD_KERNEL_MATRIX16), (34, ad.AD_KERNEL_MATRIX)):
        q, k, v, out = _tensors(Hq=Hq, Hkv=2)   # 9, 16 and 17 rows per KV head
        assert ad.attn_decode_kernel(_abi.make_args(q, k, v, scale=0.1, out=out)) == kind, Hq
    monkeypatch.setenv("AD_MFMA_TILE", "32")
    assert ad.attn_decode_kernel(_abi.make_args(q, k, v, scale=0.1, out=out)) == ad.AD_KERNEL_MATRIX
    monkeypatch.setenv("AD_MFMA_TILE", "16")
    assert ad.attn_decode_kernel(_abi.make_args(q, k, v, scale=0.1, out=out)) == ad.AD_KERNEL_MATRIX16
    monkeypatch.delenv("AD_MFMA_TILE")
    assert ad.KERNEL_NAMES[ad.AD_KERNEL_MATRIX16] == "partial_mfma16_kernel"
    q32, k32, v32, o32 = _tensors(dtype=torch.float32, Hq=64, Hkv=2)
    assert ad.attn_decode_kernel(_abi.make_args(q32, k32, v32, scale=0.1, out=o32)) == ad.AD_KERNEL_VECTOR
    kb = torch.zeros(2, 2, 64, 128, dtype=torch.uint8).permute(0, 2, 1, 3)
    ks = torch.ones(2, 2, 64, dtype=torch.float32).permute(0, 2, 1)
    f = _abi.make_args(keep[0], kb, kb, scale=0.1, out=keep[3], k_scale=ks, v_scale=ks)
    assert ad.attn_decode_kernel(f) == ad.AD_KERNEL_MATRIX16
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "valu")
    assert ad.attn_decode_kernel(f) == ad.AD_KERNEL_VECTOR
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "mfma")
    assert ad.attn_decode_kernel(a) == ad.AD_KERNEL_MATRIX16
    qm = torch.zeros(2, 1, 16, 512, dtype=torch.bfloat16)
    ckv = torch.zeros(4, 64, 1, 512, dtype=torch.bfloat16)
    m = _abi.make_args(qm, ckv, None, head_dim_qk=576, scale=0.1)
    assert ad.attn_decode_kernel(m) == ad.AD_KERNEL_MLA
    assert ad.KERNEL_NAMES[ad.AD_KERNEL_MLA] == "mla_partial_kernel"
    assert _abi.lib().attn_decode_kernel(ctypes.byref(a), None) == -1
    a.head_dim_qk = 96
    with pytest.raises(_abi.ADError):
        ad.attn_decode_kernel(a)


def test_spec_decoding_rejections():
    """Tree masks cover at most 64 query tokens; q_starts and tree_mask must be 4-byte aligned;
    MLA takes neither. Checked before any device work."""
    q, k, v, out = _tensors(Q=1)
    qp = torch.zeros(5, 8, 128, dtype=torch.bfloat16)
    outp = torch.zeros(5, 8, 128, dtype=torch.bfloat16)
    starts = torch.tensor([0, 3, 5], dtype=torch.int32)
    mask = torch.zeros(5, 3, dtype=torch.int32)
    a = _abi.make_args(qp, k, v, scale=0.1, out=outp, q_starts=starts, q_len=65, tree_mask=mask)
    assert a.batch == 2 and a.q_len == 65 and a.q_stride[1] == 8 * 128 and a.q_stride[2] == 128
    assert _abi.lib().attn_decode_kernel(ctypes.byref(a), ctypes.byref(ctypes.c_int32())) == -5
    a.q_len = 64
    assert ad.attn_decode_kernel(a) == ad.AD_KERNEL_MATRIX  # 4 heads x 64 rows per KV head
    a.tree_mask = a.tree_mask + 2
    assert _abi.lib().attn_decode_kernel(ctypes.byref(a), ctypes.byref(ctypes.c_int32())) == -4
    a.tree_mask, a.q_starts = None, a.q_starts + 1
    assert _abi.lib().attn_decode_kernel(ctypes.byref(a), ctypes.byref(ctypes.c_int32())) == -4
    qm = torch.zeros(2, 16, 512, dtype=torch.bfloat16)
    ckv = torch.zeros(4, 64, 1, 512, dtype=torch.bfloat16)
    m = _abi.make_args(qm, ckv, None, head_dim_qk=576, scale=0.1, q_starts=starts, q_len=1)
    assert _abi.lib().attn_decode_kernel(ctypes.byref(m), ctypes.byref(ctypes.c_int32())) == -5
    m = _abi.make_args(qm[None], ckv, None, head_dim_qk=576, scale=0.1, tree_mask=mask)
    assert _abi.lib().attn_decode_kernel(ctypes.byref(m), ctypes.byref(ctypes.c_int32())) == -5


def test_int4_cache_rejections(monkeypatch):
    """An int4 cache: bf16 queries, head dim 128, kv_groups 1/2/4/8, 4-byte aligned rows, not with
    MLA; rows of one group on the 16-row matrix-core kernel (the vector kernel on request), rows of
    more groups always on the vector kernel."""
    q, _, _, out = _tensors()
    kw = torch.zeros(2, 2, 64, 17, dtype=torch.int32).permute(0, 2, 1, 3)
    a = _abi.make_args(q, kw, kw, scale=0.1, out=out)
    assert a.kv_format == _abi.AD_KV_INT4 and a.kv_groups == 1 and a.head_dim_v == 128

    def kind(args):
        return _abi.lib().attn_decode_kernel(ctypes.byref(args), ctypes.byref(ctypes.c_int32()))

    assert kind(a) == 0 and ad.attn_decode_kernel(a) == ad.AD_KERNEL_MATRIX16
    monkeypatch.setenv("AD_MFMA_TILE", "32")   # the int4 form exists in 16-row units only
    assert ad.attn_decode_kernel(a) == ad.AD_KERNEL_MATRIX16
    monkeypatch.delenv("AD_MFMA_TILE")
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "valu")
    assert ad.attn_decode_kernel(a) == ad.AD_KERNEL_VECTOR
    a.kv_groups = 4
    monkeypatch.setenv("AD_PARTIAL_KERNEL", "mfma")
    assert ad.attn_decode_kernel(a) == ad.AD_KERNEL_VECTOR
    monkeypatch.delenv("AD_PARTIAL_KERNEL")
    assert ad.attn_decode_kernel(a) == ad.AD_KERNEL_VECTOR
    a.kv_groups = 1
    b = _abi.make_args(q, kw, kw, scale=0.1, out=out)
    b.kv_groups = 3
    assert kind(b) == -7
    b = _abi.make_args(q, kw, kw, scale=0.1, out=out)
    b.k = b.k + 2
    assert kind(b) == -4
    b = _abi.make_args(q, kw, kw, scale=0.1, out=out)
    b.k_stride[1] = 17  # any word stride is fine for int4 rows
    assert kind(b) == 0
    q32, _, _, out32 = _tensors(dtype=torch.float32)
    assert kind(_abi.make_args(q32, kw, kw, scale=0.1, out=out32)) == -5
    b = _abi.make_args(q, kw, kw, scale=0.1, out=out)
    b.head_dim_qk = b.head_dim_v = 64
    assert kind(b) == -5


def test_read_probe_rejections():
    L = _abi.lib()
    buf = torch.zeros(1024, dtype=torch.int32)
    sink = torch.zeros(_abi.AD_PROBE_SINK_WORDS, dtype=torch.int32)
    assert L.attn_decode_read_probe(None, 64, sink.data_ptr(), None) == -1
    assert L.attn_decode_read_probe(buf.data_ptr(), 64, None, None) == -1
    assert L.attn_decode_read_probe(buf.data_ptr() + 4, 64, sink.data_ptr(), None) == -4
    assert L.attn_decode_read_probe(buf.data_ptr(), 0, sink.data_ptr(), None) == -7
    assert L.attn_decode_read_probe(buf.data_ptr(), 40, sink.data_ptr(), None) == -7


def test_noalloc_rejects_a_step_beyond_its_scratch():
    """A step whose workspace exceeds the library's own array is rejected on the host, before any
    HIP call: 2048 query rows x 256 splits x 129 words is far beyond 32 MiB."""
    q, k, v, out = _tensors(B=64, Hq=32, Hkv=8)
    a = _abi.make_args(q, k, v, scale=0.1, out=out)
    rc = _abi.lib().attn_decode_noalloc(ctypes.byref(a), None, None, 256, None)
    assert rc == -7
    assert "scratch" in ad.attn_decode_last_error()
    assert _abi.lib().attn_decode_noalloc(None, None, None, 2, None) == -1


def test_split_page_map_limit():
    """A split of a paged cache stages its page ids in LDS: 1038 pages of keys per split (258 for
    MLA), plus two for a split that starts inside a page. With the count forced, a split of
    exactly that many pages is planned and one page more is refused (the workspace query returns
    0 and names the limit)."""
    L = _abi.lib()
    for mla, limit in ((False, 1038), (True, 258)):
        for pages, ok in ((limit, True), (limit + 1, False)):
            keys = 16 * pages
            if mla:
                q = torch.zeros(1, 1, 16, 512, dtype=torch.bfloat16)
                ckv = torch.zeros(pages + 2, 16, 1, 512, dtype=torch.bfloat16)
                a = _abi.make_args(q, ckv, None, scale=0.1, kv_len_max=keys, out=q.clone(), head_dim_qk=576)
            else:
                q = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
                pool = torch.zeros(pages + 2, 1, 16, 128, dtype=torch.bfloat16).permute(0, 2, 1, 3)
                a = _abi.make_args(q, pool, pool, scale=0.1, kv_len_max=keys, out=q.clone())
            pg = _abi.make_paged(torch.zeros(1, pages + 2, dtype=torch.int32), 16)
            n = L.attn_decode_workspace_size(ctypes.byref(a), ctypes.byref(pg), None, 1)
            assert (n > 0) == ok, (mla, pages, n, _abi.attn_decode_last_error())
            if not ok:
                assert "pages/blocks per split" in _abi.attn_decode_last_error()


def test_work_unit_limit():
    """The whole-step entry keeps one 4-byte arrival counter per work unit (sequence x KV head x
    block of query rows) in a fixed 1 MiB region: 262,144 units at most. One unit more is refused
    on the host, before any HIP call. (A call at the limit would go on to launch, so it is not
    made here: the pointers are host memory.)"""
    limit = (1 << 20) // 4
    a, keep = _args()
    a.num_q_heads, a.num_kv_heads = 16, 4   # 4 rows per KV head: one row block per KV head
    a.batch = limit // 4 + 1                # one sequence past the limit; no kernel reads the strides
    a.q_stride[0] = a.k_stride[0] = a.v_stride[0] = a.out_stride[0] = 0
    a.q_stride[2] = a.out_stride[2] = a.k_stride[2] = a.v_stride[2] = 0
    assert _decode_call(a)[0] == -5
    assert "work units" in _abi.attn_decode_last_error()
