"""CPU bounds check of the MLA partial pass's HBM -> LDS copies and LDS accesses
(tests/mla_layout_check.cpp, built here with g++ against the kernel's own offset header): on the
full MLA workload at its planned split, on the small MLA parity cases at several split counts, and
on poisoned pools. No GPU is used."""
import ctypes
import os
import subprocess
import tempfile

import pytest
import torch

from attention_decode_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


class Geometry(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_splits", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("bt_stride", ctypes.c_int64), ("pool_pages", ctypes.c_int64), ("ckv_s", ctypes.c_int64 * 2),
                ("kpe_s", ctypes.c_int64 * 2), ("ckv_elems", ctypes.c_int64), ("kpe_elems", ctypes.c_int64),
                ("q_s0", ctypes.c_int64), ("q2_s0", ctypes.c_int64), ("q_elems", ctypes.c_int64),
                ("q2_elems", ctypes.c_int64)]


@pytest.fixture(scope="module")
def checker():
    d = tempfile.mkdtemp(prefix="mla_layout_")
    so = os.path.join(d, "mla_layout_check.so")
    subprocess.run(["g++", "-std=c++17", "-O2", "-shared", "-fPIC", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "attention_decode_amd", "csrc"),
                    os.path.join(HERE, "mla_layout_check.cpp"), "-o", so], check=True)
    lib = ctypes.CDLL(so)
    lib.mla_layout_check.argtypes = [ctypes.POINTER(Geometry), ctypes.c_char_p, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_long)]
    lib.mla_layout_check.restype = ctypes.c_int
    return lib


def chunk_of(kv_len_max, S):
    return max(-(-(-(-kv_len_max // S)) // 16) * 16, 16)


def check(lib, w, S, chunk=None):
    sl = w.seq_lens.to(torch.int32).contiguous()
    bt = w.block_table.to(torch.int32).contiguous()
    g = Geometry()
    g.batch, g.num_splits, g.page_size = w.batch, S, w.page_size
    g.chunk = chunk_of(w.kv_len_max, S) if chunk is None else chunk
    g.seq_lens, g.block_table, g.bt_stride = sl.data_ptr(), bt.data_ptr(), bt.stride(0)
    g.pool_pages = w.k.shape[0]
    g.ckv_s = (ctypes.c_int64 * 2)(w.k.stride(0), w.k.stride(1))
    g.kpe_s = (ctypes.c_int64 * 2)(w.kpe.stride(0), w.kpe.stride(1))
    g.ckv_elems, g.kpe_elems = w.k.numel(), w.kpe.numel()
    g.q_s0, g.q2_s0 = w.q.stride(0), w.q_pe.stride(0)
    g.q_elems, g.q2_elems = w.q.numel(), w.q_pe.numel()
    msg = ctypes.create_string_buffer(512)
    n = ctypes.c_long(0)
    rc = lib.mla_layout_check(ctypes.byref(g), msg, 512, ctypes.byref(n))
    assert rc == 0, msg.value.decode()
    return n.value


def test_full_mla_workload(checker):
    """32 sequences of 8192 keys on 64-key pages, 4 splits of 2048 keys (the plan for 256 CUs) and 8
    of 1024."""
    n = check(checker, inputs.make(5), 4)
    assert n > 10 ** 7
    n = check(checker, inputs.make(5), 8)
    assert n > 10 ** 7


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("H,page,lens,Q", [
    (128, 64, [1, 31, 33, 700], 1), (128, 16, [64, 1000, 5], 1), (16, 32, [300, 2], 1),
    (160, 64, [257, 90], 1), (64, 16, [500, 77], 2), (32, 64, [640, 129], 3), (128, 16, [4128, 17], 1),
])
def test_small_mla_cases(checker, H, page, lens, Q, S):
    w = inputs.mla(batch=len(lens), num_heads=H, kv_len=max(lens), page_size=page, seq_lens=lens, q_len=Q, seed=3)
    check(checker, w, S)


@pytest.mark.parametrize("S", [1, 4])
def test_poisoned_pools(checker, S):
    for lens, page in (([5, 64, 250, 1000, 31], 16), ([8192, 1, 4000], 64)):
        w = inputs.mla(batch=len(lens), num_heads=128, kv_len=max(lens), page_size=page, seq_lens=lens, seed=9,
                       poison=True)
        check(checker, w, S)


def test_a_misplaced_split_is_caught(checker):
    """The check is not vacuous. Splits must start on 16-key boundaries (the planner rounds the
    split length up to 16) so that each wave's group of 8 rotary rows lies in one page; with splits
    of 12 keys a group crosses a page boundary, its lanes past the boundary would read the next
    slots of the old page, and the check reports exactly that."""
    w = inputs.mla(batch=1, num_heads=16, kv_len=300, page_size=16, seq_lens=[300], seed=4)
    check(checker, w, 25, chunk=16 * 1)                     # 16-key splits: fine
    with pytest.raises(AssertionError, match="rotary copy reads another key's row"):
        check(checker, w, 25, chunk=12)
