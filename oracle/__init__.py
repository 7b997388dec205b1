"""fp64 CPU oracle for single-step decode attention -- test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. The product package (``attention_decode_amd``) never imports it, and the
two share no code: this wrapper only marshals CPU tensors into the plain C loops of
``oracle.c`` (see that file's header for the definition and the passages it follows).

Layout conventions (all element strides, last dimension contiguous):
  q, q2          [batch, q_len, num_q_heads, dim]
  k, k2, v       contiguous cache: [batch, kv_len, num_kv_heads, dim]
                 paged cache:      [num_pages, page_size, num_kv_heads, dim] + block_table
Any tensor may be a permuted view (for example a head-major cache viewed token-major).
A quantised cache passes k and v as uint8 OCP E4M3 bytes with k_scale / v_scale: fp32
[batch, kv_len, num_kv_heads] (paged: [num_pages, page_size, num_kv_heads]) views of the row
scales, any strides (zero strides broadcast one scale).
Variable query lengths: with q_starts ([batch + 1] packed token offsets) q (and q2) are packed
[tokens, num_q_heads, dim], q_len (the largest per-sequence count, the tree-mask row pitch) is
passed explicitly, and out / lse come back packed as [tokens, num_q_heads, ...]. A tree mask is
int32/uint32 [token rows, ceil(q_len / 32)] (bit i of a row: draft key i visible).
An int4 cache passes k and v as int32 views [..., n_groups + dim / 8] (coefficient words, then
the packed values; see oracle.c) with int4_groups = n_groups; dim_v is then dim_qk.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16, E4M3, INT4 = 0, 1, 2, 3, 4
_TYPE = {torch.float64: F64, torch.float32: F32, torch.bfloat16: BF16, torch.uint8: E4M3, torch.int32: INT4}


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("dim_qk", ctypes.c_int32), ("dim_qk2", ctypes.c_int32), ("dim_v", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("q_type", ctypes.c_int32), ("kv_type", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_stride", ctypes.c_int64 * 3),
        ("q2", ctypes.c_void_p), ("q2_stride", ctypes.c_int64 * 3),
        ("k", ctypes.c_void_p), ("k_stride", ctypes.c_int64 * 3),
        ("k2", ctypes.c_void_p), ("k2_stride", ctypes.c_int64 * 3),
        ("v", ctypes.c_void_p), ("v_stride", ctypes.c_int64 * 3),
        ("seq_lens", ctypes.c_void_p), ("kv_len", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int64), ("page_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_void_p), ("nb_stride", ctypes.c_int64 * 2),
        ("block_idx", ctypes.c_void_p), ("idx_stride", ctypes.c_int64 * 3), ("block_size", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("key_lo", ctypes.c_int32), ("key_hi", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p), ("ks_stride", ctypes.c_int64 * 3),
        ("v_scale", ctypes.c_void_p), ("vs_stride", ctypes.c_int64 * 3),
        ("q_starts", ctypes.c_void_p), ("tree_mask", ctypes.c_void_p),
        ("n_groups", ctypes.c_int32),
    ]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math: IEEE fp64 throughout)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror",
           source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


class Oracle:
    """ctypes handle on one build of oracle.c."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_attend.argtypes = [ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_attend.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_merge.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_get_threads.restype = ctypes.c_int
        self.lib = lib

    # ------------------------------------------------------------------ helpers
    @staticmethod
    def _strides3(t: torch.Tensor):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("expected a 4-D tensor with a contiguous last dimension")
        return (ctypes.c_int64 * 3)(*t.stride()[:3])

    @staticmethod
    def _cpu(t):
        if t is None:
            return None
        if not isinstance(t, torch.Tensor):
            t = torch.as_tensor(t)
        if t.device.type != "cpu":
            raise ValueError("the oracle takes CPU tensors")
        return t

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    def threads(self) -> int:
        return int(self.lib.oracle_get_threads())

    # ------------------------------------------------------------------ attention
    def attend(self, q, k, v, *, scale: float, seq_lens=None, kv_len: int | None = None,
               q2=None, k2=None, block_table=None, page_size: int = 0,
               num_blocks=None, block_idx=None, block_size: int = 0,
               causal: bool = False, window: int = 0, key_range=None, rows=None, k_scale=None, v_scale=None,
               q_starts=None, q_len: int | None = None, tree_mask=None, int4_groups: int = 0):
        """Returns (out, lse) as float64 numpy arrays.

        out is [batch, q_len, num_q_heads, dim_v] (packed [tokens, num_q_heads, dim_v] with
        q_starts; [len(rows), dim_v] when rows is given) and lse has the same leading shape. Rows
        are flat indices n*num_q_heads + hq of token row n = b*q_len + t (q_starts[b] + t).
        """
        q, k, v, q2, k2 = (self._cpu(x) for x in (q, k, v, q2, k2))
        keep = [q, k, v, q2, k2]
        qs = None
        if q_starts is not None:  # packed queries: view them as [1, tokens, Hq, D] for the strides
            qs = self._cpu(q_starts).to(torch.int32).contiguous()
            keep.append(qs)
            if q.dim() != 3 or q_len is None:
                raise ValueError("with q_starts, q is packed [tokens, heads, dim] and q_len is given")
            q = q.unsqueeze(0)
            q2 = None if q2 is None else q2.unsqueeze(0)
            keep += [q, q2]
        _, Q, Hq, Dqk = q.shape
        B = q.shape[0]
        if qs is not None:
            B, Q = qs.numel() - 1, int(q_len)
        Hkv = k.shape[2]
        if q.dtype not in _TYPE or k.dtype not in _TYPE or v.dtype != k.dtype or q.dtype in (torch.uint8, torch.int32):
            raise ValueError("unsupported element types")
        if (k.dtype == torch.int32) != (int4_groups > 0):
            raise ValueError("an int4 (int32) cache needs int4_groups, and only it takes them")
        if int4_groups and k.shape[3] != int4_groups + Dqk // 8:
            raise ValueError("int4 rows hold n_groups coefficient words and dim / 8 packed words")
        if (k.dtype == torch.uint8) != (k_scale is not None and v_scale is not None):
            raise ValueError("an fp8 (uint8) cache needs k_scale and v_scale, and only it takes them")
        P = Problem()
        P.batch, P.q_len, P.num_q_heads, P.num_kv_heads = B, Q, Hq, Hkv
        P.dim_qk, P.dim_v = Dqk, (Dqk if int4_groups else v.shape[3])
        P.n_groups = int(int4_groups)
        P.scale = float(scale)
        P.q_type, P.kv_type = _TYPE[q.dtype], _TYPE[k.dtype]
        P.q, P.q_stride = q.data_ptr(), self._strides3(q)
        P.k, P.k_stride = k.data_ptr(), self._strides3(k)
        P.v, P.v_stride = v.data_ptr(), self._strides3(v)
        if q2 is not None:
            if q2.dtype != q.dtype or k2.dtype != k.dtype:
                raise ValueError("q2/k2 must match q/k element types")
            P.dim_qk2 = q2.shape[3]
            P.q2, P.q2_stride = q2.data_ptr(), self._strides3(q2)
            P.k2, P.k2_stride = k2.data_ptr(), self._strides3(k2)
        if seq_lens is not None:
            sl = self._cpu(seq_lens).to(torch.int32).contiguous()
            keep.append(sl)
            P.seq_lens = sl.data_ptr()
        else:
            if kv_len is None:
                if block_table is not None:
                    raise ValueError("a paged cache needs seq_lens or kv_len")
                kv_len = k.shape[1]
            P.kv_len = int(kv_len)
        if block_table is not None:
            bt = self._cpu(block_table).to(torch.int32).contiguous()
            keep.append(bt)
            P.block_table, P.bt_stride, P.page_size = bt.data_ptr(), bt.stride(0), int(page_size)
        if num_blocks is not None:
            nb = self._cpu(num_blocks).to(torch.int32).contiguous()
            ix = self._cpu(block_idx).to(torch.int32).contiguous()
            keep += [nb, ix]
            P.num_blocks, P.nb_stride = nb.data_ptr(), (ctypes.c_int64 * 2)(*nb.stride())
            P.block_idx, P.idx_stride = ix.data_ptr(), (ctypes.c_int64 * 3)(*ix.stride())
            P.block_size = int(block_size)
        if k_scale is not None:
            ks, vs = self._cpu(k_scale), self._cpu(v_scale)
            if ks.dtype != torch.float32 or vs.dtype != torch.float32 or ks.dim() != 3 or vs.dim() != 3:
                raise ValueError("k_scale / v_scale must be 3-D float32 views")
            keep += [ks, vs]
            P.k_scale, P.ks_stride = ks.data_ptr(), (ctypes.c_int64 * 3)(*ks.stride())
            P.v_scale, P.vs_stride = vs.data_ptr(), (ctypes.c_int64 * 3)(*vs.stride())
        P.causal, P.window = int(bool(causal)), int(window)
        if qs is not None:
            P.q_starts = qs.data_ptr()
        if tree_mask is not None:
            tm = self._cpu(tree_mask).to(torch.int32).contiguous()
            if tm.dim() != 2 or tm.shape[1] != (Q + 31) // 32:
                raise ValueError("tree_mask must be [token rows, ceil(q_len / 32)]")
            keep.append(tm)
            P.tree_mask = tm.data_ptr()
        if key_range is None:
            P.key_lo, P.key_hi = 0, -1
        else:
            P.key_lo, P.key_hi = int(key_range[0]), int(key_range[1])

        Dv = P.dim_v
        tokens = int(qs[-1]) if qs is not None else B * Q
        if rows is None:
            n = tokens * Hq
            rows_arr = None
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            n = rows_arr.size
        out = np.zeros((n, Dv), dtype=np.float64)
        lse = np.zeros((n,), dtype=np.float64)
        rc = self.lib.oracle_attend(ctypes.byref(P),
                                    None if rows_arr is None else rows_arr.ctypes.data,
                                    n, out.ctypes.data, lse.ctypes.data)
        del keep
        if rc != 0:
            raise ValueError(f"oracle_attend rejected the problem (rc={rc})")
        if rows is None:
            if qs is not None:
                return out.reshape(tokens, Hq, Dv), lse.reshape(tokens, Hq)
            return out.reshape(B, Q, Hq, Dv), lse.reshape(B, Q, Hq)
        return out, lse

    # ------------------------------------------------------------------ merge
    def merge(self, part_o, part_lse):
        """part_o [rows, S, Dv], part_lse [rows, S] (float64-convertible) -> (out [rows, Dv], lse [rows])."""
        po = np.ascontiguousarray(np.asarray(part_o, dtype=np.float64))
        pl = np.ascontiguousarray(np.asarray(part_lse, dtype=np.float64))
        rows, S, Dv = po.shape
        if pl.shape != (rows, S):
            raise ValueError("part_lse must be [rows, splits]")
        out = np.zeros((rows, Dv), dtype=np.float64)
        lse = np.zeros((rows,), dtype=np.float64)
        rc = self.lib.oracle_merge(rows, S, Dv, po.ctypes.data, pl.ctypes.data, out.ctypes.data,
                                   lse.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_merge rejected its arguments (rc={rc})")
        return out, lse


_DEFAULT: Oracle | None = None


def load() -> Oracle:
    """The oracle built in-tree, compiled first if no build is present."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
