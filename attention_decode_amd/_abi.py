"""ctypes binding of include/attn_decode.h.

Argument marshalling only: every function here fills the C descriptors from torch tensors
(device memory, element strides, the current HIP stream) and calls the library. All of the
decode step runs in the library's HIP kernels. There is no fallback: if the library is not
built, or a call is rejected, an exception says so.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libattn_decode.so")

AD_F32, AD_BF16 = 0, 1
AD_KV_SAME, AD_KV_FP8_E4M3, AD_KV_INT4 = 0, 1, 2
AD_KERNEL_VECTOR, AD_KERNEL_MATRIX, AD_KERNEL_MLA, AD_KERNEL_MATRIX16 = 0, 1, 2, 3
AD_MAX_SPLITS = 256
AD_PROBE_SINK_WORDS = 4096
AD_NOALLOC_SCRATCH_BYTES = 32 << 20
STATUS = {0: "AD_OK", -1: "AD_E_NULL", -2: "AD_E_DTYPE", -3: "AD_E_SHAPE", -4: "AD_E_ALIGN",
          -5: "AD_E_UNSUPPORTED", -6: "AD_E_WORKSPACE", -7: "AD_E_RANGE"}
_DTYPE = {torch.float32: AD_F32, torch.bfloat16: AD_BF16}

I64x3 = ctypes.c_int64 * 3


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_stride", I64x3),
        ("k", ctypes.c_void_p), ("k_stride", I64x3),
        ("v", ctypes.c_void_p), ("v_stride", I64x3),
        ("seq_lens", ctypes.c_void_p), ("kv_len_max", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("out_stride", I64x3),
        ("lse", ctypes.c_void_p),
        ("kv_format", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p), ("k_scale_stride", I64x3),
        ("v_scale", ctypes.c_void_p), ("v_scale_stride", I64x3),
        ("q_starts", ctypes.c_void_p), ("tree_mask", ctypes.c_void_p),
        ("kv_groups", ctypes.c_int32),
    ]


class Paged(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int64), ("page_size", ctypes.c_int32)]


class Sparse(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_void_p), ("block_idx", ctypes.c_void_p),
                ("nb_stride", ctypes.c_int64 * 2), ("idx_stride", I64x3),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32)]


class ADError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}: {msg}")
        self.code = code


_LIB = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it with `python -m attention_decode_amd.build` "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIBRARY)
        P = ctypes.POINTER
        L.attn_decode_plan.argtypes = [P(DecodeArgs), P(Paged), P(Sparse), P(ctypes.c_int32), P(ctypes.c_int32)]
        L.attn_decode_workspace_size.argtypes = [P(DecodeArgs), P(Paged), P(Sparse), ctypes.c_int32]
        L.attn_decode_workspace_size.restype = ctypes.c_size_t
        L.attn_decode_splitkv.argtypes = [P(DecodeArgs), P(Paged), P(Sparse), ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
        L.attn_decode_merge.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, P(ctypes.c_int64), ctypes.c_void_p,
                                        ctypes.c_void_p]
        L.attn_decode.argtypes = [P(DecodeArgs), P(Paged), P(Sparse), ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]
        L.attn_decode_noalloc.argtypes = [P(DecodeArgs), P(Paged), P(Sparse), ctypes.c_int32, ctypes.c_void_p]
        L.attn_decode_noalloc.restype = ctypes.c_int
        L.attn_decode_launches.argtypes = [P(DecodeArgs), P(Paged), P(Sparse), ctypes.c_int32, P(ctypes.c_int32)]
        L.attn_decode_kernel.argtypes = [P(DecodeArgs), P(ctypes.c_int32)]
        L.attn_decode_paged.argtypes = [P(DecodeArgs), P(Paged), ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
        L.attn_decode_mla.argtypes = [P(DecodeArgs), ctypes.c_void_p, P(ctypes.c_int64), ctypes.c_void_p,
                                      P(ctypes.c_int64), P(Paged), ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
        L.attn_decode_mla_splitkv.argtypes = [P(DecodeArgs), ctypes.c_void_p, P(ctypes.c_int64), ctypes.c_void_p,
                                              P(ctypes.c_int64), P(Paged), ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]
        L.attn_decode_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.attn_decode_read_probe.restype = ctypes.c_int
        L.attn_decode_last_error.restype = ctypes.c_char_p
        for fn in ("attn_decode", "attn_decode_launches", "attn_decode_kernel", "attn_decode_plan", "attn_decode_splitkv", "attn_decode_merge", "attn_decode_paged",
                   "attn_decode_mla", "attn_decode_mla_splitkv"):
            getattr(L, fn).restype = ctypes.c_int
        _LIB = L
    return _LIB


def attn_decode_last_error() -> str:
    return lib().attn_decode_last_error().decode()


def _check(fn, rc):
    if rc != 0:
        raise ADError(fn, rc, attn_decode_last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _s3(t):
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor")
    return I64x3(*t.stride()[:3])


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_args(q, k, v, *, scale, seq_lens=None, kv_len_max=None, causal=False, window=0, out=None, lse=None,
              head_dim_qk=None, k_scale=None, v_scale=None, q_starts=None, q_len=None, tree_mask=None):
    """Fill an ad_decode_args from tensors (q [B,Q,Hq,D]; k/v token-major 4-D views). uint8 k / v
    are an E4M3 cache, with k_scale / v_scale fp32 3-D views indexed like the cache rows.
    Variable query lengths: q_starts int32 [B + 1] with q (and out) packed [tokens, Hq, D] and
    q_len the largest per-sequence count. tree_mask: int32 [token rows, ceil(q_len / 32)].
    int32 k / v are an int4 cache: rows of n_groups coefficient words then D / 8 packed words
    (n_groups is read off the row length)."""
    a = DecodeArgs()
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    a.dtype = _DTYPE[q.dtype]
    if q_starts is not None:  # packed rows: view as [1, tokens, Hq, D]; q_stride[0] is unused
        if q.dim() != 3 or q_len is None:
            raise ValueError("with q_starts, q is packed [tokens, heads, dim] and q_len is given")
        q = q.unsqueeze(0)
        out = None if out is None else out.unsqueeze(0)
        a.q_starts = _ptr(q_starts)
    a.tree_mask = _ptr(tree_mask)
    a.batch, a.q_len, a.num_q_heads = q.shape[0], q.shape[1], q.shape[2]
    if q_starts is not None:
        a.batch, a.q_len = q_starts.numel() - 1, int(q_len)
    a.num_kv_heads = k.shape[2]
    a.head_dim_qk = q.shape[3] if head_dim_qk is None else head_dim_qk
    a.head_dim_v = (v if v is not None else k).shape[3]
    if k.dtype == torch.int32:
        a.kv_format = AD_KV_INT4
        a.kv_groups = k.shape[3] - q.shape[3] // 8
        a.head_dim_v = q.shape[3]
    a.scale = float(scale)
    a.q, a.q_stride = _ptr(q), _s3(q)
    a.k, a.k_stride = _ptr(k), _s3(k)
    if v is not None:
        a.v, a.v_stride = _ptr(v), _s3(v)
    a.seq_lens = _ptr(seq_lens)
    a.kv_len_max = int(k.shape[1] if kv_len_max is None else kv_len_max)
    a.causal, a.window = int(bool(causal)), int(window)
    if k.dtype == torch.uint8:
        if k_scale is None or v_scale is None or k_scale.dim() != 3 or v_scale.dim() != 3:
            raise ValueError("an E4M3 (uint8) cache needs 3-D k_scale and v_scale")
        a.kv_format = AD_KV_FP8_E4M3
        a.k_scale, a.k_scale_stride = _ptr(k_scale), I64x3(*k_scale.stride())
        a.v_scale, a.v_scale_stride = _ptr(v_scale), I64x3(*v_scale.stride())
    if out is not None:
        a.out, a.out_stride = _ptr(out), _s3(out)
    a.lse = _ptr(lse)
    return a


def make_paged(block_table, page_size):
    p = Paged()
    p.block_table = _ptr(block_table)
    p.bt_stride = block_table.stride(0)
    p.page_size = int(page_size)
    return p


def make_sparse(num_blocks, block_idx, block_size):
    s = Sparse()
    s.num_blocks, s.block_idx = _ptr(num_blocks), _ptr(block_idx)
    s.nb_stride = (ctypes.c_int64 * 2)(*num_blocks.stride())
    s.idx_stride = I64x3(*block_idx.stride())
    s.block_size = int(block_size)
    s.max_blocks = int(block_idx.shape[-1])
    return s


# ------------------------------------------------------------------------------ entry points
def attn_decode_plan(args: DecodeArgs, paged: Paged | None = None, sparse: Sparse | None = None):
    S, C = ctypes.c_int32(), ctypes.c_int32()
    _check("attn_decode_plan", lib().attn_decode_plan(ctypes.byref(args), ctypes.byref(paged) if paged else None,
                                                      ctypes.byref(sparse) if sparse else None,
                                                      ctypes.byref(S), ctypes.byref(C)))
    return S.value, C.value


def attn_decode_workspace_size(args: DecodeArgs, paged: Paged | None = None, num_splits: int = 0,
                               sparse: Sparse | None = None) -> int:
    n = lib().attn_decode_workspace_size(ctypes.byref(args), ctypes.byref(paged) if paged else None,
                                         ctypes.byref(sparse) if sparse else None, num_splits)
    if n == 0:
        raise ADError("attn_decode_workspace_size", 0, attn_decode_last_error())
    return n


def attn_decode_splitkv(args: DecodeArgs, paged: Paged | None, sparse: Sparse | None, num_splits: int, part_o,
                        part_lse, stream=None):
    _check("attn_decode_splitkv",
           lib().attn_decode_splitkv(ctypes.byref(args), ctypes.byref(paged) if paged else None,
                                     ctypes.byref(sparse) if sparse else None, num_splits,
                                     _ptr(part_o), _ptr(part_lse), _stream(stream)))


def attn_decode_merge(part_o, part_lse, num_splits, out, lse=None, stream=None, splits_per_batch=None):
    """part_o [B,Q,Hq,S,Dv] fp32, part_lse [B,Q,Hq,S] -> out [B,Q,Hq,Dv] (any strides), lse [B,Q,Hq];
    splits_per_batch: optional int32 device tensor [B], the leading splits of each sequence to merge."""
    B, Q, Hq, _, Dv = part_o.shape
    _check("attn_decode_merge",
           lib().attn_decode_merge(_ptr(part_o), _ptr(part_lse), _ptr(splits_per_batch), num_splits, B, Q, Hq, Dv,
                                   _DTYPE[out.dtype], _ptr(out), I64x3(*out.stride()[:3]), _ptr(lse),
                                   _stream(stream)))


def attn_decode(args: DecodeArgs, paged: Paged | None, sparse: Sparse | None, num_splits: int, workspace,
                stream=None):
    """One-launch decode step; `workspace` (uint8 device tensor) must be zero-filled before its first use."""
    _check("attn_decode",
           lib().attn_decode(ctypes.byref(args), ctypes.byref(paged) if paged else None,
                             ctypes.byref(sparse) if sparse else None, num_splits, _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_decode_noalloc(args: DecodeArgs, paged: Paged | None, sparse: Sparse | None, num_splits: int,
                        stream=None):
    """attn_decode in the library's own workspace (no workspace argument, nothing allocated)."""
    _check("attn_decode_noalloc",
           lib().attn_decode_noalloc(ctypes.byref(args), ctypes.byref(paged) if paged else None,
                                     ctypes.byref(sparse) if sparse else None, num_splits, _stream(stream)))


def attn_decode_launches(args: DecodeArgs, paged: Paged | None = None, sparse: Sparse | None = None,
                         num_splits: int = 0) -> int:
    n = ctypes.c_int32()
    _check("attn_decode_launches",
           lib().attn_decode_launches(ctypes.byref(args), ctypes.byref(paged) if paged else None,
                                      ctypes.byref(sparse) if sparse else None, num_splits, ctypes.byref(n)))
    return n.value


KERNEL_NAMES = {0: "partial_valu_kernel", 1: "partial_mfma_kernel", 2: "mla_partial_kernel",
                3: "partial_mfma16_kernel"}


def attn_decode_kernel(args: DecodeArgs) -> int:
    """AD_KERNEL_VECTOR / AD_KERNEL_MATRIX16 / AD_KERNEL_MATRIX / AD_KERNEL_MLA: the partial-pass kernel the calls run
    (KERNEL_NAMES maps it to the kernel's name in a profile)."""
    k = ctypes.c_int32()
    _check("attn_decode_kernel", lib().attn_decode_kernel(ctypes.byref(args), ctypes.byref(k)))
    return k.value


def attn_decode_paged(args: DecodeArgs, paged: Paged, num_splits: int, workspace, stream=None):
    _check("attn_decode_paged",
           lib().attn_decode_paged(ctypes.byref(args), ctypes.byref(paged), num_splits, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_decode_mla_splitkv(args: DecodeArgs, kpe, q_pe, paged: Paged, num_splits: int, part_o, part_lse,
                            stream=None):
    _check("attn_decode_mla_splitkv",
           lib().attn_decode_mla_splitkv(ctypes.byref(args), _ptr(kpe), _s3(kpe), _ptr(q_pe), _s3(q_pe),
                                         ctypes.byref(paged), num_splits, _ptr(part_o), _ptr(part_lse),
                                         _stream(stream)))


def attn_decode_mla(args: DecodeArgs, kpe, q_pe, paged: Paged, num_splits: int, workspace, stream=None):
    _check("attn_decode_mla",
           lib().attn_decode_mla(ctypes.byref(args), _ptr(kpe), _s3(kpe), _ptr(q_pe), _s3(q_pe),
                                 ctypes.byref(paged), num_splits, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_decode_read_probe(src, sink, stream=None):
    """Stream all of `src` (a 16-byte aligned device tensor) through the library's read probe;
    sink: int32/uint32 device tensor of AD_PROBE_SINK_WORDS words."""
    nbytes = src.numel() * src.element_size()
    if sink.numel() < AD_PROBE_SINK_WORDS:
        raise ValueError("sink too small")
    _check("attn_decode_read_probe", lib().attn_decode_read_probe(_ptr(src), nbytes, _ptr(sink), _stream(stream)))
