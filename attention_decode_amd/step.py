"""One decode step of a workload, prepared once and replayed.

DecodeStep fills the C descriptors for a device-resident Workload, allocates its outputs, partial
buffers and workspace, and each call enqueues the whole step on the current stream:
  contiguous / block-sparse cache: attn_decode_splitkv + attn_decode_merge
  paged cache:                     attn_decode_paged (partial pass + merge inside)
  MLA:                             attn_decode_mla (partial pass + merge inside)
"""
from __future__ import annotations

import torch

from . import _abi
from .inputs import Workload


class DecodeStep:
    def __init__(self, w: Workload, num_splits: int | None = None, out=None, lse=None):
        if w.q.device.type != "cuda":
            raise ValueError("DecodeStep needs the workload on the GPU")
        self.w = w
        dev = w.q.device
        B, Q, Hq, Dv = w.batch, w.q_len, w.num_q_heads, w.head_dim_v
        self.out = torch.empty(B, Q, Hq, Dv, dtype=w.dtype, device=dev) if out is None else out
        self.lse = torch.empty(B, Q, Hq, dtype=torch.float32, device=dev) if lse is None else lse
        forced = num_splits if num_splits is not None else (w.num_splits or 0)
        common = dict(scale=w.scale, seq_lens=w.seq_lens, kv_len_max=w.kv_len_max, causal=w.causal,
                      window=w.window, out=self.out, lse=self.lse)
        self.sparse = self.paged = None
        if w.kind == "contiguous":
            self.args = _abi.make_args(w.q, w.k, w.v, **common)
            if w.num_blocks is not None:
                self.sparse = _abi.make_sparse(w.num_blocks, w.block_idx, w.block_size)
            self.splits = forced or _abi.attn_decode_plan(self.args, None, self.sparse)[0]
            self.part_o = torch.empty(B, Q, Hq, self.splits, Dv, dtype=torch.float32, device=dev)
            self.part_lse = torch.empty(B, Q, Hq, self.splits, dtype=torch.float32, device=dev)
        else:
            if w.kind == "mla":
                self.args = _abi.make_args(w.q, w.k, None, head_dim_qk=w.head_dim_qk, **common)
            else:
                self.args = _abi.make_args(w.q, w.k, w.v, **common)
            self.paged = _abi.make_paged(w.block_table, w.page_size)
            self.splits = forced or _abi.attn_decode_plan(self.args, self.paged, None)[0]
            nbytes = _abi.attn_decode_workspace_size(self.args, self.paged, self.splits)
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def __call__(self, stream=None):
        w = self.w
        if w.kind == "contiguous":
            _abi.attn_decode_splitkv(self.args, None, self.sparse, self.splits, self.part_o, self.part_lse, stream)
            _abi.attn_decode_merge(self.part_o, self.part_lse, self.splits, self.out, self.lse, stream)
        elif w.kind == "paged":
            _abi.attn_decode_paged(self.args, self.paged, self.splits, self.workspace, stream)
        else:
            _abi.attn_decode_mla(self.args, w.kpe, w.q_pe, self.paged, self.splits, self.workspace, stream)
        return self.out, self.lse
