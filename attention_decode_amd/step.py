"""One decode step of a workload, prepared once and replayed.

DecodeStep fills the C descriptors for a device-resident Workload, allocates its outputs and
workspace, and each call enqueues the whole step on the current stream:
  contiguous / block-sparse / paged cache: attn_decode (one launch: the partial pass, whose last
      split per work unit merges); with fused=False, attn_decode_splitkv + attn_decode_merge and
      the partials are kept in part_o / part_lse
  MLA: attn_decode_mla (partial pass + merge)
With packed variable-length queries (w.q_starts) out / lse are packed [tokens, Hq, ...] too; the
separate public merge takes whole [B, q_len] rows, so that form needs fused=True (attn_decode
still picks one or two launches itself).
"""
from __future__ import annotations

import torch

from . import _abi
from .inputs import Workload


class DecodeStep:
    def __init__(self, w: Workload, num_splits: int | None = None, out=None, lse=None, fused: bool = True):
        if w.q.device.type != "cuda":
            raise ValueError("DecodeStep needs the workload on the GPU")
        self.w = w
        dev = w.q.device
        B, Q, Hq, Dv = w.batch, w.q_len, w.num_q_heads, w.head_dim_v
        rows = (w.q.shape[0],) if w.q_starts is not None else (B, Q)
        if w.q_starts is not None and not fused:
            raise ValueError("packed variable-length queries need fused=True")
        self.out = torch.empty(*rows, Hq, Dv, dtype=w.dtype, device=dev) if out is None else out
        self.lse = torch.empty(*rows, Hq, dtype=torch.float32, device=dev) if lse is None else lse
        forced = num_splits if num_splits is not None else (w.num_splits or 0)
        common = dict(scale=w.scale, seq_lens=w.seq_lens if w.lens_given else None, kv_len_max=w.kv_len_max,
                      causal=w.causal,
                      window=w.window, out=self.out, lse=self.lse, q_starts=w.q_starts,
                      q_len=w.q_len if w.q_starts is not None else None, tree_mask=w.tree_mask)
        self.sparse = self.paged = None
        self.fused = fused and w.kind != "mla"
        if w.kind == "mla":
            self.args = _abi.make_args(w.q, w.k, None, head_dim_qk=w.head_dim_qk, **common)
        else:
            self.args = _abi.make_args(w.q, w.k, w.v, k_scale=w.k_scale, v_scale=w.v_scale, **common)
        if w.kind in ("paged", "mla"):
            self.paged = _abi.make_paged(w.block_table, w.page_size)
        if w.num_blocks is not None:
            self.sparse = _abi.make_sparse(w.num_blocks, w.block_idx, w.block_size)
        self.splits = forced or _abi.attn_decode_plan(self.args, self.paged, self.sparse)[0]
        if self.fused or w.kind == "mla":
            # zero-filled once: the single-launch merge counts arrivals in it and leaves it zeroed
            nbytes = _abi.attn_decode_workspace_size(self.args, self.paged, self.splits, self.sparse)
            self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        else:
            self.part_o = torch.empty(B, Q, Hq, self.splits, Dv, dtype=torch.float32, device=dev)
            self.part_lse = torch.empty(B, Q, Hq, self.splits, dtype=torch.float32, device=dev)

    def __call__(self, stream=None):
        w = self.w
        if w.kind == "mla":
            _abi.attn_decode_mla(self.args, w.kpe, w.q_pe, self.paged, self.splits, self.workspace, stream)
        elif self.fused:
            _abi.attn_decode(self.args, self.paged, self.sparse, self.splits, self.workspace, stream)
        else:
            _abi.attn_decode_splitkv(self.args, self.paged, self.sparse, self.splits, self.part_o, self.part_lse,
                                     stream)
            _abi.attn_decode_merge(self.part_o, self.part_lse, self.splits, self.out, self.lse, stream)
        return self.out, self.lse
