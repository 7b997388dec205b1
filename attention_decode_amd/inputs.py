"""Seeded synthetic decode-attention workloads.

This module draws inputs only: shapes, random values, page permutations, block lists. It holds
none of the attention arithmetic, and both the HIP path and the CPU reference read the tensors it
returns. Every draw comes from ``torch.Generator('cpu')`` seeded with ``1000 + config`` (or the
given seed) in a fixed order, so the same workload is produced on any machine. An fp8 cache is
quantised here, as input preparation (the library and the CPU reference only dequantise it).

The workloads (sizes of the decode benchmarks this library is measured on; 6 is the fp8 form of 3):

1. tiny MHA: B=1, 8 q heads = 8 KV heads, D=64, 1 query, KV len 512 contiguous, fp32,
   scale 1/8, forced 4 KV splits then merge.
2. GQA contiguous: B=16, 32 q / 8 KV heads, D=128, 1 query, KV len 4096, bf16, scale 1/sqrt(128).
3. paged GQA ragged: B=64, 32 q / 8 KV heads, D=128, bf16, page 16, seq lens uniform in
   [128, 8192], block table = random permutation of a shared page pool.
4. block-sparse + speculative: B=8, 64 q / 8 KV heads, D=128, 4 query tokens at the tail of KV
   len 32768, bf16, KV blocks of 128 listed per (b, KV head), causal + sliding window 4096.
5. MLA: B=32, 128 q heads on one latent KV head, q/k dim 576 (512 latent + 64 rope), v dim 512
   (the latent), KV len 8192, bf16, paged with page 64, scale 1/sqrt(192).
6. workload 3 with its cache quantised to OCP E4M3 (fp8) bytes with one fp32 scale per (token, KV
   head) row for K and for V (the same lengths and values before quantisation).
7. speculative decoding over workload 3's shape: B=64 paged sequences (lengths uniform in
   [128, 8192], page 16, 32 q / 8 KV heads, D=128, bf16), each with 1 to 8 draft tokens (uniform)
   as packed variable-length queries, and a random token tree per sequence as the tree mask
   (token t sees itself and its ancestors among the drafts).
8. workload 3 with its cache quantised to int4: every K and V row one group of 128 4-bit fields
   with an fp16 scale and shift (mslk's row-wise int4 layout), from the same values.

Cache layouts: a contiguous cache is stored head-major ``[B, Hkv, L, D]``; a paged pool is stored
``[pages, Hkv, page_size, D]``. Both are handed out as token-major *views* ``[B, L, Hkv, D]`` /
``[pages, page_size, Hkv, D]`` whose strides say where the data really is. ``token_major(w)``
re-stores the same cache token-major (``[B, L, Hkv, D]`` / ``[pages, page_size, Hkv, D]`` in
memory, every key's heads side by side), with the same values.
"""
from __future__ import annotations

import copy
import math
from dataclasses import dataclass, field

import torch

NUM_CONFIGS = 8


@dataclass
class Workload:
    config: int
    name: str
    kind: str                      # "contiguous" | "paged" | "mla"
    dtype: torch.dtype
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    scale: float
    kv_len_max: int
    seq_lens: torch.Tensor         # int32 [B]
    q: torch.Tensor                # [B, Q, Hq, Dqk]  (MLA: the 512 latent dims, q_nope)
    k: torch.Tensor                # token-major view (MLA: ckv pool view [pages, page, 1, 512])
    v: torch.Tensor                # token-major view (MLA: the same ckv view)
    causal: bool = False
    window: int = 0
    num_splits: int | None = None  # forced split count (config 1), else None
    # paged
    block_table: torch.Tensor | None = None
    page_size: int = 0
    # block-sparse
    num_blocks: torch.Tensor | None = None
    block_idx: torch.Tensor | None = None
    block_size: int = 0
    # MLA second score part
    q_pe: torch.Tensor | None = None   # [B, Q, Hq, 64]
    kpe: torch.Tensor | None = None    # [pages, page, 1, 64]
    # quantised cache: "fp8" = k / v hold OCP E4M3 bytes, with fp32 row scales (views indexed like
    # the cache rows: [B, L, Hkv] contiguous, [pages, page, Hkv] paged; zero strides for one scale
    # per tensor)
    kv_format: str = "same"   # "same" | "fp8" | "int4"
    kv_groups: int = 0        # int4: coefficient groups per row
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None
    # speculative decoding: packed variable-length queries (q is then [tokens, Hq, D] and q_len
    # the largest count) and a tree mask over each sequence's last Q_b keys (int32 words,
    # [token rows, ceil(q_len / 32)])
    q_starts: torch.Tensor | None = None
    tree_mask: torch.Tensor | None = None
    # "head": the cache (and its row scales) stored head-major; "token": stored token-major
    layout: str = "head"
    # False: the library is told nothing about per-sequence lengths (seq_lens = NULL, every
    # sequence has kv_len_max keys); seq_lens still holds those lengths for the reference
    lens_given: bool = True
    storage: dict = field(default_factory=dict)

    def to(self, device) -> "Workload":
        """Copy every tensor to `device`, keeping the storage layout the views point into."""
        out = copy.copy(self)
        out.storage = {name: t.to(device) for name, t in self.storage.items()}
        for f in ("seq_lens", "block_table", "num_blocks", "block_idx", "q_starts", "tree_mask"):
            t = getattr(self, f)
            if t is not None:
                setattr(out, f, t.to(device))
        return _finish(out)

    def kv_bytes_by_group(self) -> list:
        """Bytes of K and V (MLA: ckv + kpe once) that a decode step must read, per (sequence, KV
        head) as [B][Hkv] (MLA: one latent head): each key once if it is inside the sequence,
        inside a listed block (block-sparse cache), and visible to at least one query row under
        the causal / sliding-window bounds."""
        lens = [int(x) for x in self.seq_lens.to("cpu")]
        counts = self.q_counts()
        per_tok = self.bytes_per_key()
        heads = 1 if self.kind == "mla" else self.num_kv_heads
        out = []
        for b, L in enumerate(lens):
            Qb = counts[b]
            hi = L if Qb else 0                                               # newest query sits at L - 1
            lo = max(0, L - Qb - self.window + 1) if self.window else 0      # oldest key of the first query
            row = []
            for h in range(heads):
                if self.num_blocks is None:
                    n = max(0, hi - lo)
                else:
                    n = 0
                    for blk in self.block_idx[b, h, :int(self.num_blocks[b, h])].tolist():
                        n += max(0, min((blk + 1) * self.block_size, hi) - max(blk * self.block_size, lo))
                row.append(n * per_tok)
            out.append(row)
        return out

    def kv_bytes_listed(self) -> int:
        """Bytes of every listed block of a block-sparse cache inside its sequence (each key once per
        KV head), whether or not a query row sees it; kv_bytes() for other caches."""
        if self.num_blocks is None:
            return self.kv_bytes()
        per_tok = self.bytes_per_key()
        n = 0
        for b, L in enumerate(int(x) for x in self.seq_lens.to("cpu")):
            for h in range(self.num_kv_heads):
                for blk in self.block_idx[b, h, :int(self.num_blocks[b, h])].tolist():
                    n += max(0, min((blk + 1) * self.block_size, L) - blk * self.block_size)
        return n * per_tok

    def q_counts(self) -> list:
        """Query tokens of each sequence: q_len, or the differences of q_starts."""
        if self.q_starts is None:
            return [self.q_len] * self.batch
        qs = [int(x) for x in self.q_starts.to("cpu")]
        return [qs[b + 1] - qs[b] for b in range(self.batch)]

    def bytes_per_key(self) -> int:
        """Bytes one key costs per KV head: its K and V rows (MLA: ckv + kpe once), plus its two
        fp32 row scales when an fp8 cache has one scale per row."""
        if self.kv_format == "int4":  # K and V rows of kv_groups + D / 8 words
            return 4 * (2 * self.kv_groups + (self.head_dim_qk + self.head_dim_v) // 8)
        es = 1 if self.kv_format == "fp8" else torch.finfo(self.dtype).bits // 8
        if self.kind == "mla":
            return self.head_dim_qk * es
        per = (self.head_dim_qk + self.head_dim_v) * es
        if self.kv_format == "fp8" and self.k_scale is not None and self.k_scale.stride() != (0, 0, 0):
            per += 8
        return per

    def kv_bytes(self) -> int:
        """Total of kv_bytes_by_group: the algorithmic KV bytes of one decode step."""
        return sum(sum(r) for r in self.kv_bytes_by_group())

    def flops(self) -> int:
        """Multiply-adds x 2 of one step over the visible keys: q.k (head_dim_qk) and p.v (head_dim_v)
        for every query row of each KV head."""
        per_key = self.bytes_per_key()
        heads_per_kv = self.num_q_heads if self.kind == "mla" else self.num_q_heads // self.num_kv_heads
        counts = self.q_counts()
        keys_rows = sum(sum(x) // per_key * counts[b] * heads_per_kv for b, x in enumerate(self.kv_bytes_by_group()))
        return keys_rows * (self.head_dim_qk + self.head_dim_v) * 2


# token-major view of each storage tensor: (storage name, permutation) per field
_VIEWS = {
    "contiguous": {"q": ("q", None), "k": ("k", (0, 2, 1, 3)), "v": ("v", (0, 2, 1, 3))},
    "paged": {"q": ("q", None), "k": ("k", (0, 2, 1, 3)), "v": ("v", (0, 2, 1, 3))},
    "mla": {"q": ("q", None), "q_pe": ("q_pe", None), "k": ("ckv", None), "v": ("ckv", None),
            "kpe": ("kpe", None)},
}


def _randn(g, shape, dtype):
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def _finish(w: Workload) -> Workload:
    token = w.layout == "token"
    for f, (src, perm) in _VIEWS[w.kind].items():
        cache = f in ("k", "v") and w.kind != "mla"
        setattr(w, f, w.storage[src].permute(*perm) if perm and not (cache and token) else w.storage[src])
    for f in ("k_scale", "v_scale"):  # row scales of an fp8 cache, stored like the cache
        t = w.storage.get(f)
        if t is not None:
            rows = tuple(w.k.shape[:3])
            setattr(w, f, t.reshape(1, 1, 1).expand(*rows) if t.numel() == 1 else t if token else t.permute(0, 2, 1))
    return w


def token_major(w: Workload) -> Workload:
    """The same workload with its contiguous or paged cache (and fp8 row scales) stored token-major:
    [B, L, Hkv, D] / [pages, page_size, Hkv, D] in memory instead of head-major. Values, lengths,
    page tables and block lists are unchanged, so the logical cache is the same bit for bit."""
    if w.kind == "mla" or w.layout == "token":
        raise ValueError("token_major takes a head-major contiguous or paged workload")
    out = copy.copy(w)
    out.storage = dict(w.storage)
    for name in ("k", "v"):
        out.storage[name] = w.storage[name].permute(0, 2, 1, 3).contiguous()
    for name in ("k_scale", "v_scale"):
        t = w.storage.get(name)
        if t is not None and t.numel() > 1:
            out.storage[name] = t.permute(0, 2, 1).contiguous()
    out.layout = "token"
    return _finish(out)


E4M3_MAX = 448.0  # largest finite OCP E4M3 magnitude


def quantize_e4m3(x: torch.Tensor, per: str):
    """Input preparation for an fp8 cache: OCP E4M3 bytes of x / scale (round to nearest even,
    PyTorch's float8_e4m3fn cast) and the fp32 scales, one per row of the last dimension
    (per="token": amax of the row / 448) or one for the tensor (per="tensor")."""
    x = x.float()
    if per == "token":
        amax = x.abs().amax(dim=-1)
        scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        q = x / scale[..., None]
    elif per == "tensor":
        amax = x.abs().max()
        scale = (amax / E4M3_MAX if amax > 0 else torch.ones(())).reshape(1)
        q = x / scale
    else:
        raise ValueError(per)
    return q.to(torch.float8_e4m3fn).view(torch.uint8), scale.float().contiguous()


INT4_POISON = 0x7E007E00  # a word whose halves are both fp16 NaN (a coefficient word of NaN)


def quantize_int4(x: torch.Tensor, groups: int) -> torch.Tensor:
    """Input preparation for an int4 cache: every row of the last dimension D is split into
    `groups` groups; per group the shift is the minimum and the scale (max - min) / 15, both
    rounded to fp16, and each value becomes the nearest field in 0..15 of
    (x - shift) / scale. Returns int32 words [..., groups + D / 8]: the coefficient words (fp16
    scale in the low half, shift in the high half), then the fields, field d % 8 of word d / 8."""
    x = x.float()
    D = x.shape[-1]
    xg = x.reshape(*x.shape[:-1], groups, D // groups)
    lo, hi = xg.amin(dim=-1), xg.amax(dim=-1)
    shift = lo.to(torch.float16)
    scale = ((hi - lo) / 15.0).to(torch.float16)
    safe = torch.where(scale.float() > 0, scale.float(), torch.ones_like(scale.float()))
    f = torch.round((xg - shift.float()[..., None]) / safe[..., None]).clamp(0, 15).to(torch.int64)
    f = torch.where((scale.float() > 0)[..., None], f, torch.zeros_like(f)).reshape(*x.shape[:-1], D // 8, 8)
    packed = torch.zeros(f.shape[:-1], dtype=torch.int64)
    for j in range(8):
        packed |= f[..., j] << (4 * j)
    coef = (scale.view(torch.int16).to(torch.int64) & 0xFFFF) | ((shift.view(torch.int16).to(torch.int64) & 0xFFFF) << 16)
    words = torch.cat([coef, packed], dim=-1)
    return torch.where(words >= 2 ** 31, words - 2 ** 32, words).to(torch.int32)


def contiguous(*, config=0, name="custom", batch, num_q_heads, num_kv_heads, head_dim, kv_len,
               q_len=1, dtype=torch.bfloat16, scale=None, seq_lens=None, seed=0,
               causal=False, window=0, num_splits=None, kv_format="same", kv_scales="token",
               kv_groups=1) -> Workload:
    """Head-major contiguous cache [B, Hkv, L, D]; `seq_lens` (list) may be ragged (<= kv_len).
    kv_format="fp8": K and V are quantised to E4M3 with row (kv_scales="token") or tensor scales;
    kv_format="int4": to 4-bit fields with kv_groups fp16 scale / shift pairs per row."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (batch, q_len, num_q_heads, head_dim), dtype)
    k = _randn(g, (batch, num_kv_heads, kv_len, head_dim), dtype)
    v = _randn(g, (batch, num_kv_heads, kv_len, head_dim), dtype)
    sl = torch.full((batch,), kv_len, dtype=torch.int32) if seq_lens is None else \
        torch.as_tensor(seq_lens, dtype=torch.int32)
    w = Workload(config=config, name=name, kind="contiguous", dtype=dtype, batch=batch, q_len=q_len,
                 num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim_qk=head_dim,
                 head_dim_v=head_dim, scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                 kv_len_max=kv_len, seq_lens=sl, q=None, k=None, v=None, causal=causal, window=window,
                 num_splits=num_splits, kv_format=kv_format)
    w.storage = {"q": q, "k": k, "v": v}
    if kv_format == "int4":
        w.kv_groups = kv_groups
        w.storage["k"], w.storage["v"] = quantize_int4(k, kv_groups), quantize_int4(v, kv_groups)
    if kv_format == "fp8":
        w.storage["k"], w.storage["k_scale"] = quantize_e4m3(k, kv_scales)
        w.storage["v"], w.storage["v_scale"] = quantize_e4m3(v, kv_scales)
    return _finish(w)


def paged(*, config=0, name="custom", seq_lens, num_q_heads, num_kv_heads, head_dim, page_size,
          q_len=1, dtype=torch.bfloat16, scale=None, seed=0, poison=False, max_pages=None,
          causal=False, window=0, shuffle_pages=True, kv_format="same", kv_scales="token",
          kv_groups=1) -> Workload:
    """Paged cache: pool [pages, Hkv, page_size, D] (head-major pages), block table [B, max_pages].

    The logical content of sequence b depends only on the seed and seq_lens; the physical page
    order is a random permutation. With ``poison`` the pool gets ~5% extra pages nobody
    references, every page and tail slot not covered by a sequence holds NaN, the table is padded
    with -1, and a different permutation is used -- the logical KV is unchanged. kv_format="fp8":
    the same logical K and V quantised to E4M3 (row or tensor scales; poisoned slots hold the E4M3
    NaN code and NaN scales).
    """
    g = torch.Generator().manual_seed(seed)
    sl = torch.as_tensor(seq_lens, dtype=torch.int32)
    B = sl.numel()
    pages_b = [(int(x) + page_size - 1) // page_size for x in sl]
    n_logical = sum(pages_b)
    q = _randn(g, (B, q_len, num_q_heads, head_dim), dtype)
    k_log = _randn(g, (n_logical, num_kv_heads, page_size, head_dim), dtype)
    v_log = _randn(g, (n_logical, num_kv_heads, page_size, head_dim), dtype)
    n_pool = n_logical + (max(1, n_logical // 20) if poison else 0)
    pg = torch.Generator().manual_seed(seed + (7919 if poison else 0))
    perm = torch.randperm(n_pool, generator=pg)[:n_logical] if shuffle_pages else torch.arange(n_logical)
    fill = float("nan") if poison else 0.0
    k_pool = torch.full((n_pool, num_kv_heads, page_size, head_dim), fill, dtype=dtype)
    v_pool = torch.full((n_pool, num_kv_heads, page_size, head_dim), fill, dtype=dtype)
    k_pool[perm] = k_log
    v_pool[perm] = v_log
    mp = max(pages_b) if max_pages is None else max_pages
    bt = torch.full((B, max(mp, 1)), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(pages_b):
        bt[b, :n] = perm[off:off + n].to(torch.int32)
        # slots past the end of the sequence in its last page
        tail = int(sl[b]) - (n - 1) * page_size if n else page_size
        if poison and n and tail < page_size:
            k_pool[bt[b, n - 1], :, tail:] = float("nan")
            v_pool[bt[b, n - 1], :, tail:] = float("nan")
        off += n
    w = Workload(config=config, name=name, kind="paged", dtype=dtype, batch=B, q_len=q_len,
                 num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim_qk=head_dim,
                 head_dim_v=head_dim, scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                 kv_len_max=mp * page_size, seq_lens=sl, q=None, k=None, v=None,
                 block_table=bt, page_size=page_size, causal=causal, window=window, kv_format=kv_format)
    w.storage = {"q": q, "k": k_pool, "v": v_pool}
    if kv_format == "int4":
        w.kv_groups = kv_groups
        for name_, pool in (("k", k_pool), ("v", v_pool)):
            live = ~torch.isnan(pool).any(dim=-1)                    # rows that hold a key
            words = quantize_int4(torch.nan_to_num(pool), kv_groups)
            words[~live] = INT4_POISON                                  # NaN coefficients where nothing belongs
            w.storage[name_] = words
    if kv_format == "fp8":
        for name_, pool in (("k", k_pool), ("v", v_pool)):
            live = ~torch.isnan(pool).any(dim=-1)                    # rows that hold a key
            qbytes, sc = quantize_e4m3(torch.nan_to_num(pool), kv_scales)
            qbytes[~live] = 0x7F                                       # E4M3 NaN where nothing belongs
            if kv_scales == "token":
                sc = torch.where(live, sc, torch.full_like(sc, float("nan")))
            w.storage[name_], w.storage[name_ + "_scale"] = qbytes, sc
    return _finish(w)


def window_block_list(kv_len: int, q_len: int, window: int, block_size: int):
    """Blocks that hold at least one key inside the causal sliding window of some query row of a
    q_len-token query at the tail of a kv_len cache (the 'causal + window expressed as block
    lists' input of the block-sparse workload). Returned ascending."""
    first_key = max(0, kv_len - q_len - window + 1)   # oldest key the first query can see
    last_key = kv_len - 1                               # newest key the last query can see
    return list(range(first_key // block_size, last_key // block_size + 1))


def sparse(*, config=0, name="custom", batch, num_q_heads, num_kv_heads, head_dim, kv_len, q_len,
           block_size, blocks, dtype=torch.bfloat16, scale=None, seed=0, causal=True, window=0,
           poison=False, seq_lens=None, kv_format="same", kv_scales="token", kv_groups=1) -> Workload:
    """Contiguous head-major cache with a per-(b, KV head) list of KV blocks: ``blocks`` is one list
    shared by every (b, KV head), or a nested list blocks[b][h] of lists of any lengths (the index
    array is padded with -1, which is never read). With ``poison`` every key outside the listed
    blocks of its own (b, h), and every key at or past seq_lens[b], holds NaN."""
    w = contiguous(config=config, name=name, batch=batch, num_q_heads=num_q_heads,
                   num_kv_heads=num_kv_heads, head_dim=head_dim, kv_len=kv_len, q_len=q_len,
                   dtype=dtype, scale=scale, seed=seed, causal=causal, window=window, seq_lens=seq_lens,
                   kv_format=kv_format, kv_scales=kv_scales, kv_groups=kv_groups)
    if blocks and isinstance(blocks[0], (list, tuple)):
        lists = [[list(blocks[b][h]) for h in range(num_kv_heads)] for b in range(batch)]
    else:
        lists = [[list(blocks) for _ in range(num_kv_heads)] for _ in range(batch)]
    nmax = max(1, max(len(x) for row in lists for x in row))
    w.num_blocks = torch.tensor([[len(x) for x in row] for row in lists], dtype=torch.int32)
    w.block_idx = torch.full((batch, num_kv_heads, nmax), -1, dtype=torch.int32)
    for b in range(batch):
        for h in range(num_kv_heads):
            if lists[b][h]:
                w.block_idx[b, h, :len(lists[b][h])] = torch.as_tensor(lists[b][h], dtype=torch.int32)
    w.block_size = block_size
    if poison:
        for b in range(batch):
            for h in range(num_kv_heads):
                keep = torch.zeros(kv_len, dtype=torch.bool)
                for blk in lists[b][h]:
                    keep[blk * block_size:(blk + 1) * block_size] = True
                keep[int(w.seq_lens[b]):] = False
                for name_ in ("k", "v"):
                    if w.kv_format == "int4":  # NaN coefficients
                        w.storage[name_][b, h, ~keep, :] = INT4_POISON
                    elif w.kv_format == "fp8":  # the E4M3 NaN code, and NaN row scales
                        w.storage[name_][b, h, ~keep, :] = 0x7F
                        if w.storage[name_ + "_scale"].numel() > 1:
                            w.storage[name_ + "_scale"][b, h, ~keep] = float("nan")
                    else:
                        w.storage[name_][b, h, ~keep, :] = float("nan")
    return w


def mla(*, config=0, name="custom", batch, num_heads, kv_len, page_size, dim_latent=512, dim_rope=64,
        dtype=torch.bfloat16, scale=None, seed=0, seq_lens=None, poison=False, q_len=1, causal=False,
        window=0) -> Workload:
    """MLA: q_nope [B,Q,H,512], q_pe [B,Q,H,64], ckv pool [pages, page, 512] and kpe pool
    [pages, page, 64] (one shared latent KV head), block table from a random page permutation."""
    g = torch.Generator().manual_seed(seed)
    sl = torch.full((batch,), kv_len, dtype=torch.int32) if seq_lens is None else \
        torch.as_tensor(seq_lens, dtype=torch.int32)
    pages_b = [(int(x) + page_size - 1) // page_size for x in sl]
    n_logical = sum(pages_b)
    q = _randn(g, (batch, q_len, num_heads, dim_latent), dtype)
    q_pe = _randn(g, (batch, q_len, num_heads, dim_rope), dtype)
    ckv_log = _randn(g, (n_logical, page_size, dim_latent), dtype)
    kpe_log = _randn(g, (n_logical, page_size, dim_rope), dtype)
    n_pool = n_logical + (max(1, n_logical // 20) if poison else 0)
    pg = torch.Generator().manual_seed(seed + (7919 if poison else 0))
    perm = torch.randperm(n_pool, generator=pg)[:n_logical]
    fill = float("nan") if poison else 0.0
    ckv = torch.full((n_pool, page_size, dim_latent), fill, dtype=dtype)
    kpe = torch.full((n_pool, page_size, dim_rope), fill, dtype=dtype)
    ckv[perm] = ckv_log
    kpe[perm] = kpe_log
    mp = max(pages_b)
    bt = torch.full((batch, mp), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(pages_b):
        bt[b, :n] = perm[off:off + n].to(torch.int32)
        tail = int(sl[b]) - (n - 1) * page_size
        if poison and tail < page_size:
            ckv[bt[b, n - 1], tail:] = float("nan")
            kpe[bt[b, n - 1], tail:] = float("nan")
        off += n
    w = Workload(config=config, name=name, kind="mla", dtype=dtype, batch=batch, q_len=q_len,
                 num_q_heads=num_heads, num_kv_heads=1, head_dim_qk=dim_latent + dim_rope,
                 head_dim_v=dim_latent, scale=(1.0 / math.sqrt(192)) if scale is None else scale,
                 kv_len_max=mp * page_size, seq_lens=sl, q=None, k=None, v=None,
                 block_table=bt, page_size=page_size, causal=causal, window=window)
    w.storage = {"q": q, "q_pe": q_pe, "ckv": ckv.view(n_pool, page_size, 1, dim_latent),
                 "kpe": kpe.view(n_pool, page_size, 1, dim_rope)}
    return _finish(w)


def random_tree_masks(g, counts, q_len):
    """Tree masks of random draft-token trees, one tree per sequence with counts[b] tokens: the
    parent of token i >= 1 is uniform in [0, i) and token 0 is the root; token t sees itself and
    its ancestors. Returns int32 [sum(counts), ceil(q_len / 32)] words, bit i of a row = draft i."""
    words = (q_len + 31) // 32
    rows = []
    for n in counts:
        parent = [-1] + [int(torch.randint(0, i, (1,), generator=g)) for i in range(1, n)]
        for t in range(n):
            bits, i = 0, t
            while i >= 0:
                bits |= 1 << i
                i = parent[i]
            rows.append([(bits >> (32 * w)) & 0xFFFFFFFF for w in range(words)])
    m = torch.tensor(rows, dtype=torch.int64).reshape(len(rows), words)
    return torch.where(m >= 2 ** 31, m - 2 ** 32, m).to(torch.int32)


def with_spec(w: Workload, counts=None, tree: bool = False, seed: int = 0) -> Workload:
    """Speculative-decoding form of a workload whose q is [B, q_len, Hq, D]: with `counts`, the
    first counts[b] query tokens of each sequence become packed variable-length queries
    (q [tokens, Hq, D], q_starts [B + 1]); with `tree`, a random token tree per sequence becomes
    the tree mask (drawn from torch.Generator seeded with `seed`)."""
    if w.kind == "mla":
        raise ValueError("MLA takes no variable query lengths or tree masks")
    out = copy.copy(w)
    out.storage = dict(w.storage)
    if counts is not None:
        counts = [int(c) for c in counts]
        if len(counts) != w.batch or min(counts) < 0 or max(counts) > w.q_len:
            raise ValueError("counts must give 0..q_len tokens per sequence")
        q = w.storage["q"]
        out.storage["q"] = torch.cat([q[b, :counts[b]] for b in range(w.batch)]).contiguous()
        starts = [0]
        for c in counts:
            starts.append(starts[-1] + c)
        out.q_starts = torch.tensor(starts, dtype=torch.int32)
    if tree:
        g = torch.Generator().manual_seed(seed)
        out.tree_mask = random_tree_masks(g, out.q_counts(), w.q_len)
    return _finish(out)


def make(config: int, *, seed: int | None = None, poison: bool = False) -> Workload:
    """One of the five benchmark workloads, generated on the CPU."""
    s = 1000 + config if seed is None else seed
    if config == 1:
        return contiguous(config=1, name="tiny_mha_fp32_split4", batch=1, num_q_heads=8, num_kv_heads=8,
                          head_dim=64, kv_len=512, dtype=torch.float32, scale=1.0 / 8.0, seed=s,
                          num_splits=4)
    if config == 2:
        return contiguous(config=2, name="gqa_bf16_contiguous", batch=16, num_q_heads=32, num_kv_heads=8,
                          head_dim=128, kv_len=4096, dtype=torch.bfloat16, seed=s)
    if config == 3:
        g = torch.Generator().manual_seed(s)
        lens = torch.randint(128, 8193, (64,), generator=g, dtype=torch.int64).tolist()
        return paged(config=3, name="paged_gqa_bf16_ragged", seq_lens=lens, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, page_size=16, dtype=torch.bfloat16, seed=s + 1, poison=poison,
                     max_pages=512)
    if config == 4:
        blocks = window_block_list(32768, 4, 4096, 128)
        return sparse(config=4, name="sparse_spec_bf16", batch=8, num_q_heads=64, num_kv_heads=8,
                      head_dim=128, kv_len=32768, q_len=4, block_size=128, blocks=blocks,
                      dtype=torch.bfloat16, seed=s, causal=True, window=4096, poison=poison)
    if config == 5:
        return mla(config=5, name="mla_bf16_paged64", batch=32, num_heads=128, kv_len=8192, page_size=64,
                   dtype=torch.bfloat16, scale=1.0 / math.sqrt(192), seed=s, poison=poison)
    if config == 6:  # workload 3's lengths and values, the cache quantised to E4M3 with row scales
        s3 = 1003 if seed is None else seed
        g = torch.Generator().manual_seed(s3)
        lens = torch.randint(128, 8193, (64,), generator=g, dtype=torch.int64).tolist()
        return paged(config=6, name="paged_gqa_fp8_ragged", seq_lens=lens, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, page_size=16, dtype=torch.bfloat16, seed=s3 + 1, poison=poison,
                     max_pages=512, kv_format="fp8", kv_scales="token")
    if config == 8:  # workload 3's lengths and values, the cache quantised to int4, one group per row
        s8 = 1003 if seed is None else seed
        g = torch.Generator().manual_seed(s8)
        lens = torch.randint(128, 8193, (64,), generator=g, dtype=torch.int64).tolist()
        return paged(config=8, name="paged_gqa_int4_ragged", seq_lens=lens, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, page_size=16, dtype=torch.bfloat16, seed=s8 + 1, poison=poison,
                     max_pages=512, kv_format="int4", kv_groups=1)
    if config == 7:  # workload 3's shape with 1-8 draft tokens per sequence and a token tree each
        s7 = 1007 if seed is None else seed
        g = torch.Generator().manual_seed(s7)
        lens = torch.randint(128, 8193, (64,), generator=g, dtype=torch.int64).tolist()
        counts = torch.randint(1, 9, (64,), generator=g, dtype=torch.int64).tolist()
        base = paged(config=7, name="paged_gqa_bf16_spec_tree", seq_lens=lens, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, page_size=16, q_len=8, dtype=torch.bfloat16, seed=s7 + 1, poison=poison,
                     max_pages=512)
        return with_spec(base, counts=counts, tree=True, seed=s7 + 2)
    raise ValueError(f"unknown workload {config}")
