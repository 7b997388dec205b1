"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` handle and raises AssertionError when the oracle disagrees
with a library routine (PyTorch's scaled_dot_product_attention / logsumexp in fp64), a closed
form, a hand-listed visibility set (tests/golden/visibility.json) or an invariant the method
must satisfy (paging, splitting, layout, widening). The pins are plain functions so the mutation
test can run them against deliberately broken builds of the oracle.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _gen(seed):
    return torch.Generator().manual_seed(seed)


def _randn(g, *shape, dtype=torch.float64):
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    diff = np.where(same_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), f"{what}: non-finite mismatch"
    assert diff.max(initial=0.0) <= tol, f"{what}: max |diff| {diff.max()} > {tol}"


def _sdpa(q, k, v, scale, mask):
    """Library attention: q [B,Q,Hq,D], k/v [B,L,Hkv,D], mask [B,Q,L] bool (True = visible).
    Returns out [B,Q,Hq,Dv] and lse [B,Q,Hq], both fp64."""
    B, Q, Hq, _ = q.shape
    Hkv = k.shape[2]
    qh = q.permute(0, 2, 1, 3).double()
    kh = k.permute(0, 2, 1, 3).double().contiguous()
    vh = v.permute(0, 2, 1, 3).double().contiguous()
    m = mask[:, None, :, :]
    out = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=m, scale=scale, enable_gqa=True)
    kx = kh.repeat_interleave(Hq // Hkv, dim=1)
    s = torch.matmul(qh, kx.transpose(-1, -2).contiguous()) * scale
    lse = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def _library_mask(B, Q, L, seq_lens, causal, window):
    """Visibility from torch's triangular-matrix routines: tril/triu with a diagonal offset put
    each query at the bottom-right (position L - Q + t)."""
    masks = []
    for b in range(B):
        Lb = int(seq_lens[b])
        m = torch.zeros(Q, L, dtype=torch.bool)
        sub = torch.ones(Q, Lb, dtype=torch.bool)
        if causal:
            sub = sub.tril(diagonal=Lb - Q)
        if window:
            sub = sub.triu(diagonal=Lb - Q - window + 1)
        m[:, :Lb] = sub
        masks.append(m)
    return torch.stack(masks)


# ---------------------------------------------------------------------------------------------
def pin_library_attention(orc):
    """Ragged GQA attention equals PyTorch SDPA (fp64) and logsumexp."""
    g = _gen(11)
    B, Q, Hq, Hkv, D, Dv, L = 3, 1, 6, 2, 8, 5, 13
    q = _randn(g, B, Q, Hq, D)
    k = _randn(g, B, L, Hkv, D)
    v = _randn(g, B, L, Hkv, Dv)
    lens = torch.tensor([13, 9, 1], dtype=torch.int32)
    scale = 0.37
    out, lse = orc.attend(q, k, v, scale=scale, seq_lens=lens)
    ref_o, ref_l = _sdpa(q, k, v, scale, _library_mask(B, Q, L, lens, False, 0))
    _close(out, ref_o, what="out")
    _close(lse, ref_l, what="lse")


def pin_library_causal_window(orc):
    """Multi-query decode with bottom-right causal + window equals SDPA with a tril/triu mask."""
    g = _gen(12)
    B, Q, Hq, Hkv, D, L = 2, 4, 8, 2, 6, 19
    q = _randn(g, B, Q, Hq, D)
    k = _randn(g, B, L, Hkv, D)
    v = _randn(g, B, L, Hkv, D)
    lens = torch.tensor([19, 11], dtype=torch.int32)
    for causal, window in ((True, 0), (True, 5), (False, 7)):
        out, lse = orc.attend(q, k, v, scale=0.5, seq_lens=lens, causal=causal, window=window)
        ref_o, ref_l = _sdpa(q, k, v, 0.5, _library_mask(B, Q, L, lens, causal, window))
        _close(out, ref_o, what=f"out causal={causal} window={window}")
        _close(lse, ref_l, what=f"lse causal={causal} window={window}")


def pin_library_block_list(orc):
    """A block list equals SDPA with a mask built from block membership (torch.isin)."""
    g = _gen(13)
    B, Q, Hq, Hkv, D, L, bs = 2, 2, 4, 2, 8, 24, 4
    q = _randn(g, B, Q, Hq, D)
    k = _randn(g, B, L, Hkv, D)
    v = _randn(g, B, L, Hkv, D)
    lens = torch.tensor([24, 22], dtype=torch.int32)
    blocks = torch.tensor([[[1, 2, 5], [0, 3, 5]], [[2, 4, 5], [5, 1, 0]]], dtype=torch.int32)
    nb = torch.tensor([[3, 2], [3, 3]], dtype=torch.int32)
    out, lse = orc.attend(q, k, v, scale=0.3, seq_lens=lens, num_blocks=nb, block_idx=blocks,
                          block_size=bs, causal=True, window=9)
    base = _library_mask(B, Q, L, lens, True, 9)
    for b in range(B):
        for h in range(Hkv):
            listed = blocks[b, h, : nb[b, h]].long()
            keep = torch.isin(torch.arange(L) // bs, listed)
            m = base[b:b + 1] & keep
            qq = q[b:b + 1, :, h * 2:(h + 1) * 2]
            ro, rl = _sdpa(qq, k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1], 0.3, m)
            _close(out[b:b + 1, :, h * 2:(h + 1) * 2], ro, what=f"out b={b} h={h}")
            _close(lse[b:b + 1, :, h * 2:(h + 1) * 2], rl, what=f"lse b={b} h={h}")


def pin_golden_visibility(orc):
    """scale = 0 and one-hot V reveal the visible set: out_j = 1/n for visible j, lse = ln n."""
    with open(os.path.join(GOLDEN, "visibility.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        L, Q = c["kv_len"], c["q_len"]
        q = torch.ones(1, Q, 1, 4, dtype=torch.float64)
        k = torch.ones(1, max(L, 1), 1, 4, dtype=torch.float64)
        v = torch.eye(max(L, 1), dtype=torch.float64).view(1, max(L, 1), 1, max(L, 1))
        kw = dict(scale=0.0, seq_lens=torch.tensor([L], dtype=torch.int32),
                  causal=c["causal"], window=c["window"])
        if c["blocks"] is not None:
            kw.update(num_blocks=torch.tensor([[len(c["blocks"])]], dtype=torch.int32),
                      block_idx=torch.tensor([[c["blocks"]]], dtype=torch.int32),
                      block_size=c["block_size"])
        out, lse = orc.attend(q, k, v, **kw)
        for t, vis in enumerate(c["visible"]):
            expect = np.zeros(max(L, 1))
            if vis:
                expect[vis] = 1.0 / len(vis)
                assert abs(lse[0, t, 0] - math.log(len(vis))) <= TOL, f"{c['name']} t={t} lse"
            else:
                assert lse[0, t, 0] == -math.inf, f"{c['name']} t={t}: expected an empty row"
            _close(out[0, t, 0], expect, what=f"{c['name']} t={t}")


def pin_one_visible_key(orc):
    """A single visible key returns its value row and lse = its logit."""
    g = _gen(14)
    q = _randn(g, 1, 1, 2, 8)
    k = _randn(g, 1, 9, 1, 8)
    v = _randn(g, 1, 9, 1, 8)
    lens = torch.tensor([9], dtype=torch.int32)
    # block 2 of size 4 covers keys 8..11, of which only key 8 exists
    out, lse = orc.attend(q, k, v, scale=0.7, seq_lens=lens, num_blocks=torch.tensor([[1]]),
                          block_idx=torch.tensor([[[2]]]), block_size=4)
    for h in range(2):
        _close(out[0, 0, h], v[0, 8, 0].numpy(), what="out")
        s = 0.7 * float((q[0, 0, h] * k[0, 8, 0]).sum())
        assert abs(lse[0, 0, h] - s) <= TOL, "lse"


def pin_identical_keys(orc):
    """n identical keys with logit s give the mean of their values and lse = s + ln n."""
    g = _gen(15)
    n, D = 7, 8
    q = _randn(g, 1, 1, 1, D)
    k = _randn(g, 1, 1, 1, D).expand(1, n, 1, D).contiguous()
    v = _randn(g, 1, n, 1, D)
    out, lse = orc.attend(q, k, v, scale=0.9)
    s = 0.9 * float((q[0, 0, 0] * k[0, 0, 0]).sum())
    _close(out[0, 0, 0], v[0, :, 0].mean(0).numpy(), what="mean")
    assert abs(lse[0, 0, 0] - (s + math.log(n))) <= TOL


def pin_constant_values(orc):
    """V identical for every key gives that value whatever the scores."""
    g = _gen(16)
    q = _randn(g, 2, 3, 4, 8) * 5
    k = _randn(g, 2, 17, 2, 8)
    c = _randn(g, 8)
    v = c.view(1, 1, 1, 8).expand(2, 17, 2, 8).contiguous()
    out, _ = orc.attend(q, k, v, scale=1.3, seq_lens=torch.tensor([17, 4]), causal=True, window=6)
    for idx in np.ndindex(2, 3, 4):
        _close(out[idx], c.numpy(), tol=1e-13, what="constant V")


def pin_large_logits(orc):
    """Logits near +-1000 (exp overflows without the max shift) match logsumexp."""
    q = torch.tensor([[[[1.0, 0.0]]]], dtype=torch.float64)
    k = torch.tensor([[[1000.0, 0]], [[999.0, 0]], [[-1000.0, 0]]], dtype=torch.float64).view(1, 3, 1, 2)
    v = torch.tensor([[[1.0, 2.0]], [[3.0, 4.0]], [[5.0, 6.0]]], dtype=torch.float64).view(1, 3, 1, 2)
    out, lse = orc.attend(q, k, v, scale=1.0)
    logits = torch.tensor([1000.0, 999.0, -1000.0], dtype=torch.float64)
    w = torch.softmax(logits, 0)
    _close(lse[0, 0, 0], float(torch.logsumexp(logits, 0)), what="lse")
    _close(out[0, 0, 0], (w[:, None] * v[0, :, 0]).sum(0).numpy(), what="out")


def pin_empty_rows(orc):
    """No visible key: out = 0 and lse = -inf (zero-length sequence, empty key range)."""
    g = _gen(17)
    q = _randn(g, 2, 1, 2, 4)
    k = _randn(g, 2, 5, 1, 4)
    v = _randn(g, 2, 5, 1, 4)
    out, lse = orc.attend(q, k, v, scale=1.0, seq_lens=torch.tensor([0, 5], dtype=torch.int32))
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))
    out, lse = orc.attend(q, k, v, scale=1.0, key_range=(5, 9))
    assert np.all(out == 0) and np.all(lse == -np.inf)


def pin_paged_equals_contiguous(orc):
    """The same logical cache scattered over a permuted page pool gives bit-identical results."""
    g = _gen(18)
    B, Q, Hq, Hkv, D, P = 3, 2, 4, 2, 8, 4
    lens = [13, 4, 9]
    L = max(lens)
    q = _randn(g, B, Q, Hq, D)
    k = _randn(g, B, L, Hkv, D)
    v = _randn(g, B, L, Hkv, D)
    npb = [(x + P - 1) // P for x in lens]
    perm = torch.randperm(sum(npb) + 3, generator=g)
    kp = torch.full((sum(npb) + 3, P, Hkv, D), float("nan"), dtype=torch.float64)
    vp = kp.clone()
    bt = torch.full((B, max(npb)), -1, dtype=torch.int32)
    i = 0
    for b in range(B):
        for p in range(npb[b]):
            phys = int(perm[i])
            i += 1
            bt[b, p] = phys
            n = min(P, lens[b] - p * P)
            kp[phys, :n] = k[b, p * P:p * P + n]
            vp[phys, :n] = v[b, p * P:p * P + n]
    sl = torch.tensor(lens, dtype=torch.int32)
    a = orc.attend(q, k, v, scale=0.6, seq_lens=sl, causal=True, window=5)
    b_ = orc.attend(q, kp, vp, scale=0.6, seq_lens=sl, block_table=bt, page_size=P, causal=True, window=5)
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1]), "paged != contiguous"


def pin_layout_and_rows(orc):
    """Head-major storage viewed token-major equals a token-major copy, and a row subset equals
    the same rows of the full result (both bit-identical)."""
    g = _gen(19)
    B, Q, Hq, Hkv, D, L = 2, 1, 8, 4, 8, 11
    q = _randn(g, B, Q, Hq, D)
    kh = _randn(g, B, Hkv, L, D)
    vh = _randn(g, B, Hkv, L, D)
    k_view, v_view = kh.permute(0, 2, 1, 3), vh.permute(0, 2, 1, 3)
    a = orc.attend(q, k_view, v_view, scale=0.4)
    b_ = orc.attend(q, k_view.contiguous(), v_view.contiguous(), scale=0.4)
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1])
    rows = [15, 0, 7, 8]
    o, l_ = orc.attend(q, k_view, v_view, scale=0.4, rows=rows)
    flat_o, flat_l = a[0].reshape(-1, D), a[1].reshape(-1)
    assert np.array_equal(o, flat_o[rows]) and np.array_equal(l_, flat_l[rows])


def pin_widening(orc):
    """bf16 and fp32 inputs are widened exactly: same result as the same values given in fp64."""
    g = _gen(20)
    for dt in (torch.bfloat16, torch.float32):
        q = _randn(g, 1, 1, 2, 8, dtype=dt)
        k = _randn(g, 1, 6, 1, 8, dtype=dt)
        v = _randn(g, 1, 6, 1, 8, dtype=dt)
        a = orc.attend(q, k, v, scale=0.25)
        b_ = orc.attend(q.double(), k.double(), v.double(), scale=0.25)
        assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1]), f"widening {dt}"


def pin_mla_two_part_score(orc):
    """MLA: score = q_nope.ckv + q_pe.kpe with V = ckv equals attention on the concatenated
    576-style key (V = its first columns), and equals SDPA on it."""
    g = _gen(21)
    B, H, L, Dn, Dr = 2, 4, 10, 8, 4
    qn = _randn(g, B, 1, H, Dn)
    qp = _randn(g, B, 1, H, Dr)
    ckv = _randn(g, B, L, 1, Dn)
    kpe = _randn(g, B, L, 1, Dr)
    lens = torch.tensor([10, 6], dtype=torch.int32)
    o1, l1 = orc.attend(qn, ckv, ckv, q2=qp, k2=kpe, scale=0.2, seq_lens=lens)
    qcat = torch.cat([qn, qp], dim=-1)
    kcat = torch.cat([ckv, kpe], dim=-1)
    o2, l2 = orc.attend(qcat, kcat, kcat[..., :Dn], scale=0.2, seq_lens=lens)
    _close(o1, o2, what="two-part vs concatenated out")
    _close(l1, l2, what="two-part vs concatenated lse")
    ro, rl = _sdpa(qcat, kcat, kcat[..., :Dn].contiguous(), 0.2, _library_mask(B, 1, L, lens, False, 0))
    _close(o1, ro, what="MLA vs SDPA out")
    _close(l1, rl, what="MLA vs SDPA lse")


def pin_merge_closed_form(orc):
    """Two partials with lse (0, ln 3) weigh 1 : 3; merged lse = ln 4."""
    po = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    pl = np.array([[0.0, math.log(3.0)]])
    out, lse = orc.merge(po, pl)
    _close(out[0], [0.25, 0.75], what="merged out")
    _close(lse[0], math.log(4.0), what="merged lse")


def pin_merge_identities(orc):
    """S = 1 is the identity; a partial merged with itself keeps o and gains ln 2; an empty
    (0, -inf) slot changes nothing; all-empty gives (0, -inf)."""
    g = np.random.default_rng(22)
    po = g.standard_normal((5, 1, 6))
    pl = g.standard_normal((5, 1))
    o, l_ = orc.merge(po, pl)
    _close(o, po[:, 0], what="S=1 out")
    _close(l_, pl[:, 0], what="S=1 lse")
    o, l_ = orc.merge(np.concatenate([po, po], 1), np.concatenate([pl, pl], 1))
    _close(o, po[:, 0], tol=1e-14, what="self-merge out")
    _close(l_, pl[:, 0] + math.log(2.0), tol=1e-14, what="self-merge lse")
    o, l_ = orc.merge(np.concatenate([po, np.zeros_like(po)], 1),
                      np.concatenate([pl, np.full_like(pl, -np.inf)], 1))
    _close(o, po[:, 0], what="empty slot out")
    _close(l_, pl[:, 0], what="empty slot lse")
    o, l_ = orc.merge(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(o == 0) and np.all(l_ == -np.inf)


def pin_split_then_merge(orc):
    """Attention over key ranges [s*c, (s+1)*c) merged with the LSE weights equals the unsplit
    result, including an empty trailing range."""
    g = _gen(23)
    B, Q, Hq, Hkv, D, L = 2, 2, 4, 2, 8, 37
    q = _randn(g, B, Q, Hq, D)
    k = _randn(g, B, L, Hkv, D)
    v = _randn(g, B, L, Hkv, D)
    lens = torch.tensor([37, 23], dtype=torch.int32)
    whole_o, whole_l = orc.attend(q, k, v, scale=0.45, seq_lens=lens, causal=True)
    c = 10
    parts = [orc.attend(q, k, v, scale=0.45, seq_lens=lens, causal=True, key_range=(s * c, (s + 1) * c))
             for s in range(5)]
    po = np.stack([p[0].reshape(-1, D) for p in parts], axis=1)
    pl = np.stack([p[1].reshape(-1) for p in parts], axis=1)
    assert np.all(pl[:, 4] == -np.inf) and np.all(po[:, 4] == 0)
    mo, ml = orc.merge(po, pl)
    _close(mo, whole_o.reshape(-1, D), what="merged out")
    _close(ml, whole_l.reshape(-1), what="merged lse")


def pin_key_order_invariance(orc):
    """Reordering the keys of an unmasked contiguous cache leaves the result unchanged."""
    g = _gen(24)
    q = _randn(g, 1, 1, 3, 8)
    k = _randn(g, 1, 12, 3, 8)
    v = _randn(g, 1, 12, 3, 8)
    perm = torch.randperm(12, generator=g)
    a = orc.attend(q, k, v, scale=0.8)
    b_ = orc.attend(q, k[:, perm].contiguous(), v[:, perm].contiguous(), scale=0.8)
    _close(a[0], b_[0], what="out")
    _close(a[1], b_[1], what="lse")



# ------------------------------------------------------------------ fp8 (E4M3) cache
def _e4m3_lib(bytes_u8):
    """Library decode of OCP E4M3 bytes (torch.float8_e4m3fn), widened to fp64."""
    return bytes_u8.view(torch.float8_e4m3fn).double()


def _fp8_one_key(orc, v_bytes, k_bytes, ks, vs, q):
    """One sequence, one KV head, one visible key: out = dequantised v row, lse = its logit."""
    Dk, Dv = k_bytes.numel(), v_bytes.numel()
    k = k_bytes.reshape(1, 1, 1, Dk)
    v = v_bytes.reshape(1, 1, 1, Dv)
    kscale = torch.tensor([ks], dtype=torch.float32).reshape(1, 1, 1)
    vscale = torch.tensor([vs], dtype=torch.float32).reshape(1, 1, 1)
    return orc.attend(q, k, v, scale=0.7, seq_lens=torch.tensor([1], dtype=torch.int32),
                      k_scale=kscale, v_scale=vscale)


def pin_e4m3_decode_library(orc):
    """Every non-NaN E4M3 byte, as a value row behind one visible key, comes back as PyTorch's
    float8_e4m3fn decoding times the row scale; the logit uses the key bytes' decoding times the
    key scale."""
    allb = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    finite = allb[(allb & 0x7F) != 0x7F]  # 254 bytes: S.1111.111 is NaN
    g = _gen(31)
    kb = finite[torch.randperm(finite.numel(), generator=g)[:40]]
    q = _randn(g, 1, 1, 2, 40) * 0.01
    for ks, vs in ((1.0, 1.0), (0.375, 2.5), (3.0, 0.0078125)):
        out, lse = _fp8_one_key(orc, finite, kb, ks, vs, q)
        _close(out[0, 0, 0], (_e4m3_lib(finite) * vs).numpy(), tol=0.0, what="dequantised values")
        for h in range(2):
            s = 0.7 * float((q[0, 0, h] * (_e4m3_lib(kb) * ks)).sum())
            assert abs(lse[0, 0, h] - s) <= 1e-12 * max(1.0, abs(s)), "logit of the dequantised key"


def pin_e4m3_closed_forms(orc):
    """Values the E4M3 definition fixes: 0x38 = 1, 0xC0 = -2, 0x7E = 448 (largest), 0x08 = 2^-6
    (smallest normal), 0x01 = 2^-9 (smallest subnormal), 0x80 = 0x00 = 0, 0x39 = 1.125, 0x07 =
    7 * 2^-9, and 0x7F / 0xFF are NaN."""
    codes = torch.tensor([0x38, 0xC0, 0x7E, 0x08, 0x01, 0x80, 0x00, 0x39, 0x07], dtype=torch.int32).to(torch.uint8)
    want = [1.0, -2.0, 448.0, 2.0 ** -6, 2.0 ** -9, -0.0, 0.0, 1.125, 7 * 2.0 ** -9]
    q = torch.zeros(1, 1, 1, 4, dtype=torch.float64)
    kb = torch.tensor([0x38] * 4, dtype=torch.int32).to(torch.uint8)
    out, _ = _fp8_one_key(orc, codes, kb, 1.0, 1.0, q)
    assert out[0, 0, 0].tolist() == want, out[0, 0, 0].tolist()  # (an output of -0 reads as +0)
    nan_row = torch.tensor([0x7F, 0xFF, 0x38], dtype=torch.int32).to(torch.uint8)
    out, _ = _fp8_one_key(orc, nan_row, kb, 1.0, 1.0, q)
    assert math.isnan(out[0, 0, 0, 0]) and math.isnan(out[0, 0, 0, 1]) and out[0, 0, 0, 2] == 1.0


def _fp8_cache(g, B, L, Hkv, D):
    """Random E4M3 bytes (no NaN codes) for K and V, plus positive row scales for each, the K
    scales stored head-major and the V scales token-major (different strides)."""
    def bytes_():
        x = torch.randint(0, 256, (B, L, Hkv, D), generator=g, dtype=torch.int32)
        x = torch.where((x & 0x7F) == 0x7F, x - 1, x)
        return x.to(torch.uint8)
    k, v = bytes_(), bytes_()
    ks = (torch.rand(B, Hkv, L, generator=g, dtype=torch.float64) * 0.1 + 0.01).float().permute(0, 2, 1)
    vs = (torch.rand(B, L, Hkv, generator=g, dtype=torch.float64) * 0.1 + 0.01).float()
    return k, v, ks, vs


def pin_fp8_equals_dequantised(orc):
    """Attention over an E4M3 cache with row scales equals attention over the fp64 cache built by
    PyTorch's decoding times the scales (GQA, ragged lengths, causal + window, two query tokens)."""
    g = _gen(32)
    B, Q, Hq, Hkv, D, L = 3, 2, 4, 2, 16, 23
    k, v, ks, vs = _fp8_cache(g, B, L, Hkv, D)
    q = _randn(g, B, Q, Hq, D) * 0.05
    lens = torch.tensor([23, 5, 17], dtype=torch.int32)
    kd = _e4m3_lib(k) * ks.double()[..., None]
    vd = _e4m3_lib(v) * vs.double()[..., None]
    a = orc.attend(q, k, v, scale=0.8, seq_lens=lens, causal=True, window=9, k_scale=ks, v_scale=vs)
    b = orc.attend(q, kd, vd, scale=0.8, seq_lens=lens, causal=True, window=9)
    _close(a[0], b[0], tol=1e-12, what="out")
    _close(a[1], b[1], tol=1e-12, what="lse")


def pin_fp8_paged_and_broadcast(orc):
    """An E4M3 cache and its scales scattered over a permuted page pool give the contiguous result
    bit for bit; one scale per tensor given with zero strides equals a full scale array holding
    that value everywhere."""
    g = _gen(33)
    B, Q, Hq, Hkv, D, P = 2, 1, 4, 2, 8, 4
    lens = [11, 6]
    L = max(lens)
    k, v, ks, vs = _fp8_cache(g, B, L, Hkv, D)
    q = _randn(g, B, Q, Hq, D) * 0.05
    npb = [(x + P - 1) // P for x in lens]
    perm = torch.randperm(sum(npb) + 2, generator=g)
    kp = torch.full((sum(npb) + 2, P, Hkv, D), 0x7F, dtype=torch.uint8)  # NaN where nothing belongs
    vp = kp.clone()
    ksp = torch.full((sum(npb) + 2, P, Hkv), float("nan"), dtype=torch.float32)
    vsp = ksp.clone()
    bt = torch.full((B, max(npb)), -1, dtype=torch.int32)
    i = 0
    for b in range(B):
        for p in range(npb[b]):
            phys = int(perm[i])
            i += 1
            bt[b, p] = phys
            n = min(P, lens[b] - p * P)
            kp[phys, :n], vp[phys, :n] = k[b, p * P:p * P + n], v[b, p * P:p * P + n]
            ksp[phys, :n], vsp[phys, :n] = ks[b, p * P:p * P + n], vs[b, p * P:p * P + n]
    sl = torch.tensor(lens, dtype=torch.int32)
    a = orc.attend(q, k, v, scale=0.9, seq_lens=sl, k_scale=ks, v_scale=vs)
    b_ = orc.attend(q, kp, vp, scale=0.9, seq_lens=sl, block_table=bt, page_size=P, k_scale=ksp, v_scale=vsp)
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1]), "paged fp8 != contiguous fp8"
    one_k = torch.tensor([0.03125], dtype=torch.float32).reshape(1, 1, 1).expand(B, L, Hkv)
    one_v = torch.tensor([0.0625], dtype=torch.float32).reshape(1, 1, 1).expand(B, L, Hkv)
    c = orc.attend(q, k, v, scale=0.9, seq_lens=sl, k_scale=one_k, v_scale=one_v)
    d = orc.attend(q, k, v, scale=0.9, seq_lens=sl, k_scale=one_k.contiguous(), v_scale=one_v.contiguous())
    assert one_k.stride() == (0, 0, 0)
    assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1]), "broadcast scale != full array"


# ------------------------------------------------------------------ speculative decoding
def _random_tree(g, n):
    """Parent of draft token i (i >= 1) uniform in [0, i); token 0 is the root."""
    return [-1] + [int(torch.randint(0, i, (1,), generator=g)) for i in range(1, n)]


def _tree_dense(parents):
    """[n, n] bool: token t sees draft key i iff i is t or one of its ancestors (walks the parent
    pointers; no bit packing involved)."""
    n = len(parents)
    m = torch.zeros(n, n, dtype=torch.bool)
    for t in range(n):
        i = t
        while i >= 0:
            m[t, i] = True
            i = parents[i]
    return m


def _pack_rows(dense, words):
    """bool [rows, <= 32*words] -> int32 [rows, words], bit i of the row at word i // 32, bit i % 32
    (numpy's little-endian bit packing, read back as little-endian 32-bit words)."""
    rows = dense.shape[0]
    full = np.zeros((rows, 32 * words), dtype=np.uint8)
    full[:, :dense.shape[1]] = dense.numpy()
    by = np.packbits(full, axis=1, bitorder="little")
    return torch.from_numpy(by.view("<u4").astype(np.int64).astype(np.int32).reshape(rows, words))


def _spec_problem(g, Qs, lens, Qmax, Hq=4, Hkv=2, D=6):
    B = len(Qs)
    L = max(lens)
    starts = torch.tensor([0] + list(np.cumsum(Qs)), dtype=torch.int32)
    T = int(starts[-1])
    q = _randn(g, T, Hq, D)
    k = _randn(g, B, L, Hkv, D)
    v = _randn(g, B, L, Hkv, D)
    return q, k, v, starts, torch.tensor(lens, dtype=torch.int32)


def pin_tree_mask_library(orc):
    """Packed tree masks over ragged draft counts (some above 32, so rows span two words) equal
    SDPA per sequence with a dense mask from the trees' ancestor sets, alone and with causal +
    window."""
    g = _gen(31)
    Qmax = 40
    Qs, lens = [5, 40, 0, 1, 33], [23, 61, 9, 4, 40]
    q, k, v, starts, sl = _spec_problem(g, Qs, lens, Qmax)
    W = (Qmax + 31) // 32
    dense_rows, trees = [], []
    for b, n in enumerate(Qs):
        tr = _tree_dense(_random_tree(g, n)) if n else torch.zeros(0, 0, dtype=torch.bool)
        trees.append(tr)
        dense_rows.append(tr)
    tm = _pack_rows(torch.cat([torch.nn.functional.pad(t, (0, Qmax - t.shape[1])) for t in dense_rows]), W)
    # and an arbitrary bit pattern (rows need not contain the first draft, or themselves)
    bits = [torch.rand(n, n, generator=g) < 0.5 for n in Qs]
    tb = _pack_rows(torch.cat([torch.nn.functional.pad(t, (0, Qmax - t.shape[1])) for t in bits]), W)
    for causal, window, mask, dense in ((False, 0, tm, trees), (True, 17, tm, trees), (False, 0, tb, bits)):
        out, lse = orc.attend(q, k, v, scale=0.45, seq_lens=sl, q_starts=starts, q_len=Qmax, tree_mask=mask,
                              causal=causal, window=window)
        for b, n in enumerate(Qs):
            if n == 0:
                continue
            Lb, s0 = lens[b], int(starts[b])
            m = _library_mask(1, n, Lb, [Lb], causal, window)[0]
            m[:, Lb - n:] &= dense[b]
            ro, rl = _sdpa(q[None, s0:s0 + n], k[b:b + 1, :Lb], v[b:b + 1, :Lb], 0.45, m[None])
            _close(out[s0:s0 + n], ro[0], what=f"out b={b} causal={causal}")
            _close(lse[s0:s0 + n], rl[0], what=f"lse b={b} causal={causal}")


def pin_tree_chain_is_causal(orc):
    """A chain-shaped tree (token t sees drafts 0..t) is the bottom-right causal mask, and a mask
    with every bit set changes nothing."""
    g = _gen(32)
    B, Q, Hq, Hkv, D, L = 3, 6, 4, 2, 5, 17
    q = _randn(g, B, Q, Hq, D)
    k = _randn(g, B, L, Hkv, D)
    v = _randn(g, B, L, Hkv, D)
    lens = torch.tensor([17, 6, 11], dtype=torch.int32)
    chain = torch.ones(Q, Q, dtype=torch.bool).tril()
    tm = _pack_rows(chain.repeat(B, 1), 1)
    a = orc.attend(q, k, v, scale=0.6, seq_lens=lens, tree_mask=tm)
    c = orc.attend(q, k, v, scale=0.6, seq_lens=lens, causal=True)
    _close(a[0], c[0], what="chain out")
    _close(a[1], c[1], what="chain lse")
    every = torch.full((B * Q, 1), -1, dtype=torch.int32)
    a = orc.attend(q, k, v, scale=0.6, seq_lens=lens, tree_mask=every, window=4)
    c = orc.attend(q, k, v, scale=0.6, seq_lens=lens, window=4)
    _close(a[0], c[0], what="all-ones out")
    _close(a[1], c[1], what="all-ones lse")


def pin_varlen_equals_separate(orc):
    """Packed queries with per-sequence token counts (including 0) equal each sequence computed
    alone with its own q_len, causal and windowed."""
    g = _gen(33)
    Qs, lens = [3, 0, 1, 4], [12, 5, 9, 4]
    q, k, v, starts, sl = _spec_problem(g, Qs, lens, 4)
    for causal, window in ((True, 0), (True, 3), (False, 0)):
        out, lse = orc.attend(q, k, v, scale=0.8, seq_lens=sl, q_starts=starts, q_len=4,
                              causal=causal, window=window)
        assert out.shape == (sum(Qs), 4, 6)
        for b, n in enumerate(Qs):
            if n == 0:
                continue
            s0 = int(starts[b])
            ro, rl = orc.attend(q[None, s0:s0 + n], k[b:b + 1], v[b:b + 1], scale=0.8,
                                seq_lens=sl[b:b + 1], causal=causal, window=window)
            _close(out[s0:s0 + n], ro[0], what=f"out b={b}")
            _close(lse[s0:s0 + n], rl[0], what=f"lse b={b}")
    # a packed row below q_starts[0] belongs to no sequence
    shifted = starts + 2
    qq = torch.cat([_randn(g, 2, 4, 6), q])
    out, lse = orc.attend(qq, k, v, scale=0.8, seq_lens=sl, q_starts=shifted, q_len=4)
    assert np.all(out[:2] == 0) and np.all(np.isneginf(lse[:2]))
    ref = orc.attend(q, k, v, scale=0.8, seq_lens=sl, q_starts=starts, q_len=4)
    _close(out[2:], ref[0], what="offset start out")


# ------------------------------------------------------------------ int4 cache
def _int4_rows(g, rows_shape, D, n_groups):
    """Random 4-bit fields, fp16 scales and shifts per (row, group), the packed int32 rows built
    from them with numpy bit operations, and the dequantised values computed from the fields
    directly (field * scale + shift in fp64)."""
    n = torch.randint(0, 16, (*rows_shape, D), generator=g)
    sc = (torch.rand(*rows_shape, n_groups, generator=g) * 0.2 + 1e-3).to(torch.float16)
    sh = (torch.randn(*rows_shape, n_groups, generator=g)).to(torch.float16)
    sc.view(-1)[0] = torch.tensor(3e-6, dtype=torch.float16)  # a subnormal half scale
    gs = D // n_groups
    deq = n.double() * sc.double().repeat_interleave(gs, -1) + sh.double().repeat_interleave(gs, -1)
    nn = n.numpy().astype(np.uint32).reshape(-1, D // 8, 8)
    packed = np.zeros(nn.shape[:2], dtype=np.uint32)
    for j in range(8):
        packed |= nn[:, :, j] << np.uint32(4 * j)
    coef = (sc.view(torch.int16).numpy().astype(np.uint32) & 0xFFFF) | \
           ((sh.view(torch.int16).numpy().astype(np.uint32) & 0xFFFF) << 16)
    words = np.concatenate([coef.reshape(-1, n_groups), packed], axis=1)
    t = torch.from_numpy(words.view(np.int32).copy()).reshape(*rows_shape, n_groups + D // 8)
    return t, deq


def pin_int4_library(orc):
    """Attention over packed int4 rows (1, 2, 4 and 8 groups; a subnormal half scale) equals fp64
    SDPA over the values computed from the fields; the paged layout gives the same bits."""
    g = _gen(41)
    B, Q, Hq, Hkv, D, L, P = 2, 2, 4, 2, 64, 21, 8
    lens = torch.tensor([21, 13], dtype=torch.int32)
    q = _randn(g, B, Q, Hq, D)
    for ng in (1, 2, 4, 8):
        kw, kd = _int4_rows(g, (B, Hkv, L), D, ng)
        vw, vd = _int4_rows(g, (B, Hkv, L), D, ng)
        k, v = kw.permute(0, 2, 1, 3), vw.permute(0, 2, 1, 3)
        out, lse = orc.attend(q, k, v, scale=0.3, seq_lens=lens, causal=True, int4_groups=ng)
        ref_o, ref_l = _sdpa(q, kd.permute(0, 2, 1, 3), vd.permute(0, 2, 1, 3), 0.3,
                             _library_mask(B, Q, L, lens, True, 0))
        _close(out, ref_o, what=f"int4 out groups={ng}")
        _close(lse, ref_l, what=f"int4 lse groups={ng}")
        # paged: page p of sequence b is pool page perm[b*npg + p]
        npg = (L + P - 1) // P
        perm = torch.randperm(B * npg, generator=g)
        pool_k = torch.zeros(B * npg, Hkv, P, ng + D // 8, dtype=torch.int32)
        pool_v = torch.zeros_like(pool_k)
        kp = torch.nn.functional.pad(kw, (0, 0, 0, npg * P - L))
        vp = torch.nn.functional.pad(vw, (0, 0, 0, npg * P - L))
        for b in range(B):
            for pg in range(npg):
                pool_k[perm[b * npg + pg]] = kp[b, :, pg * P:(pg + 1) * P]
                pool_v[perm[b * npg + pg]] = vp[b, :, pg * P:(pg + 1) * P]
        bt = perm.reshape(B, npg).to(torch.int32)
        o2, l2 = orc.attend(q, pool_k.permute(0, 2, 1, 3), pool_v.permute(0, 2, 1, 3), scale=0.3, seq_lens=lens,
                            causal=True, block_table=bt, page_size=P, int4_groups=ng)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2), f"paged int4 != contiguous, groups={ng}"


def pin_int4_one_key(orc):
    """One visible key: the output is that key's value row, field * scale + shift, exactly."""
    g = _gen(42)
    D = 64
    for ng in (1, 8):
        kw, _ = _int4_rows(g, (1, 1, 1), D, ng)
        vw, vd = _int4_rows(g, (1, 1, 1), D, ng)
        q = _randn(g, 1, 1, 1, D)
        out, lse = orc.attend(q, kw.permute(0, 2, 1, 3), vw.permute(0, 2, 1, 3), scale=1.0, int4_groups=ng)
        assert np.array_equal(out.reshape(-1), vd.reshape(-1).numpy()), f"one key, groups={ng}"


ALL_PINS = [
    pin_library_attention, pin_library_causal_window, pin_library_block_list, pin_golden_visibility,
    pin_one_visible_key, pin_identical_keys, pin_constant_values, pin_large_logits, pin_empty_rows,
    pin_paged_equals_contiguous, pin_layout_and_rows, pin_widening, pin_mla_two_part_score,
    pin_merge_closed_form, pin_merge_identities, pin_split_then_merge, pin_key_order_invariance,
    pin_e4m3_decode_library, pin_e4m3_closed_forms, pin_fp8_equals_dequantised, pin_fp8_paged_and_broadcast,
    pin_tree_mask_library, pin_tree_chain_is_causal, pin_varlen_equals_separate,
    pin_int4_library, pin_int4_one_key,
]


def run_all(orc):
    """Run every pin; return the names of the pins that failed (or raised)."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            failed.append(f"{pin.__name__}: {type(e).__name__}: {str(e)[:120]}")
    return failed
