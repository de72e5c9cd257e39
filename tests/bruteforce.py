"""Independent dense float64 brute force for tiny inputs (test helper).

Builds the full [S, S] boolean attend mask key by key (key c of query row r
is attended iff c's block is in r's selected set and c % block < vbs), then
takes an ordinary natural-exp masked softmax with numpy.  It shares nothing
with the C oracle: other language, other formulation (dense mask, natural
exponent, library logsumexp).
"""

from __future__ import annotations

import numpy as np
import torch
from scipy.special import logsumexp

LSE_EMPTY = float(np.finfo(np.float32).min)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def selected_sets(w) -> list:
    """Python sets of selected key blocks, indexed by unit u=(b*H+h)*NQ+qb."""
    NQ, NK = w.NQ, w.NK
    out = []
    for b in range(w.B):
        for h in range(w.H):
            for qb in range(NQ):
                if w.form == "lut":
                    sb, sh = w.meta_strides
                    row = b * sb + h * sh + qb
                    n = int(w.q2k_num[row])
                    n = max(0, min(n, w.q2k_idx.shape[-1]))
                    s = {int(x) for x in w.q2k_idx[row, :n].tolist()
                         if 0 <= int(x) < NK}
                else:
                    sb, sh = w.mask_strides
                    row = b * sb + h * sh + qb
                    s = {kb for kb in range(NK) if int(w.mask[row, kb]) != 0}
                out.append(s)
    return out


def dense_mask(w) -> np.ndarray:
    """[B, H, Sq, Sk] bool attend mask."""
    S, Sk, blk, NQ, NK = w.S, w.Sk, w.block, w.NQ, w.NK
    vbs = [blk] * NK if w.vbs is None else [
        max(0, min(blk, int(x))) for x in w.vbs.tolist()]
    sets = selected_sets(w)
    m = np.zeros((w.B, w.H, S, Sk), dtype=bool)
    for u, sel in enumerate(sets):
        qb = u % NQ
        h = (u // NQ) % w.H
        b = u // (NQ * w.H)
        for c in range(Sk):
            if c // blk in sel and c % blk < vbs[c // blk]:
                m[b, h, qb * blk:(qb + 1) * blk, c] = True
    return m


def codebook_values(codes: torch.Tensor, codebook: torch.Tensor) -> np.ndarray:
    """float64 codebook levels of i8 codes (level = code + 128) or of uint8
    bytes holding two i4 codes (element 2i in the low nibble, level =
    code + 8), by numpy indexing."""
    cb = codebook.to(torch.float64).numpy()
    c = codes.numpy()
    if c.dtype == np.int8:
        return cb[c.astype(np.int64) + 128]
    lo = (c & 15).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    idx = np.stack([lo, hi], axis=-1).reshape(*c.shape[:-1], c.shape[-1] * 2)
    return cb[idx + 8]


def kv_f64(w):
    """Decoded K and V as float64 [B,H,Sk,D], one copy per query head
    (query head h uses K/V head h // (H // Hk)); fp8: code value x block
    scale, decoded by torch's float8_e4m3fn."""
    if w.kv_fp8 or w.kv_codebook:
        if w.kv_fp8:
            k = to_f64(w.k.to(torch.float32))
            v = to_f64(w.v.to(torch.float32))
        else:
            k = codebook_values(w.k, w.k_codebook)
            v = codebook_values(w.v, w.v_codebook)
        ks = np.repeat(to_f64(w.k_scale), w.block, axis=-1)[..., None]
        vs = np.repeat(to_f64(w.v_scale), w.block, axis=-1)[..., None]
        k, v = k * ks, v * vs
    else:
        k, v = to_f64(w.k), to_f64(w.v)
    group = w.H // w.Hk
    return np.repeat(k, group, axis=1), np.repeat(v, group, axis=1)


def attention(w, mask=None):
    """(O [B,H,S,D], LSE base 2 [B,H,S]) by dense masked softmax."""
    if mask is None:
        mask = dense_mask(w)
    q = to_f64(w.q)
    k, v = kv_f64(w)
    logits = np.einsum("bhsd,bhtd->bhst", q, k) * w.sm_scale
    logits = np.where(mask, logits, -np.inf)
    any_key = mask.any(axis=-1)
    safe = np.where(any_key[..., None], logits, 0.0)
    lse_e = logsumexp(safe, axis=-1)
    p = np.where(mask, np.exp(safe - lse_e[..., None]), 0.0)
    o = np.einsum("bhst,bhtd->bhsd", p, v)
    o = np.where(any_key[..., None], o, 0.0)
    lse2 = np.where(any_key, lse_e / np.log(2.0), LSE_EMPTY)
    return o, lse2


def grads_autograd(w, dout, mask=None):
    """(dq, dk, dv) of sum(O * dout) by torch autograd through a dense
    float64 masked softmax (bf16 K/V; GQA by repeating K/V heads, whose
    gradients autograd sums back).  Rows with no attended key output 0."""
    if mask is None:
        mask = dense_mask(w)
    m = torch.from_numpy(mask)
    q = w.q.to(torch.float64).requires_grad_(True)
    k = w.k.to(torch.float64).requires_grad_(True)
    v = w.v.to(torch.float64).requires_grad_(True)
    group = w.H // w.Hk
    kr = k.repeat_interleave(group, dim=1)
    vr = v.repeat_interleave(group, dim=1)
    logits = torch.matmul(q, kr.transpose(-1, -2)) * w.sm_scale
    a = torch.where(m, logits, torch.full_like(logits, -torch.inf))
    mx = a.max(dim=-1, keepdim=True).values.detach()
    mx = torch.where(torch.isfinite(mx), mx, torch.zeros_like(mx))
    e = torch.where(m, torch.exp(a - mx), torch.zeros_like(a))
    den = e.sum(dim=-1, keepdim=True)
    p = e / torch.where(den > 0, den, torch.ones_like(den))
    o = torch.matmul(p, vr)
    (o * dout.to(torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()
