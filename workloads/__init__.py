"""Seeded synthetic inputs for block-sparse attention forward.

This module only draws inputs: it holds none of the attention arithmetic, and
both the HIP path and the CPU oracle consume what it makes.  Everything is
drawn on the CPU from ``torch.Generator().manual_seed(seed)`` in a fixed
order (Q, K, V, then the sparsity metadata), so a seed names an input.

The five named workloads follow the shapes and value distributions of the
block-sparse attention problem statement (FastVideo "block_sparse_attn_sm100a.py":
BHSD bf16 tensors, head dim 128, 64- and 128-token blocks, per-row LUT counts
that may be zero, -1 padding, per-block valid-token counts; rocke
"sparse_attention.py": an i8 Jenga mask bitmap; rocke "sage_attention.py":
fp8 e4m3 K/V with per-block fp32 scales).  They stand in for video-model
attention inputs; no dataset is used.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

HEAD_DIM = 128


@dataclass
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    block: int
    form: str  # "lut" or "bitmap"
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    k_scale: Optional[torch.Tensor] = None  # fp32 [B, Hk, NK] (fp8 K/V only)
    v_scale: Optional[torch.Tensor] = None
    q2k_idx: Optional[torch.Tensor] = None  # int32 [rows, max_kv]
    q2k_num: Optional[torch.Tensor] = None  # int32 [rows]
    meta_strides: tuple = (0, 0)  # (sb, sh): row of (b, h, qb) = b*sb + h*sh + qb
    mask: Optional[torch.Tensor] = None  # int8 [rows, NK]
    mask_strides: tuple = (0, 0)
    vbs: Optional[torch.Tensor] = None  # int32 [NK] or None (all full)
    k_codebook: Optional[torch.Tensor] = None  # fp32 [256] (i8) / [16] (i4)
    v_codebook: Optional[torch.Tensor] = None
    sm_scale: float = 1.0 / (HEAD_DIM ** 0.5)
    extra: dict = field(default_factory=dict)

    @property
    def NQ(self) -> int:
        return self.S // self.block

    @property
    def Hk(self) -> int:
        """Key/value heads (query head h reads K/V head h // (H // Hk))."""
        return int(self.k.shape[1])

    @property
    def Sk(self) -> int:
        """Key sequence length."""
        return int(self.k.shape[2])

    @property
    def NK(self) -> int:
        return self.Sk // self.block

    @property
    def n_units(self) -> int:
        return self.B * self.H * self.NQ

    @property
    def kv_fp8(self) -> bool:
        return self.k.dtype == torch.float8_e4m3fn

    @property
    def kv_codebook(self) -> bool:
        """K/V stored as i8 codes (int8) or packed i4 codes (uint8)."""
        return self.k.dtype in (torch.int8, torch.uint8)


CONFIG_NAMES = [
    "vsa_tiny_b1h1s512_blk64",
    "jenga_bitmap_b1h16s4096_blk64_p0.5",
    "vsa_video_b1h24s49152_blk64_96of768",
    "vsa_blk128_b1h40s32768_counts0to64",
    "vsa_fp8kv_b2h12s16384_blk64_64of256",
]


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def _randn(g, shape, std=1.0, dtype=torch.bfloat16):
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def _distinct_rows(g, rows: int, nk: int, take: int) -> torch.Tensor:
    """``rows`` independent draws of ``take`` distinct block indices in
    [0, nk), each row in random order (first ``take`` of a random
    permutation)."""
    r = torch.rand((rows, nk), generator=g)
    return r.argsort(dim=-1)[:, :take].to(torch.int32)


def quantize_fp8_per_block(x: torch.Tensor, block: int):
    """Per-(b, h, key block) fp8 e4m3 quantisation of an fp32 [B,H,S,D]
    tensor: scale = amax/448 over each [block, D] tile, codes =
    (x/scale) cast to float8_e4m3fn.  Returns (codes, scale [B,H,NK])."""
    B, H, S, D = x.shape
    t = x.reshape(B, H, S // block, block * D)
    amax = t.abs().amax(dim=-1)
    scale = (amax / 448.0).clamp_min(torch.finfo(torch.float32).tiny)
    codes = (t / scale[..., None]).to(torch.float8_e4m3fn).reshape(B, H, S, D)
    return codes, scale.to(torch.float32).contiguous()


def make_codebook(g, n: int) -> torch.Tensor:
    """A sorted, nonuniform fp32 codebook of n levels whose values are exact
    in bf16 (seeded normal draws, rounded to bf16)."""
    cb = torch.randn((n,), generator=g, dtype=torch.float32).sort().values
    return cb.to(torch.bfloat16).to(torch.float32).contiguous()


def quantize_codebook_per_block(x: torch.Tensor, block: int,
                                codebook: torch.Tensor, bits: int):
    """Per-(b, h, key block) codebook quantisation of an fp32 [B,H,S,D]
    tensor: scale = amax / max|codebook| over each [block, D] tile, code =
    the nearest codebook level of x/scale.  bits 8: int8 codes in [-128, 127]
    (level = code + 128); bits 4: uint8 bytes of two codes in [-8, 7] (level
    = code + 8), element 2i in the low nibble.  Returns (codes, scale
    [B,H,NK])."""
    B, H, S, D = x.shape
    t = x.reshape(B, H, S // block, block * D)
    amax = t.abs().amax(dim=-1)
    scale = (amax / codebook.abs().max()).clamp_min(torch.finfo(torch.float32).tiny)
    y = (t / scale[..., None]).reshape(-1)
    # nearest level: compare with the midpoints of the sorted codebook
    mids = (codebook[1:] + codebook[:-1]) * 0.5
    level = torch.searchsorted(mids, y.contiguous())
    level = level.reshape(B, H, S, D)
    if bits == 8:
        codes = (level - 128).to(torch.int8)
    else:
        c = (level - 8) & 15  # two's complement nibbles
        codes = (c[..., 0::2] | (c[..., 1::2] << 4)).to(torch.uint8)
    return codes.contiguous(), scale.to(torch.float32).contiguous()


def make_config(i: int, seed: Optional[int] = None) -> Workload:
    """Named workload i (0..4), drawn with ``seed`` (default: i)."""
    g = _gen(i if seed is None else seed)
    D = HEAD_DIM
    if i == 0:  # tiny VSA LUT case: the oracle finishes it in well under a second
        B, H, S, blk = 1, 1, 512, 64
        NQ = S // blk
        q, k, v = (_randn(g, (B, H, S, D)) for _ in range(3))
        rows = B * H * NQ
        idx = torch.full((rows, 8), -1, dtype=torch.int32)
        idx[:, :4] = _distinct_rows(g, rows, NQ, 4)
        num = torch.full((rows,), 4, dtype=torch.int32)
        vbs = torch.tensor([64] * 7 + [40], dtype=torch.int32)
        return Workload(CONFIG_NAMES[0], B, H, S, D, blk, "lut", q, k, v,
                        q2k_idx=idx, q2k_num=num, meta_strides=(H * NQ, NQ),
                        vbs=vbs)
    if i == 1:  # Jenga bitmap, one [64,64] mask shared by every head
        B, H, S, blk = 1, 16, 4096, 64
        NQ = S // blk
        q, k, v = (_randn(g, (B, H, S, D)) for _ in range(3))
        mask = (torch.rand((NQ, NQ), generator=g) < 0.5).to(torch.int8)
        mask.fill_diagonal_(1)
        return Workload(CONFIG_NAMES[1], B, H, S, D, blk, "bitmap", q, k, v,
                        mask=mask, mask_strides=(0, 0), vbs=None)
    if i == 2:  # video-shaped VSA: 96 of 768 blocks per q-block, sorted
        B, H, S, blk = 1, 24, 49152, 64
        NQ = S // blk
        q, k, v = (_randn(g, (B, H, S, D)) for _ in range(3))
        rows = B * H * NQ
        idx = _distinct_rows(g, rows, NQ, 96).sort(dim=-1).values.contiguous()
        num = torch.full((rows,), 96, dtype=torch.int32)
        vbs = torch.randint(16, 65, (NQ,), generator=g, dtype=torch.int32)
        return Workload(CONFIG_NAMES[2], B, H, S, D, blk, "lut", q, k, v,
                        q2k_idx=idx, q2k_num=num, meta_strides=(H * NQ, NQ),
                        vbs=vbs)
    if i == 3:  # 128-token blocks, counts uniform in [0, 64], -1 padding
        B, H, S, blk = 1, 40, 32768, 128
        NQ = S // blk
        q, k, v = (_randn(g, (B, H, S, D), std=0.5) for _ in range(3))
        rows = B * H * NQ
        num = torch.randint(0, 65, (rows,), generator=g, dtype=torch.int32)
        idx = _distinct_rows(g, rows, NQ, 64)
        pad = torch.arange(64, dtype=torch.int32)[None, :] >= num[:, None]
        idx = torch.where(pad, torch.full_like(idx, -1), idx).contiguous()
        vbs = torch.randint(32, 129, (NQ,), generator=g, dtype=torch.int32)
        assert int((num == 0).sum()) >= 1, "workload must contain count-0 rows"
        return Workload(CONFIG_NAMES[3], B, H, S, D, blk, "lut", q, k, v,
                        q2k_idx=idx, q2k_num=num, meta_strides=(H * NQ, NQ),
                        vbs=vbs)
    if i == 4:  # fp8 e4m3 K/V with per-64-token-block fp32 scales
        B, H, S, blk = 2, 12, 16384, 64
        NQ = S // blk
        q = _randn(g, (B, H, S, D))
        kf = torch.randn((B, H, S, D), generator=g, dtype=torch.float32)
        vf = torch.randn((B, H, S, D), generator=g, dtype=torch.float32)
        k, ks = quantize_fp8_per_block(kf, blk)
        v, vs = quantize_fp8_per_block(vf, blk)
        del kf, vf
        rows = B * H * NQ
        idx = _distinct_rows(g, rows, NQ, 64)
        num = torch.full((rows,), 64, dtype=torch.int32)
        return Workload(CONFIG_NAMES[4], B, H, S, D, blk, "lut", q, k, v,
                        k_scale=ks, v_scale=vs, q2k_idx=idx, q2k_num=num,
                        meta_strides=(H * NQ, NQ), vbs=None)
    raise ValueError(f"no workload {i}")


def make_random(seed: int, *, B=1, H=2, S=512, block=64, form="lut",
                density=0.5, max_kv=None, count_mode="fixed", vbs_mode="full",
                kv="bf16", std=1.0, shared_meta=False, pad_value=-1,
                sort=False, Hk=None, Sk=None) -> Workload:
    """Small random workloads for parity and invariance tests.

    count_mode: "fixed" (round(density*NK) per row), "uniform" (U{0..max_kv}),
    "zero" (every row 0).  vbs_mode: "full" (None), "random" (U{0..block}),
    "partial" (U{1..block}), "zero_some" (some blocks 0), "edges" (counts
    at and around multiples of 16, and 0), "tiny" (U{1..4}: runs of many
    short blocks).  kv: "bf16" or
    "fp8", or "i8cb" / "i4cb" (codebook-coded K/V with seeded bf16-exact
    codebooks).  Hk (key/value heads, default H) and Sk (key length, default
    S) give grouped-query and rectangular cases."""
    g = _gen(seed)
    D = HEAD_DIM
    Hk = H if Hk is None else Hk
    Sk = S if Sk is None else Sk
    NQ = S // block
    NK = Sk // block
    q = _randn(g, (B, H, S, D), std=std)
    kc = vc = None
    if kv == "bf16":
        k = _randn(g, (B, Hk, Sk, D), std=std)
        v = _randn(g, (B, Hk, Sk, D), std=std)
        ks = vs = None
    elif kv == "fp8":
        k, ks = quantize_fp8_per_block(
            torch.randn((B, Hk, Sk, D), generator=g) * std, block)
        v, vs = quantize_fp8_per_block(
            torch.randn((B, Hk, Sk, D), generator=g) * std, block)
    elif kv in ("i8cb", "i4cb"):
        bits = 8 if kv == "i8cb" else 4
        kc = make_codebook(g, 1 << bits)
        vc = make_codebook(g, 1 << bits)
        k, ks = quantize_codebook_per_block(
            torch.randn((B, Hk, Sk, D), generator=g) * std, block, kc, bits)
        v, vs = quantize_codebook_per_block(
            torch.randn((B, Hk, Sk, D), generator=g) * std, block, vc, bits)
    else:
        raise ValueError(kv)
    rows = NQ if shared_meta else B * H * NQ
    strides = (0, 0) if shared_meta else (H * NQ, NQ)
    if vbs_mode == "full":
        vbs = None
    elif vbs_mode == "random":
        vbs = torch.randint(0, block + 1, (NK,), generator=g, dtype=torch.int32)
    elif vbs_mode == "partial":
        vbs = torch.randint(1, block + 1, (NK,), generator=g, dtype=torch.int32)
    elif vbs_mode == "zero_some":
        vbs = torch.randint(0, block + 1, (NK,), generator=g, dtype=torch.int32)
        vbs[torch.rand((NK,), generator=g) < 0.3] = 0
    elif vbs_mode == "edges":
        vals = sorted({v for m in range(0, block + 1, 16) for v in (m - 1, m, m + 1)
                       if 0 <= v <= block} | {2, 3})
        pick = torch.randint(0, len(vals), (NK,), generator=g)
        vbs = torch.tensor(vals, dtype=torch.int32)[pick]
    elif vbs_mode == "tiny":
        vbs = torch.randint(1, 5, (NK,), generator=g, dtype=torch.int32)
    else:
        raise ValueError(vbs_mode)
    if form == "bitmap":
        mask = (torch.rand((rows, NK), generator=g) < density).to(torch.int8)
        return Workload(f"random_bitmap_{seed}", B, H, S, D, block, "bitmap",
                        q, k, v, k_scale=ks, v_scale=vs, mask=mask,
                        mask_strides=strides, vbs=vbs, k_codebook=kc,
                        v_codebook=vc)
    if max_kv is None:
        max_kv = NK
    take = min(max_kv, NK)
    idx = torch.full((rows, max_kv), pad_value, dtype=torch.int32)
    sel = _distinct_rows(g, rows, NK, take)
    if sort:
        sel = sel.sort(dim=-1).values
    idx[:, :take] = sel
    if count_mode == "fixed":
        n = max(0, min(take, round(density * NK)))
        num = torch.full((rows,), n, dtype=torch.int32)
    elif count_mode == "uniform":
        num = torch.randint(0, take + 1, (rows,), generator=g, dtype=torch.int32)
    elif count_mode == "zero":
        num = torch.zeros((rows,), dtype=torch.int32)
    else:
        raise ValueError(count_mode)
    padm = torch.arange(max_kv, dtype=torch.int32)[None, :] >= num[:, None]
    idx = torch.where(padm, torch.full_like(idx, pad_value), idx).contiguous()
    return Workload(f"random_lut_{seed}", B, H, S, D, block, "lut", q, k, v,
                    k_scale=ks, v_scale=vs, q2k_idx=idx, q2k_num=num,
                    meta_strides=strides, vbs=vbs, k_codebook=kc,
                    v_codebook=vc)
