"""Seeded synthetic inputs for the Evoformer biased-attention forward pass.

This module only draws and rounds numbers: it holds none of the attention
arithmetic, and both the HIP path's tests and the oracle's tests take their
inputs from it.  Values are drawn in float32 with numpy's PCG64 generators and
rounded to the storage type with round-to-nearest-even; bf16 and f16 are
returned as uint16 bit patterns, f32 as float32.

The workloads follow the four attention variants of the page "DeepSpeed
DS4Sci_EvoformerAttention 内核实战指南" (hmyw.cn), section 5.3: MSA row
attention (mask + pair bias), MSA column attention (mask only) and triangle
attention around the starting / ending node (mask + pair bias projected from a
pair tensor).  Masks are additive: 0 for kept keys and -1e9 for removed ones
(section 5.2 of the same page).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MASK_NEG = -1.0e9


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> stored representation of `dtype` ("f32", "bf16", "f16")."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        with np.errstate(over="ignore"):  # -1e9 and other large values become -inf / inf
            return np.ascontiguousarray(x.astype(np.float16).view(np.uint16))
    raise ValueError(dtype)


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored representation -> float32 (exact for every supported dtype)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype == "f16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float32)
    raise ValueError(dtype)


@dataclass
class Workload:
    """One seeded problem: stored inputs plus a description."""
    name: str
    dtype: str
    shape: tuple  # (B, N, L, H, D)
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    mask: Optional[np.ndarray]
    pair: Optional[np.ndarray]
    meta: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        B, N, L, H, D = self.shape
        return 4 * B * N * H * L * L * D


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def random_problem(B, N, L, H, D, dtype="bf16", seed=0, mask="tail", pair="normal",
                   mask_frac=0.1, qkv_scale=1.0, bias_scale=1.0) -> Workload:
    """A generic seeded problem of any shape.

    mask: None | "tail" (per-sequence random tail of up to mask_frac*L keys set
          to -1e9) | "random" (each key removed with probability mask_frac) |
          "normal" (N(0, bias_scale^2) values, no removal) | "zero".
    pair: None | "normal" (N(0, bias_scale^2)) | "zero" | "int8" (k / 32 for
          uniform int8 k: exact in every storage format and cheap to draw for
          pair matrices of ~10^9 elements, filled in bands of rows).
    """
    ss = np.random.SeedSequence(seed)
    rq, rk, rv, rm, rp = [np.random.default_rng(s) for s in ss.spawn(5)]
    q = to_storage(qkv_scale * _normal(rq, (B, N, L, H, D)), dtype)
    k = to_storage(qkv_scale * _normal(rk, (B, N, L, H, D)), dtype)
    v = to_storage(_normal(rv, (B, N, L, H, D)), dtype)
    m = None
    if mask is not None:
        mf = np.zeros((B, N, 1, 1, L), np.float32)
        if mask == "tail":
            tmax = int(np.floor(mask_frac * L))
            t = rm.integers(0, tmax + 1, size=(B, N))
            for b in range(B):
                for n in range(N):
                    if t[b, n]:
                        mf[b, n, 0, 0, L - t[b, n]:] = MASK_NEG
        elif mask == "random":
            mf[rm.random((B, N, 1, 1, L)) < mask_frac] = MASK_NEG
        elif mask == "normal":
            mf = bias_scale * _normal(rm, (B, N, 1, 1, L))
        elif mask != "zero":
            raise ValueError(mask)
        m = to_storage(mf, dtype)
    p = None
    if pair is not None:
        if pair == "normal":
            p = to_storage(bias_scale * _normal(rp, (B, 1, H, L, L)), dtype)
        elif pair == "zero":
            p = to_storage(np.zeros((B, 1, H, L, L), np.float32), dtype)
        elif pair == "int8":
            p = np.empty((B, 1, H, L, L), np.float32 if dtype == "f32" else np.uint16)
            band = 2048
            for b in range(B):
                for h in range(H):
                    for r0 in range(0, L, band):
                        r1 = min(L, r0 + band)
                        k8 = rp.integers(-128, 128, size=(r1 - r0, L), dtype=np.int8)
                        p[b, 0, h, r0:r1] = to_storage(k8.astype(np.float32) / 32, dtype)
        else:
            raise ValueError(pair)
    return Workload(f"random_{B}x{N}x{L}x{H}x{D}_{dtype}", dtype, (B, N, L, H, D), q, k, v, m, p,
                    {"seed": seed, "mask": mask, "pair": pair})


def random_dout(shape, dtype="bf16", seed=0, scale=1.0) -> np.ndarray:
    """Seeded incoming gradient dO for the backward pass: N(0, scale^2) in the
    storage format, shaped like the output [B, N, L, H, D]."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x0D0]))
    return to_storage(scale * _normal(rng, tuple(shape)), dtype)


def trimul_problem(B, C, L, dtype="bf16", seed=0, scale=1.0):
    """Seeded operands of the triangle multiplication: a, w ~ N(0, scale^2), [B, C, L, L] in the storage format.
    The named size is TRIMUL_WORKLOAD (a pair representation of 384 residues with 128 channels)."""
    ra, rw = [np.random.default_rng(s) for s in np.random.SeedSequence([seed, 0x7A1]).spawn(2)]
    return (to_storage(scale * _normal(ra, (B, C, L, L)), dtype), to_storage(scale * _normal(rw, (B, C, L, L)), dtype))


TRIMUL_WORKLOAD = dict(name="trimul_bf16_384x128", B=1, C=128, L=384, dtype="bf16")


# ---------------------------------------------------------------------------
# The five named workloads.  Each draws from SeedSequence(1000 + c) spawned
# into six streams used in a fixed order: q, k, v, mask, pair tensor z, W.
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: dict(name="msa_row_f32_tiny", variant="msa_row", B=1, N=16, L=64, H=8, D=32, dtype="f32"),
    2: dict(name="msa_row_bf16", variant="msa_row", B=1, N=128, L=256, H=8, D=32, dtype="bf16"),
    3: dict(name="msa_col_bf16", variant="msa_col", B=1, N=256, L=1024, H=8, D=32, dtype="bf16"),
    4: dict(name="tri_start_bf16_384", variant="tri_start", B=1, N=384, L=384, H=4, D=32, dtype="bf16"),
    5: dict(name="tri_end_bf16_768", variant="tri_end", B=1, N=768, L=768, H=4, D=32, dtype="bf16"),
}


def _projected_pair(rz, rw, L, H, transpose):
    """pair[h,i,j] = sum_c z[i,j,c] W[c,h] (z[j,i,c] for the ending node), in float64.

    z ~ N(0,1) [L,L,128] and W ~ N(0, 1/128) [128,H]: a stand-in for the
    caller's linear projection of the pair representation to per-head biases.
    """
    C = 128
    z = _normal(rz, (L, L, C))
    w = _normal(rw, (C, H)) / np.float32(np.sqrt(C))
    proj = z.reshape(L * L, C).astype(np.float64) @ w.astype(np.float64)  # [(i j), h]
    proj = proj.reshape(L, L, H).transpose(2, 0, 1)  # [h, i, j] = sum_c z[i,j,c] w[c,h]
    if transpose:
        proj = proj.transpose(0, 2, 1)  # [h, i, j] = sum_c z[j,i,c] w[c,h]
    return np.ascontiguousarray(proj.astype(np.float32))[None, None]  # [1,1,H,L,L]


def workload(c: int, dtype: str | None = None) -> Workload:
    """Inputs of named workload c (1..5); `dtype` stores the same drawn values
    in another format ("f32", "bf16", "f16") instead of the workload's own."""
    w = WORKLOADS[c]
    B, N, L, H, D, dt = w["B"], w["N"], w["L"], w["H"], w["D"], w["dtype"]
    name = w["name"]
    if dtype is not None and dtype != dt:
        name = name.replace(dt, dtype) if dt in name else f"{name}_{dtype}"
        dt = dtype
    ss = np.random.SeedSequence(1000 + c)
    rq, rk, rv, rmask, rz, rw = [np.random.default_rng(s) for s in ss.spawn(6)]
    q = to_storage(_normal(rq, (B, N, L, H, D)), dt)
    k = to_storage(_normal(rk, (B, N, L, H, D)), dt)
    v = to_storage(_normal(rv, (B, N, L, H, D)), dt)
    meta = {"variant": w["variant"], "seed": 1000 + c}
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    if c == 1:
        mf[..., 56:] = MASK_NEG                      # last 8 residues of every sequence
        pair = _normal(rz, (B, 1, H, L, L))
    elif c == 2:
        t = rmask.integers(0, int(np.floor(0.1 * L)) + 1, size=N)  # tail of 0..25 keys
        for n in range(N):
            if t[n]:
                mf[0, n, 0, 0, L - t[n]:] = MASK_NEG
        meta["tails"] = t
        pair = _normal(rz, (B, 1, H, L, L))
    elif c == 3:
        cols = rmask.choice(L, size=int(round(0.05 * L)), replace=False)  # 51 missing sequences
        mf[..., cols] = MASK_NEG
        meta["masked_keys"] = np.sort(cols)
        pair = None
    elif c == 4:
        mf[..., L - 16:] = MASK_NEG                  # last 16 residues
        pair = _projected_pair(rz, rw, L, H, transpose=False)
    elif c == 5:
        mf = None                                    # no masking
        pair = _projected_pair(rz, rw, L, H, transpose=True)
    else:
        raise ValueError(c)
    mask = None if mf is None else to_storage(mf, dt)
    pair = None if pair is None else to_storage(pair, dt)
    return Workload(name, dt, (B, N, L, H, D), q, k, v, mask, pair, meta)


def sample_rows(shape, count: int, seed: int = 7) -> np.ndarray:
    """`count` distinct seeded (b, n, h, i) row indices, always including the corners."""
    B, N, L, H, D = shape
    total = B * N * H * L
    rng = np.random.default_rng(seed)
    flat = rng.choice(total, size=min(count, total), replace=False)
    flat = np.unique(np.concatenate([flat, [0, total - 1]]))
    i = flat % L
    h = (flat // L) % H
    n = (flat // (L * H)) % N
    b = flat // (L * H * N)
    return np.stack([b, n, h, i], axis=1).astype(np.int64)
