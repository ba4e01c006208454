"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and selects rows: it holds none of the
method's arithmetic (no smoothing, rotation, nearest-centroid search, LUT or
softmax).  The only derived quantity is the smooth-factor calibration recipe
s[h, c] = sqrt(max |k|) over the keys of a head, which is an input to the
method, not a step of it.  Codebooks that are "drawn from samples of the
transformed vectors" are built by the caller: it passes the transformed
vectors in and `sample_rows` picks rows from them.

Workloads (sizes as stated for the five workloads of the method):
  tiny        B=1, H=2, S=256, S_q=1, D=64, d_k = d_v = 4, 2 outlier channels
  encode      keys [1, 8, 8192, 128], d_k = 8, 4 outlier channels
  decode      B=1, H=8, S_q=1, D=128, S_kv in {512, 2048, 8192}, random codes
  gqa_long    B=16, H_q=32, H_kv=8, S_cap=32768, ragged lengths in
              [16384, 32768], random codes
  prefill     B=4, H=8, D=128, 512 new tokens appended after 16384 prior
              tokens (random codes) in a 32768-slot buffer, S_q=512 causal
"""
from __future__ import annotations

import math

import numpy as np

SEEDS = {"tiny": 101, "encode": 102, "decode": 103, "gqa_long": 104, "prefill": 105}
N_CENTROIDS = 256
OUTLIER_FACTOR = 20.0


def outlier_normal(rng: np.random.Generator, shape, n_outliers: int,
                   factor: float = OUTLIER_FACTOR) -> np.ndarray:
    """fp16 [B, H, S, D]: N(0, 1) in fp32, `factor` times larger on
    `n_outliers` channels per head (channels drawn per head without
    replacement), then rounded to fp16 (round to nearest even)."""
    B, H, S, D = shape
    x = rng.standard_normal(shape, dtype=np.float32)
    for h in range(H):
        ch = rng.choice(D, size=n_outliers, replace=False)
        x[:, h, :, ch] *= np.float32(factor)
    return x.astype(np.float16)


def smooth_factors(keys: np.ndarray, floor: float = 1e-6) -> np.ndarray:
    """fp32 [H, D] calibration recipe: sqrt(max over batch and tokens of |k|)."""
    k = np.abs(keys.astype(np.float32))
    m = k.max(axis=(0, 2))
    return np.sqrt(np.maximum(m, np.float32(floor))).astype(np.float32)


def sample_rows(rng: np.random.Generator, vectors: np.ndarray, n: int) -> np.ndarray:
    """fp32 [n, d]: n rows of `vectors` [N, d] drawn without replacement."""
    idx = rng.choice(vectors.shape[0], size=n, replace=False)
    return np.ascontiguousarray(vectors[idx]).astype(np.float32)


def normal_codebook(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    return rng.standard_normal((n, d), dtype=np.float32)


def uniform_codes(rng: np.random.Generator, shape, n_centroids: int = N_CENTROIDS) -> np.ndarray:
    return rng.integers(0, n_centroids, size=shape, dtype=np.uint8)


def normal_fp16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def ragged_lengths(rng: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    """int32 [B] uniform in [lo, hi] inclusive."""
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def _codebook(rng, transformed, sub_dim, n=N_CENTROIDS):
    """Rows sampled from transformed sub-vectors when the caller supplies
    them, else N(0, 1) rows (the work of every kernel is independent of the
    codebook's values, so timing runs may use the latter)."""
    if transformed is None:
        return normal_codebook(rng, n, sub_dim)
    return sample_rows(rng, np.asarray(transformed).reshape(-1, sub_dim), n)


def tiny(transform_fn=None):
    """Tiny encode + decode-attend workload.

    transform_fn(keys, smooth) -> transformed keys (float array
    [B, H, S, D]); when given, the key codebook is sampled from its
    sub-vectors and the value codebook from the raw value sub-vectors.
    """
    rng = np.random.default_rng(SEEDS["tiny"])
    B, H, S, D, dk, dv = 1, 2, 256, 64, 4, 4
    k = outlier_normal(rng, (B, H, S, D), 2)
    v = outlier_normal(rng, (B, H, S, D), 2)
    q = outlier_normal(rng, (B, H, 1, D), 2)
    s = smooth_factors(k)
    kt = transform_fn(k, s) if transform_fn is not None else None
    ck = _codebook(rng, kt, dk)
    cv = _codebook(rng, v.astype(np.float32) if transform_fn is not None else None, dv)
    return dict(name="tiny", B=B, H=H, H_kv=H, S=S, S_q=1, D=D, dk=dk, dv=dv,
                keys=k, values=v, q=q, smooth=s, k_codebook=ck, v_codebook=cv,
                scale=1.0 / math.sqrt(D), causal=True, window=0)


def encode(transform_fn=None):
    """Key-encode throughput workload: keys [1, 8, 8192, 128], d_k = 8."""
    rng = np.random.default_rng(SEEDS["encode"])
    B, H, S, D, dk = 1, 8, 8192, 128, 8
    k = outlier_normal(rng, (B, H, S, D), 4)
    s = smooth_factors(k)
    kt = transform_fn(k, s) if transform_fn is not None else None
    ck = _codebook(rng, kt, dk)
    return dict(name="encode", B=B, H=H, S=S, D=D, dk=dk, keys=k, smooth=s, k_codebook=ck)


def decode(S_kv: int):
    """Single-query decode over random codes: B=1, H=8, D=128, d_k=8, d_v=4."""
    rng = np.random.default_rng(SEEDS["decode"] * 100003 + S_kv)
    B, H, D, dk, dv = 1, 8, 128, 8, 4
    # smooth factors follow the encode workload's recipe (same H and D)
    k_ref = outlier_normal(rng, (1, H, 8192, D), 4)
    s = smooth_factors(k_ref)
    return dict(name=f"decode_S{S_kv}", B=B, H_q=H, H_kv=H, S_q=1, D=D, dk=dk, dv=dv,
                S_cap=S_kv, kv_lens=None,
                q=normal_fp16(rng, (B, H, 1, D)),
                k_codes=uniform_codes(rng, (B, H, S_kv, D // dk)),
                v_codes=uniform_codes(rng, (B, H, S_kv, D // dv)),
                k_codebook=normal_codebook(rng, N_CENTROIDS, dk),
                v_codebook=normal_codebook(rng, N_CENTROIDS, dv),
                smooth=s, scale=1.0 / math.sqrt(D), causal=True, window=0)


def gqa_long(window: int = 0, k_codebook=None, smooth=None, B: int = 16, code_bits: int = 8):
    """Batched long-context GQA decode: H_q=32, H_kv=8, S_cap=32768, ragged.

    The key codebook and smooth factors are those of the encode workload
    when passed in; otherwise N(0, 1) rows and the encode recipe's smooth
    factors drawn here.  code_bits=4 draws 16-centroid codebooks and code
    rows of half the bytes: uniform random bytes, i.e. two independent
    uniform 4-bit codes per byte.
    """
    rng = np.random.default_rng(SEEDS["gqa_long"] + (0 if code_bits == 8 else 1000))
    Hq, Hkv, D, dk, dv, S_cap = 32, 8, 128, 8, 4, 32768
    n_c = N_CENTROIDS if code_bits == 8 else 16
    lens = ragged_lengths(rng, 16, 16384, 32768)[:B]
    if smooth is None:
        smooth = smooth_factors(outlier_normal(rng, (1, Hkv, 8192, D), 4))
    if k_codebook is None:
        k_codebook = normal_codebook(rng, n_c, dk)
    rb = lambda n_sub: n_sub * code_bits // 8
    return dict(name=f"gqa_long_W{window}" + ("" if code_bits == 8 else "_4bit"), B=B, H_q=Hq,
                H_kv=Hkv, S_q=1, D=D, dk=dk, dv=dv, S_cap=S_cap, kv_lens=lens, code_bits=code_bits,
                q=normal_fp16(rng, (B, Hq, 1, D)),
                k_codes=uniform_codes(rng, (B, Hkv, S_cap, rb(D // dk))),
                v_codes=uniform_codes(rng, (B, Hkv, S_cap, rb(D // dv))),
                k_codebook=np.asarray(k_codebook, dtype=np.float32),
                v_codebook=normal_codebook(rng, n_c, dv),
                smooth=np.asarray(smooth, dtype=np.float32),
                scale=1.0 / math.sqrt(D), causal=True, window=window)


def prefill(transform_fn=None):
    """Prefill chunk with cache append: B=4, H=8, D=128, 512 new tokens after
    16384 prior tokens of random codes in a 32768-slot buffer."""
    rng = np.random.default_rng(SEEDS["prefill"])
    B, H, D, dk, dv = 4, 8, 128, 8, 4
    S_new, S_prior, S_cap = 512, 16384, 32768
    k = outlier_normal(rng, (B, H, S_new, D), 4)
    v = outlier_normal(rng, (B, H, S_new, D), 4)
    q = outlier_normal(rng, (B, H, S_new, D), 4)
    s = smooth_factors(k)
    kt = transform_fn(k, s) if transform_fn is not None else None
    ck = _codebook(rng, kt, dk)
    cv = _codebook(rng, v.astype(np.float32) if transform_fn is not None else None, dv)
    k_codes = np.zeros((B, H, S_cap, D // dk), dtype=np.uint8)
    v_codes = np.zeros((B, H, S_cap, D // dv), dtype=np.uint8)
    k_codes[:, :, :S_prior] = uniform_codes(rng, (B, H, S_prior, D // dk))
    v_codes[:, :, :S_prior] = uniform_codes(rng, (B, H, S_prior, D // dv))
    return dict(name="prefill", B=B, H_q=H, H_kv=H, S_q=S_new, D=D, dk=dk, dv=dv,
                S_cap=S_cap, S_off=S_prior, kv_lens=np.full(B, S_prior + S_new, dtype=np.int32),
                keys=k, values=v, q=q, smooth=s, k_codebook=ck, v_codebook=cv,
                k_codes=k_codes, v_codes=v_codes,
                scale=1.0 / math.sqrt(D), causal=True, window=0)
