"""Plain CPU oracle for the VecInfer product-VQ KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module: only the test suite, the smoke check of the entry script
and the CPU-baseline leg of the benchmark use it.  It shares no code with the
HIP library and imports nothing from the package.

Everything here is a direct, slow, fp64 statement of what the pages define:

* "veloxquant_mlx.cache.vecinfer_cache module" page, module description:
  keys get a per-(head, channel) smooth scaling and a Walsh-Hadamard
  rotation, are product-VQ encoded against a codebook and decoded again;
  the per-token storage formula (D / d_k) * b_k / 8 bytes.
* "Metal Kernels API" page, section "VecInfer kernels":
  vecinfer_quantize_metal (nearest centroid by squared distance per
  sub-vector), vecinfer_dequant_metal (codebook gather) and
  vecinfer_encode_decode_metal (smooth -> WHT -> VQ encode -> dequant ->
  inverse WHT -> inverse smooth).
* "Metal Kernels API" page, section "Fused SDPA", metal_fused_sdpa: attention
  over the codes equals standard SDPA over the dequantized keys; queries
  align to the tail of the key axis under the causal mask; a positive
  sliding_window keeps only the last keys before each query; the query's
  dual transform satisfies q_tilde . K_tilde^T == q . K_hat^T.
* "veloxquant_mlx.cache.vecinfer_cache module" page, fused_sdpa: the raw
  query is passed in and the dual transform is applied internally.

Readings of points the pages leave open (each is listed with its reason in
the design notes of the repository):
  R1  smoothing divides on encode (k / s) and multiplies on decode; the
      query multiplies (q * s).
  R2  the transform is the normalized Sylvester Hadamard matrix
      H[i, j] = (-1)^popcount(i & j) / sqrt(D), applied as a row vector
      times H; H is symmetric and its own inverse.  An explicit invertible
      [D, D] matrix M (the encode_decode kernel's H_mat argument) may be
      given instead: encode applies x . M, decode x~ . M^-1, and the query's
      dual transform is q . (M^-1)^T.
  R3  sub-vector j covers dims [j*d, (j+1)*d).
  R4  one codebook [n_centroids, d] is shared by all sub-vectors.
  R5  squared L2 distance; exact ties resolve to the lowest index.
  R7  causal: q_abs = len - S_q + i, key t valid iff t <= q_abs.
  R8  window W > 0: key t valid iff t > q_abs - W (W keys including the
      query's own slot); W = 0 disables it.
  R9  without causal the window is only a lower bound.
  R10 a query row with no valid key outputs zeros.
  R11 GQA: query head h reads kv head h // (H_q / H_kv).
  R12 the query uses the smooth row of its kv head.
  R24 4-bit codes pack two indices per byte, the even sub-vector in the low
      nibble (the pages' rabitq_pack_values layout).
  R25 codebooks are trained by Lloyd's k-means over the pooled sub-vectors
      (the keys' after smoothing and rotation, the values' raw): the pages
      only say the keys are encoded against a pre-trained codebook.  The
      initial centroids are an input; assignment follows R5; a centroid
      with no member keeps its value; a fixed number of iterations.

Every function computes in float64.  Precision notes for comparisons with
the GPU live with the tests.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# Walsh-Hadamard transform (reading R2)
# ----------------------------------------------------------------------------
def sylvester_hadamard(D: int) -> np.ndarray:
    """Normalized Sylvester Hadamard matrix of order D (D a power of two).

    Built by the Sylvester doubling H_2n = [[H_n, H_n], [H_n, -H_n]] from
    H_1 = [1], then scaled by 1/sqrt(D) so that it is orthonormal.  The
    cache page ("veloxquant_mlx.cache.vecinfer_cache module", module
    description) and the encode_decode kernel ("Metal Kernels API",
    "VecInfer kernels", vecinfer_encode_decode_metal, argument H_mat [D, D])
    name a Walsh-Hadamard rotation; this is the natural-order one.
    """
    if D < 1 or (D & (D - 1)) != 0:
        raise ValueError(f"Hadamard order must be a power of two, got {D}")
    h = np.ones((1, 1), dtype=F64)
    while h.shape[0] < D:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(F64(D))


def _smooth_rows(smooth, n_heads: int, D: int):
    """Return smooth factors as a float64 [n_heads, D] array, or None.

    The encode_decode kernel takes smooth as [H, D] or [D] ("Metal Kernels
    API", "VecInfer kernels", vecinfer_encode_decode_metal); None means no
    smoothing (identity).
    """
    if smooth is None:
        return None
    s = np.asarray(smooth, dtype=F64)
    if s.ndim == 1:
        if s.shape[0] != D:
            raise ValueError("smooth [D] has the wrong length")
        return np.broadcast_to(s, (n_heads, D))
    if s.shape != (n_heads, D):
        raise ValueError(f"smooth must be [{n_heads}, {D}] or [{D}], got {s.shape}")
    return s


def _rotation(transform, D: int):
    """(M, M^-1) of a transform argument: False/None -> no rotation; True ->
    the normalized Sylvester matrix, its own inverse (R2); a [D, D] array ->
    that matrix and its inverse (H_mat of vecinfer_encode_decode_metal,
    "Metal Kernels API", "VecInfer kernels")."""
    if isinstance(transform, np.ndarray):
        m = np.asarray(transform, dtype=F64)
        if m.shape != (D, D):
            raise ValueError(f"transform matrix must be [{D}, {D}], got {m.shape}")
        return m, np.linalg.inv(m)
    if not transform:
        return None, None
    h = sylvester_hadamard(D)
    return h, h


# ----------------------------------------------------------------------------
# Key transform and its inverse (readings R1, R2)
# ----------------------------------------------------------------------------
def forward_transform(x: np.ndarray, smooth=None, transform: bool = False) -> np.ndarray:
    """x [B, H, S, D] -> float64 transformed vectors (x / s) . H.

    Smooth first, then rotate: the order the encode_decode kernel lists
    ("Metal Kernels API", "VecInfer kernels": smooth -> Walsh-Hadamard
    transform -> VQ encode).
    """
    x = np.asarray(x).astype(F64)
    B, H, S, D = x.shape
    s = _smooth_rows(smooth, H, D)
    if s is not None:
        x = x / s[None, :, None, :]
    m, _ = _rotation(transform, D)
    if m is not None:
        x = x @ m
    return x


def inverse_transform(xt: np.ndarray, smooth=None, transform: bool = False) -> np.ndarray:
    """Undo forward_transform: (xt . M^-1) * s; for the Sylvester matrix
    M^-1 = H (symmetric and involutory).

    The last two steps of the encode_decode chain ("Metal Kernels API",
    "VecInfer kernels": dequant -> inverse-WHT -> inverse-smooth).
    """
    xt = np.asarray(xt, dtype=F64)
    B, H, S, D = xt.shape
    _, m_inv = _rotation(transform, D)
    if m_inv is not None:
        xt = xt @ m_inv
    s = _smooth_rows(smooth, H, D)
    if s is not None:
        xt = xt * s[None, :, None, :]
    return xt


# ----------------------------------------------------------------------------
# Product-VQ encode / decode (readings R3, R4, R5)
# ----------------------------------------------------------------------------
def pvq_encode(x: np.ndarray, codebook: np.ndarray, sub_dim: int,
               chunk_rows: int = 1 << 15):
    """Nearest-centroid product VQ of x [..., D].

    "Metal Kernels API", "VecInfer kernels", vecinfer_quantize_metal: x is
    split into D // sub_dim sub-vectors; each gets the index of the centroid
    at the smallest squared distance in the [n_centroids, sub_dim] codebook.

    Returns (codes int64 [..., n_sub], gap float64 [..., n_sub]) where
    gap = (d2 - d1) / d2 from the two smallest distances d1 <= d2 (0 when
    d2 == 0); it measures how close a decision is to a tie.
    """
    x = np.asarray(x, dtype=F64)
    C = np.asarray(codebook, dtype=F64)
    if C.ndim != 2 or C.shape[1] != sub_dim:
        raise ValueError("codebook must be [n_centroids, sub_dim]")
    D = x.shape[-1]
    if D % sub_dim != 0:
        raise ValueError("D must be divisible by sub_dim")
    n_sub = D // sub_dim
    lead = x.shape[:-1]
    rows = x.reshape(-1, sub_dim)
    n_c = C.shape[0]
    codes = np.empty(rows.shape[0], dtype=np.int64)
    gap = np.empty(rows.shape[0], dtype=F64)
    for lo in range(0, rows.shape[0], chunk_rows):
        r = rows[lo:lo + chunk_rows]
        diff = r[:, None, :] - C[None, :, :]          # [n, n_c, d]
        dist = np.sum(diff * diff, axis=-1)           # [n, n_c]
        # np.argmin returns the first minimum: exact ties -> lowest index.
        codes[lo:lo + chunk_rows] = np.argmin(dist, axis=-1)
        if n_c >= 2:
            two = np.partition(dist, 1, axis=-1)[:, :2]
            d1, d2 = two[:, 0], two[:, 1]
            with np.errstate(invalid="ignore", divide="ignore"):
                g = np.where(d2 > 0, (d2 - d1) / d2, 0.0)
        else:
            g = np.full(r.shape[0], np.inf)
        gap[lo:lo + chunk_rows] = g
    return codes.reshape(*lead, n_sub), gap.reshape(*lead, n_sub)


def pvq_distances(x: np.ndarray, codebook: np.ndarray, sub_dim: int) -> np.ndarray:
    """Squared distances [..., n_sub, n_centroids] for small inputs."""
    x = np.asarray(x, dtype=F64)
    C = np.asarray(codebook, dtype=F64)
    n_sub = x.shape[-1] // sub_dim
    r = x.reshape(*x.shape[:-1], n_sub, 1, sub_dim)
    diff = r - C
    return np.sum(diff * diff, axis=-1)


def pvq_decode(codes: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Codebook gather [..., n_sub] -> [..., n_sub * sub_dim].

    "Metal Kernels API", "VecInfer kernels", vecinfer_dequant_metal.
    """
    C = np.asarray(codebook, dtype=F64)
    codes = np.asarray(codes).astype(np.int64)
    g = C[codes]                                       # [..., n_sub, d]
    return g.reshape(*codes.shape[:-1], codes.shape[-1] * C.shape[1])


def encode(keys, codebook, sub_dim, smooth=None, transform=False):
    """keys [B, H, S, D] -> (codes [B, H, S, n_sub], gap).

    smooth -> WHT -> nearest centroid ("Metal Kernels API", "VecInfer
    kernels", vecinfer_encode_decode_metal, first three steps).
    """
    xt = forward_transform(keys, smooth, transform)
    return pvq_encode(xt, codebook, sub_dim)


def decode(codes, codebook, smooth=None, transform=False) -> np.ndarray:
    """codes [B, H, S, n_sub] -> float64 reconstruction [B, H, S, D].

    dequant -> inverse WHT -> inverse smooth (last three steps of
    vecinfer_encode_decode_metal, "Metal Kernels API", "VecInfer kernels").
    """
    xt = pvq_decode(codes, codebook)
    return inverse_transform(xt, smooth, transform)


def encode_decode(keys, codebook, sub_dim, smooth=None, transform=False):
    """Round trip: (recon float64 [B, H, S, D], codes, gap)."""
    codes, gap = encode(keys, codebook, sub_dim, smooth, transform)
    return decode(codes, codebook, smooth, transform), codes, gap


# ----------------------------------------------------------------------------
# Attention over codes (readings R7-R12)
# ----------------------------------------------------------------------------
def attention_mask(kv_len: int, S_q: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [S_q, kv_len] mask of the keys each query row may attend.

    "Metal Kernels API", "Fused SDPA", metal_fused_sdpa: causal queries align
    to the tail of the key axis; a positive sliding_window keeps only the
    last sliding_window keys before each query position.  The tail alignment
    q_abs = (S_kv - S_q) + q_pos with slot j masked when j > q_abs is stated
    on the same page for rabitq_prefill_attend, which shares the convention.
    """
    i = np.arange(S_q)[:, None]
    t = np.arange(kv_len)[None, :]
    q_abs = kv_len - S_q + i
    valid = np.ones((S_q, kv_len), dtype=bool)
    if causal:
        valid &= t <= q_abs
    if window > 0:
        valid &= t > q_abs - window
    return valid


def _softmax_rows(logits: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """Row softmax over the valid entries; rows with none valid -> zeros (R10)."""
    z = np.where(valid, logits, -np.inf)
    m = np.max(z, axis=-1, keepdims=True) if z.shape[-1] else np.full(z.shape[:-1] + (1,), -np.inf)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(valid, np.exp(z - m), 0.0)
    den = np.sum(e, axis=-1, keepdims=True)
    return np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)


def attend(q, k_codes, k_codebook, v_codes, v_codebook, *, scale, causal=True,
           sliding_window=0, smooth=None, transform=False, kv_lens=None,
           rows=None):
    """Definitional attention from codes.  Returns float64 [B, H_q, S_q, D].

    K_hat = decode(k_codes) with the inverse transform and smooth, V_hat is
    the value-codebook gather; the output is plain softmax(scale . q K_hat^T)
    V_hat over the valid keys.  This is what metal_fused_sdpa is stated to
    equal ("Metal Kernels API", "Fused SDPA": mathematically identical to
    standard SDPA on the dequantized keys), with the raw query of
    VecInferKVCache.fused_sdpa ("veloxquant_mlx.cache.vecinfer_cache module",
    fused_sdpa).

    q [B, H_q, S_q, D]; k_codes [B, H_kv, S_cap, n_sub_k]; v_codes
    [B, H_kv, S_cap, n_sub_v]; kv_lens [B] (None -> S_cap).  rows, if given,
    is an iterable of (b, h) pairs; other rows are left as NaN.
    """
    q = np.asarray(q)
    B, Hq, Sq, D = q.shape
    Hkv = k_codes.shape[1]
    S_cap = k_codes.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    lens = np.full(B, S_cap) if kv_lens is None else np.asarray(kv_lens)
    s_all = _smooth_rows(smooth, Hkv, D)
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(Hq)]
        out = np.zeros((B, Hq, Sq, D), dtype=F64)
    else:
        out = np.full((B, Hq, Sq, D), np.nan, dtype=F64)
    cache = {}
    for b, h in rows:
        g = h // G
        L = int(lens[b])
        key = (b, g)
        if key not in cache:
            kc = k_codes[b:b + 1, g:g + 1, :L]
            sm = None if s_all is None else s_all[g:g + 1]
            K = decode(kc, k_codebook, sm, transform)[0, 0]          # [L, D]
            V = pvq_decode(v_codes[b, g, :L], v_codebook)            # [L, D]
            cache = {key: (K, V)}
        K, V = cache[key]
        logits = scale * (q[b, h].astype(F64) @ K.T)                 # [Sq, L]
        p = _softmax_rows(logits, attention_mask(L, Sq, causal, sliding_window))
        out[b, h] = p @ V
    return out


def query_lut(q_row: np.ndarray, k_codebook, sub_dim: int, smooth_row=None,
              transform=False) -> np.ndarray:
    """Per-subspace query LUT of one query row: LUT[j, c] = <q_tilde_j, C_k[c]>.

    q_tilde = (q * s) . H is the dual transform ("Metal Kernels API",
    "Fused SDPA": q_tilde . K_tilde^T == q . K_hat^T; "Metal Kernels API",
    "VecInfer kernels": compute_query_lut is the query-codebook LUT
    precompute for asymmetric MIPS).
    """
    qt = np.asarray(q_row, dtype=F64)
    D = qt.shape[-1]
    if smooth_row is not None:
        qt = qt * np.asarray(smooth_row, dtype=F64)
    _, m_inv = _rotation(transform, D)
    if m_inv is not None:
        qt = qt @ m_inv.T
    C = np.asarray(k_codebook, dtype=F64)
    return qt.reshape(D // sub_dim, sub_dim) @ C.T                   # [n_sub, n_c]


def lut_scores(q_row, k_codes_rows, k_codebook, sub_dim, smooth_row=None,
               transform=False) -> np.ndarray:
    """Scores q . K_hat_t^T of one query row by LUT gathers: sum_j LUT[j, code_tj]."""
    lut = query_lut(q_row, k_codebook, sub_dim, smooth_row, transform)
    codes = np.asarray(k_codes_rows).astype(np.int64)                # [L, n_sub]
    j = np.arange(codes.shape[1])[None, :]
    return np.sum(lut[j, codes], axis=1)


# ----------------------------------------------------------------------------
# Sub-byte codes: two 4-bit indices per byte
# ----------------------------------------------------------------------------
def pack_nibbles(codes) -> np.ndarray:
    """[..., n] indices (n even) -> [..., n / 2] uint8, two per byte.

    "Metal Kernels API" page, rabitq_pack_values: 4-bit indices are packed
    two per byte along the last axis, the even element in the low nibble,
    each value masked to 4 bits.  Used here for product-VQ codes of
    codebooks with at most 16 centroids (b = 4 in the storage formula).
    """
    c = np.asarray(codes).astype(np.int64)
    if c.shape[-1] % 2:
        raise ValueError("the last axis must have even length")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    """Inverse of pack_nibbles: [..., m] uint8 -> [..., 2 m] indices (int64)."""
    b = np.asarray(packed).astype(np.int64)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


# ----------------------------------------------------------------------------
# Storage accounting
# ----------------------------------------------------------------------------
def code_bytes_per_token(D: int, sub_dim: int, bits: int) -> float:
    """(D / d) * b / 8 bytes per token and head.

    The per-token key storage formula on the "veloxquant_mlx.cache.
    vecinfer_cache module" page (module description).
    """
    return (D / sub_dim) * bits / 8


def codebook_bytes(bits: int, sub_dim: int, bytes_per_entry: int) -> int:
    """2**b * d entries of bytes_per_entry bytes (amortized codebook cost,
    same page and formula; the page counts fp16 entries, the library stores
    fp32 codebooks)."""
    return (2 ** bits) * sub_dim * bytes_per_entry


# ----------------------------------------------------------------------------
# Codebook training (reading R25)
# ----------------------------------------------------------------------------
def lloyd_step(vectors, centroids):
    """One iteration of Lloyd's algorithm (k-means) on vectors [N, d].

    The codebooks the "veloxquant_mlx.cache.vecinfer_cache module" page
    encodes against come pre-trained; this is the plain k-means reading of
    that training (R25).  Assignment: every vector takes the index of its
    nearest centroid by squared distance, lowest index on exact ties (R5).
    Update: every centroid becomes the mean of the vectors assigned to it;
    one with no member keeps its value.

    Returns (new centroids float64 [k, d], labels int64 [N], inertia = the
    sum over vectors of the smallest squared distance to the centroids
    passed in, gap float64 [N] as in pvq_encode).
    """
    x = np.asarray(vectors, dtype=F64)
    C = np.asarray(centroids, dtype=F64)
    if x.ndim != 2 or C.ndim != 2 or x.shape[1] != C.shape[1]:
        raise ValueError("vectors [N, d] and centroids [k, d] expected")
    k, d = C.shape
    labels, gap = pvq_encode(x, C, d)
    labels, gap = labels[:, 0], gap[:, 0]
    diff = x - C[labels]
    inertia = float(np.sum(diff * diff))
    sums = np.zeros((k, d), dtype=F64)
    np.add.at(sums, labels, x)
    counts = np.bincount(labels, minlength=k)
    new = C.copy()
    has = counts > 0
    new[has] = sums[has] / counts[has, None]
    return new, labels, inertia, gap


def kmeans(vectors, init, iters: int):
    """`iters` Lloyd steps from the centroids `init` [k, d].

    Returns (centroids after the last update, labels of the last assignment,
    inertia of every step (list), gap of the last assignment).
    """
    C = np.asarray(init, dtype=F64)
    labels = np.zeros(np.asarray(vectors).shape[0], dtype=np.int64)
    gap = np.full(labels.shape, np.inf)
    inertia = []
    for _ in range(iters):
        C, labels, e, gap = lloyd_step(vectors, C)
        inertia.append(e)
    return C, labels, inertia, gap


def training_vectors(x, sub_dim: int, smooth=None, transform=False) -> np.ndarray:
    """The pooled sub-vectors [B * H * S * D / d, d] a codebook is trained
    on: forward_transform of x [B, H, S, D] split as in R3."""
    return forward_transform(x, smooth, transform).reshape(-1, sub_dim)
