"""Python binding of libvq: same names as the C ABI, torch tensors in and out.

Argument marshalling only: shapes are read off the tensors and checked
against each other (the C ABI receives bare pointers and sizes, so a buffer of
the wrong shape would otherwise be read or written out of bounds), device
pointers and the current HIP stream are passed to the C functions, and a
nonzero status becomes a VQError.  Every step of the computation runs in the
HIP kernels of libvq.so; there is no other implementation behind these calls.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

VQ_OK, VQ_ERR_INVALID_ARGUMENT, VQ_ERR_UNSUPPORTED, VQ_ERR_NO_DEVICE, VQ_ERR_HIP, VQ_ERR_WORKSPACE = range(6)


class VQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status
        self.message = message


def _call(name, *args, prepare=False, result=None):
    """Call the C function now, or (prepare=True) return a zero-argument
    callable that makes the same call with the already-marshalled arguments
    (for launch loops: the tensors must stay alive and unchanged in shape)."""
    lib = _lib.load()
    fn = getattr(lib, name)

    def run():
        st = fn(*args)
        if st != VQ_OK:
            raise VQError(st, lib.vq_last_error().decode() or lib.vq_status_string(st).decode())
        return result

    return run if prepare else run()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(t, name, dtype, ndim=None, shape=None):
    """dtype (one or a tuple), rank, exact shape (None entries are free) and
    contiguity.  The device is checked afterwards by _on_device, so a wrong
    shape is reported as such on any host."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        ndim = len(shape)
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if shape is not None and any(w is not None and g != w for g, w in zip(t.shape, shape)):
        want = tuple("*" if w is None else w for w in shape)
        raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    """Every tensor given (None entries skipped) lives on one and the same GPU."""
    devs = set()
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")


def _smooth(smooth, D, n_heads):
    """(tensor, rows) of the smooth factors: None, [D] (one row shared by
    every head) or [1 or n_heads, D]."""
    if smooth is None:
        return None, 1
    if smooth.dtype != torch.float32 or not smooth.is_contiguous():
        raise ValueError("smooth must be a contiguous fp32 tensor")
    if smooth.dim() == 1 and smooth.shape[0] == D:
        return smooth, 1
    if smooth.dim() == 2 and smooth.shape[1] == D and smooth.shape[0] in (1, n_heads):
        return smooth, smooth.shape[0]
    raise ValueError(f"smooth must be [{D}] or [1 or {n_heads}, {D}], got {tuple(smooth.shape)}")


def _offsets(row_offsets, B):
    """Host int32 array of the per-row write offsets (None: use S_off)."""
    if row_offsets is None:
        return None
    offs = [int(x) for x in row_offsets]
    if len(offs) != B:
        raise ValueError(f"row_offsets must hold B = {B} entries, got {len(offs)}")
    return (ctypes.c_int32 * B)(*offs)


def _n_sub(D, sub_dim, name="sub_dim"):
    if sub_dim <= 0 or D % sub_dim:
        raise ValueError(f"{name} {sub_dim} does not divide the head dim {D}")
    return D // sub_dim


def _row_bytes(n_sub, code_bits):
    """Bytes of one token's code row: one code per byte, or two (4-bit)."""
    if code_bits == 8:
        return n_sub
    if code_bits == 4:
        if n_sub % 2:
            raise ValueError("4-bit codes need an even number of sub-vectors")
        return n_sub // 2
    raise ValueError(f"code_bits must be 8 or 4, got {code_bits}")


def _transform(transform, mat, mat_inv, D):
    """(code, mat, mat_inv): transform False/0 -> none, True/1 -> the
    normalized Sylvester Walsh-Hadamard matrix, 2 (or any matrix given) ->
    the explicit [D, D] fp32 matrices mat = M and mat_inv = M^-1."""
    if mat is None and mat_inv is None:
        if transform == 2:
            raise ValueError("transform 2 needs mat and/or mat_inv")
        return int(bool(transform)), None, None
    for name, m in (("mat", mat), ("mat_inv", mat_inv)):
        if m is not None:
            _need(m, name, torch.float32, shape=(D, D))
    return 2, mat, mat_inv


def vq_supports_shape(n_centroids: int, n_sub: int, head_dim: int) -> bool:
    return bool(_lib.load().vq_supports_shape(n_centroids, n_sub, head_dim))


def vq_encode(keys, codebook, sub_dim, *, smooth=None, transform=True, codes=None,
              S_cap=None, S_off=0, row_offsets=None, code_bits=8, mat=None, mat_inv=None,
              stream=None, prepare=False):
    """Encode fp16 keys [B, H, S, D] into uint8 codes [B, H, S_cap, row_bytes]
    (row_bytes = D // sub_dim, or half that with code_bits=4: two codes per
    byte, the even sub-vector in the low nibble).

    Codes of token t of row b land in slot off_b + t (off_b = row_offsets[b]
    or S_off).  Returns the code tensor (allocated when `codes` is None)."""
    _need(keys, "keys", torch.float16, 4)
    B, H, S, D = keys.shape
    nb = _row_bytes(_n_sub(D, sub_dim), code_bits)
    _need(codebook, "codebook", torch.float32, shape=(None, sub_dim))
    if codes is None:
        codes = torch.zeros((B, H, S_cap or S, nb), dtype=torch.uint8, device=keys.device)
    _need(codes, "codes", torch.uint8, shape=(B, H, S_cap, nb))
    sm, rows = _smooth(smooth, D, H)
    offs = _offsets(row_offsets, B)
    tr, m, mi = _transform(transform, mat, mat_inv, D)
    _on_device(keys=keys, codebook=codebook, codes=codes, smooth=sm, mat=m, mat_inv=mi)
    return _call("vq_encode", _ptr(keys), B, H, S, D, _ptr(codebook), codebook.shape[0], sub_dim,
                 code_bits, _ptr(sm), rows, tr, _ptr(m), _ptr(mi), _ptr(codes), codes.shape[2], S_off, offs,
                 _stream(stream), prepare=prepare, result=codes)


def vq_encode_kv(keys, values, k_codebook, k_sub_dim, v_codebook, v_sub_dim, *, smooth=None,
                 transform=True, k_codes=None, v_codes=None, S_cap=None, S_off=0,
                 row_offsets=None, code_bits=8, mat=None, mat_inv=None, stream=None,
                 prepare=False):
    """Encode the keys (smoothed, rotated) and the values (neither) of one
    append into their code buffers; returns (k_codes, v_codes)."""
    _need(keys, "keys", torch.float16, 4)
    B, H, S, D = keys.shape
    _need(values, "values", torch.float16, shape=(B, H, S, D))
    nk = _row_bytes(_n_sub(D, k_sub_dim, "k_sub_dim"), code_bits)
    nv = _row_bytes(_n_sub(D, v_sub_dim, "v_sub_dim"), code_bits)
    _need(k_codebook, "k_codebook", torch.float32, shape=(None, k_sub_dim))
    _need(v_codebook, "v_codebook", torch.float32, shape=(None, v_sub_dim))
    if k_codes is None:
        k_codes = torch.zeros((B, H, S_cap or S, nk), dtype=torch.uint8, device=keys.device)
    if v_codes is None:
        v_codes = torch.zeros((B, H, S_cap or S, nv), dtype=torch.uint8, device=keys.device)
    _need(k_codes, "k_codes", torch.uint8, shape=(B, H, S_cap, nk))
    _need(v_codes, "v_codes", torch.uint8, shape=(B, H, k_codes.shape[2], nv))
    sm, rows = _smooth(smooth, D, H)
    offs = _offsets(row_offsets, B)
    tr, m, mi = _transform(transform, mat, mat_inv, D)
    _on_device(keys=keys, values=values, k_codebook=k_codebook, v_codebook=v_codebook,
               k_codes=k_codes, v_codes=v_codes, smooth=sm, mat=m, mat_inv=mi)
    return _call("vq_encode_kv", _ptr(keys), _ptr(values), B, H, S, D, _ptr(k_codebook),
                 k_codebook.shape[0], k_sub_dim, _ptr(sm), rows, tr, _ptr(m), _ptr(mi),
                 _ptr(v_codebook), v_codebook.shape[0], v_sub_dim, code_bits, _ptr(k_codes), _ptr(v_codes),
                 k_codes.shape[2], S_off, offs, _stream(stream), prepare=prepare,
                 result=(k_codes, v_codes))


def vq_encode_decode(keys, codebook, sub_dim, *, smooth=None, transform=True, codes=None,
                     S_cap=None, S_off=0, row_offsets=None, recon=None,
                     out_dtype=torch.float16, code_bits=8, mat=None, mat_inv=None, stream=None,
                     prepare=False):
    """Fused encode + reconstruction.  Returns (recon [B, H, S, D], codes)."""
    _need(keys, "keys", torch.float16, 4)
    B, H, S, D = keys.shape
    nb = _row_bytes(_n_sub(D, sub_dim), code_bits)
    _need(codebook, "codebook", torch.float32, shape=(None, sub_dim))
    if codes is None:
        codes = torch.zeros((B, H, S_cap or S, nb), dtype=torch.uint8, device=keys.device)
    _need(codes, "codes", torch.uint8, shape=(B, H, S_cap, nb))
    if recon is None:
        recon = torch.empty((B, H, S, D), dtype=out_dtype, device=keys.device)
    _need(recon, "recon", (torch.float32, torch.float16), shape=(B, H, S, D))
    sm, rows = _smooth(smooth, D, H)
    offs = _offsets(row_offsets, B)
    tr, m, mi = _transform(transform, mat, mat_inv, D)
    _on_device(keys=keys, codebook=codebook, codes=codes, recon=recon, smooth=sm, mat=m,
               mat_inv=mi)
    return _call("vq_encode_decode", _ptr(keys), B, H, S, D, _ptr(codebook), codebook.shape[0],
                 sub_dim, code_bits, _ptr(sm), rows, tr, _ptr(m), _ptr(mi), _ptr(codes), codes.shape[2], S_off,
                 offs, _ptr(recon), 1 if recon.dtype == torch.float16 else 0, _stream(stream),
                 prepare=prepare, result=(recon, codes))


def vq_decode(codes, codebook, *, smooth=None, transform=True, S=None, S_off=0,
              out=None, out_dtype=torch.float32, code_bits=8, mat=None, mat_inv=None,
              stream=None, prepare=False):
    """Decode slots [S_off, S_off + S) of codes [B, H, S_cap, row_bytes] into
    [B, H, S, n_sub * sub_dim] (fp32 by default); n_sub = row_bytes, or twice
    that with code_bits=4."""
    _need(codes, "codes", torch.uint8, 4)
    _need(codebook, "codebook", torch.float32, 2)
    B, H, S_cap, nb = codes.shape
    if code_bits not in (8, 4):
        raise ValueError(f"code_bits must be 8 or 4, got {code_bits}")
    n_sub = nb * 8 // code_bits
    sub_dim = codebook.shape[1]
    D = n_sub * sub_dim
    S = S_cap - S_off if S is None else S
    if out is None:
        out = torch.empty((B, H, S, D), dtype=out_dtype, device=codes.device)
    _need(out, "out", (torch.float32, torch.float16), shape=(B, H, S, D))
    sm, rows = _smooth(smooth, D, H)
    tr, m, mi = _transform(transform, mat, mat_inv, D)
    _on_device(codes=codes, codebook=codebook, out=out, smooth=sm, mat=m, mat_inv=mi)
    return _call("vq_decode", _ptr(codes), B, H, S, S_cap, S_off, _ptr(codebook), codebook.shape[0],
                 sub_dim, code_bits, _ptr(sm), rows, tr, _ptr(m), _ptr(mi), D, _ptr(out),
                 1 if out.dtype == torch.float16 else 0, _stream(stream), prepare=prepare,
                 result=out)


def vq_transform(keys, *, smooth=None, transform=True, mat=None, out=None, stream=None,
                 prepare=False):
    """Forward transform (x / s) . M of keys [B, H, S, D] fp16 into fp32
    [B, H, S, D]: the vectors the encode searches and a codebook is trained on
    (view as [-1, sub_dim] for the pooled sub-vectors)."""
    _need(keys, "keys", torch.float16, 4)
    B, H, S, D = keys.shape
    if out is None:
        out = torch.empty((B, H, S, D), dtype=torch.float32, device=keys.device)
    _need(out, "out", torch.float32, shape=(B, H, S, D))
    sm, rows = _smooth(smooth, D, H)
    tr, m, _ = _transform(transform, mat, None, D)
    _on_device(keys=keys, out=out, smooth=sm, mat=m)
    return _call("vq_transform", _ptr(keys), B, H, S, D, _ptr(sm), rows, tr, _ptr(m), _ptr(out),
                 _stream(stream), prepare=prepare, result=out)


def vq_kmeans_workspace_bytes(N, sub_dim, n_centroids) -> int:
    return int(_lib.load().vq_kmeans_workspace_bytes(N, sub_dim, n_centroids))


def vq_kmeans(vectors, centroids, iters, *, labels=None, with_labels=False, inertia=None,
              workspace=None, stream=None, prepare=False):
    """`iters` Lloyd iterations over vectors [N, d] fp32 (any contiguous
    [..., d] is taken as [N, d]); centroids [n_c, d] fp32 are updated in
    place.  Returns (centroids, labels [N] uint8 of the last assignment or
    None, inertia [iters] fp64)."""
    _need(centroids, "centroids", torch.float32, 2)
    n_c, d = centroids.shape
    _need(vectors, "vectors", torch.float32)
    if vectors.dim() < 1 or vectors.shape[-1] != d:
        raise ValueError(f"vectors must be [..., {d}], got {tuple(vectors.shape)}")
    N = vectors.numel() // d
    if labels is None and with_labels:
        labels = torch.empty(N, dtype=torch.uint8, device=centroids.device)
    if labels is not None:
        _need(labels, "labels", torch.uint8, shape=(N,))
    if inertia is None:
        inertia = torch.zeros(max(iters, 0), dtype=torch.float64, device=centroids.device)
    _need(inertia, "inertia", torch.float64, shape=(max(iters, 0),))
    need = vq_kmeans_workspace_bytes(N, d, n_c)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=centroids.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _on_device(vectors=vectors, centroids=centroids, labels=labels, inertia=inertia,
               workspace=workspace)
    return _call("vq_kmeans", _ptr(vectors), ctypes.c_longlong(N), d, _ptr(centroids), n_c, iters,
                 _ptr(labels), _ptr(inertia), _ptr(workspace), workspace.numel(), _stream(stream),
                 prepare=prepare, result=(centroids, labels, inertia))


def vq_attend_workspace_bytes(B, H_q, S_q, D, H_kv, S_cap, sliding_window=0) -> int:
    return int(_lib.load().vq_attend_workspace_bytes(B, H_q, S_q, D, H_kv, S_cap, sliding_window))


PATH_NAMES = {1: "stream", 2: "tile", 3: "lut_mfma", 4: "lut_valu"}


def vq_attend_path(B, H_q, S_q, D, k_sub_dim, v_sub_dim, n_centroids, H_kv, S_cap,
                   sliding_window=0, code_bits=8, transform=1) -> str:
    """Name of the kernel family vq_attend runs for this shape ("stream",
    "tile", "lut_mfma", "lut_valu"); raises VQError when vq_attend would
    reject the shape. Host-only."""
    lib = _lib.load()
    p = int(lib.vq_attend_path(B, H_q, S_q, D, k_sub_dim, v_sub_dim, n_centroids, code_bits,
                               int(transform), H_kv, S_cap, sliding_window))
    if p not in PATH_NAMES:
        raise VQError(VQ_ERR_UNSUPPORTED, lib.vq_last_error().decode())
    return PATH_NAMES[p]


def attend_workspace(q, k_codes, sliding_window=0):
    """A zero-filled workspace sized for vq_attend on these shapes."""
    B, Hq, Sq, D = q.shape
    n = vq_attend_workspace_bytes(B, Hq, Sq, D, k_codes.shape[1], k_codes.shape[2], sliding_window)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=q.device)


def _attend_args(q, k_codes, k_codebook, v_codes, v_codebook, smooth, kv_lens, out, code_bits):
    """Shape checks shared by the attention entry points; returns the
    marshalled sizes and the (allocated if None) output."""
    _need(q, "q", torch.float16, 4)
    B, Hq, Sq, D = q.shape
    _need(k_codebook, "k_codebook", torch.float32, 2)
    _need(v_codebook, "v_codebook", torch.float32, 2)
    dk, dv = k_codebook.shape[1], v_codebook.shape[1]
    nk = _row_bytes(_n_sub(D, dk, "key sub_dim"), code_bits)
    nv = _row_bytes(_n_sub(D, dv, "value sub_dim"), code_bits)
    if k_codebook.shape[0] != v_codebook.shape[0]:
        raise ValueError("key and value codebooks disagree on n_centroids")
    _need(k_codes, "k_codes", torch.uint8, shape=(B, None, None, nk))
    Hkv, S_cap = k_codes.shape[1], k_codes.shape[2]
    _need(v_codes, "v_codes", torch.uint8, shape=(B, Hkv, S_cap, nv))
    if kv_lens is not None:
        _need(kv_lens, "kv_lens", torch.int32, shape=(B,))
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.float16, device=q.device)
    _need(out, "out", torch.float16, shape=(B, Hq, Sq, D))
    sm, rows = _smooth(smooth, D, Hkv)
    return B, Hq, Sq, D, dk, dv, Hkv, S_cap, sm, rows, out


def vq_attend(q, k_codes, k_codebook, v_codes, v_codebook, *, scale, smooth=None,
              transform=True, kv_lens=None, causal=True, sliding_window=0, out=None,
              workspace=None, code_bits=8, mat=None, mat_inv=None, stream=None, prepare=False):
    """Attention of raw fp16 queries [B, H_q, S_q, D] over key/value codes
    [B, H_kv, S_cap, row_bytes] (code_bits wide); returns fp16 [B, H_q, S_q, D]."""
    B, Hq, Sq, D, dk, dv, Hkv, S_cap, sm, rows, out = _attend_args(
        q, k_codes, k_codebook, v_codes, v_codebook, smooth, kv_lens, out, code_bits)
    if workspace is None:
        workspace = attend_workspace(q, k_codes, sliding_window)
    _need(workspace, "workspace", None, 1)
    tr, m, mi = _transform(transform, mat, mat_inv, D)
    _on_device(q=q, k_codes=k_codes, k_codebook=k_codebook, v_codes=v_codes,
               v_codebook=v_codebook, kv_lens=kv_lens, out=out, workspace=workspace, smooth=sm,
               mat=m, mat_inv=mi)
    return _call("vq_attend", _ptr(q), B, Hq, Sq, D, _ptr(k_codes), _ptr(k_codebook),
                 dk, _ptr(sm), rows, tr, _ptr(m), _ptr(mi), _ptr(v_codes),
                 _ptr(v_codebook), dv, k_codebook.shape[0], code_bits, Hkv, S_cap,
                 _ptr(kv_lens), float(scale), int(bool(causal)), int(sliding_window), _ptr(out),
                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream),
                 prepare=prepare, result=out)


def vq_decode_step(q, k_new, v_new, k_codes, k_codebook, v_codes, v_codebook, *, scale, kv_lens,
                   smooth=None, transform=True, causal=True, sliding_window=0, out=None,
                   workspace=None, code_bits=8, stream=None, prepare=False):
    """One decode step in one launch: the codes of the new token k_new /
    v_new [B, H_kv, 1, D] (fp16) go to slot kv_lens[b] - 1 of k_codes /
    v_codes (kv_lens: device int32 [B], the lengths after the append), then
    the attention of q [B, H_q, 1, D] over the updated caches, as
    vq_encode_kv + vq_attend; returns fp16 [B, H_q, 1, D].  Shapes off the
    streaming kernel raise VQError (UNSUPPORTED): use those two calls."""
    B, Hq, Sq, D, dk, dv, Hkv, S_cap, sm, rows, out = _attend_args(
        q, k_codes, k_codebook, v_codes, v_codebook, smooth, kv_lens, out, code_bits)
    if Sq != 1:
        raise ValueError(f"q must hold one query position per row (S_q = 1, got {Sq})")
    if kv_lens is None:
        raise ValueError("kv_lens (the lengths after the append) is required")
    _need(k_new, "k_new", torch.float16, shape=(B, Hkv, 1, D))
    _need(v_new, "v_new", torch.float16, shape=(B, Hkv, 1, D))
    if workspace is None:
        workspace = attend_workspace(q, k_codes, sliding_window)
    _need(workspace, "workspace", None, 1)
    tr, m, mi = _transform(transform, None, None, D)
    _on_device(q=q, k_new=k_new, v_new=v_new, k_codes=k_codes, k_codebook=k_codebook,
               v_codes=v_codes, v_codebook=v_codebook, kv_lens=kv_lens, out=out,
               workspace=workspace, smooth=sm)
    return _call("vq_decode_step", _ptr(q), _ptr(k_new), _ptr(v_new), B, Hq, D, _ptr(k_codes),
                 _ptr(k_codebook), dk, _ptr(sm), rows, tr, _ptr(v_codes), _ptr(v_codebook), dv,
                 k_codebook.shape[0], code_bits, Hkv, S_cap, _ptr(kv_lens), float(scale),
                 int(bool(causal)), int(sliding_window), _ptr(out), _ptr(workspace),
                 workspace.numel() * workspace.element_size(), _stream(stream), prepare=prepare,
                 result=out)


def vq_attend_noalloc(q, k_codes, k_codebook, v_codes, v_codebook, *, scale, smooth=None,
                      transform=True, kv_lens=None, causal=True, sliding_window=0, out=None,
                      code_bits=8, mat=None, mat_inv=None, stream=None, prepare=False):
    """vq_attend with the split partials in the library's per-GPU device
    scratch array instead of a workspace (no device allocation when `out` is
    given).  Calls that overlap on one GPU race; shapes needing more than
    VQ_NOALLOC_SCRATCH_BYTES of partials raise VQError."""
    B, Hq, Sq, D, dk, dv, Hkv, S_cap, sm, rows, out = _attend_args(
        q, k_codes, k_codebook, v_codes, v_codebook, smooth, kv_lens, out, code_bits)
    tr, m, mi = _transform(transform, mat, mat_inv, D)
    _on_device(q=q, k_codes=k_codes, k_codebook=k_codebook, v_codes=v_codes,
               v_codebook=v_codebook, kv_lens=kv_lens, out=out, smooth=sm, mat=m, mat_inv=mi)
    return _call("vq_attend_noalloc", _ptr(q), B, Hq, Sq, D, _ptr(k_codes), _ptr(k_codebook),
                 dk, _ptr(sm), rows, tr, _ptr(m), _ptr(mi), _ptr(v_codes),
                 _ptr(v_codebook), dv, k_codebook.shape[0], code_bits, Hkv, S_cap,
                 _ptr(kv_lens), float(scale), int(bool(causal)), int(sliding_window), _ptr(out),
                 _stream(stream), prepare=prepare, result=out)
