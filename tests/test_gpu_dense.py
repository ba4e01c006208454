"""GPU parity of an explicit transform matrix (transform = 2: the H_mat [D, D]
argument of vecinfer_encode_decode_metal, "Metal Kernels API", "VecInfer
kernels"): encode rotates x / s by M, decode by M^-1, the query's dual
transform is (q * s) . (M^-1)^T.  The GPU receives M and M^-1 in fp32; the
oracle takes M alone (fp64) and inverts it itself.  Bars as in
test_gpu_parity."""
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import (synth, vq_attend, vq_attend_path, vq_decode, vq_encode,
                                     vq_encode_decode, vq_encode_kv)
from test_gpu_parity import DEV, check_attn, check_codes, check_recon, dev, oracle_attend

pytestmark = pytest.mark.gpu


def random_orthogonal(rng, D):
    """Q of a Gaussian matrix's QR: orthogonal, neither symmetric nor involutory."""
    qm, r = np.linalg.qr(rng.standard_normal((D, D)))
    return qm * np.sign(np.diag(r))[None, :]


def general_matrix(rng, D):
    """A well-conditioned matrix that is not orthogonal: I + 0.3 N(0, 1) / sqrt(D)."""
    return np.eye(D) + 0.3 * rng.standard_normal((D, D)) / math.sqrt(D)


def mats(M):
    """The fp32 device matrices the C ABI takes: M and M^-1."""
    return dev(M.astype(np.float32)), dev(np.linalg.inv(M).astype(np.float32))


@pytest.mark.parametrize("kind,B,H,S,D,d,n_c,bits", [
    ("orthogonal", 1, 2, 37, 128, 8, 256, 8),
    ("orthogonal", 1, 8, 2100, 128, 8, 256, 8),
    ("general", 2, 3, 301, 64, 4, 256, 8),
    ("general", 1, 2, 777, 32, 16, 64, 8),
    ("orthogonal", 2, 4, 500, 128, 8, 16, 4),
    ("general", 1, 3, 129, 64, 8, 11, 4),
])
def test_encode_decode_dense(kind, B, H, S, D, d, n_c, bits):
    rng = np.random.default_rng(2000 + S + D + d + bits)
    M = random_orthogonal(rng, D) if kind == "orthogonal" else general_matrix(rng, D)
    k = synth.outlier_normal(rng, (B, H, S, D), 2)
    s = synth.smooth_factors(k)
    C = synth.sample_rows(rng, O.forward_transform(k, s, M).reshape(-1, d), n_c)
    m, mi = mats(M)
    rec, codes = vq_encode_decode(dev(k), dev(C), d, smooth=dev(s), out_dtype=torch.float32,
                                  code_bits=bits, mat=m, mat_inv=mi)
    only = vq_encode(dev(k), dev(C), d, smooth=dev(s), code_bits=bits, mat=m)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    assert np.array_equal(only.cpu().numpy(), codes)
    c8 = O.unpack_nibbles(codes) if bits == 4 else codes
    tag = f"dense {kind} D{D} d{d} n_c{n_c} {bits}-bit S{S}"
    check_codes(k, C, d, s, M, c8, tag)
    ref = O.decode(c8, C, s, M)
    check_recon(rec.cpu().numpy(), ref, "fp32", tag)
    out = vq_decode(dev(codes), dev(C), smooth=dev(s), code_bits=bits, mat_inv=mi)
    out16 = vq_decode(dev(codes), dev(C), smooth=dev(s), code_bits=bits, mat_inv=mi,
                      out_dtype=torch.float16)
    torch.cuda.synchronize()
    check_recon(out.cpu().numpy(), ref, "fp32", tag + " decode")
    check_recon(out16.cpu().numpy(), ref, "fp16", tag + " decode fp16")


def test_encode_kv_dense():
    rng = np.random.default_rng(2101)
    B, H, S, D, dk, dv, S_cap = 16, 8, 1, 128, 8, 4, 64
    M = random_orthogonal(rng, D)
    k = synth.outlier_normal(rng, (B, H, S, D), 4)
    v = synth.outlier_normal(rng, (B, H, S, D), 4)
    s = synth.smooth_factors(k)
    Ck = synth.sample_rows(rng, O.forward_transform(k, s, M).reshape(-1, dk), 256)
    Cv = synth.sample_rows(rng, v.astype(np.float64).reshape(-1, dv), 256)
    offs = [int(x) for x in rng.integers(0, S_cap, size=B)]
    m, mi = mats(M)
    kc = torch.zeros((B, H, S_cap, D // dk), dtype=torch.uint8, device=DEV)
    vc = torch.zeros((B, H, S_cap, D // dv), dtype=torch.uint8, device=DEV)
    vq_encode_kv(dev(k), dev(v), dev(Ck), dk, dev(Cv), dv, smooth=dev(s), k_codes=kc, v_codes=vc,
                 row_offsets=offs, mat=m, mat_inv=mi)
    torch.cuda.synchronize()
    kc, vc = kc.cpu().numpy(), vc.cpu().numpy()
    got_k = np.stack([kc[b, :, o:o + S] for b, o in enumerate(offs)])
    got_v = np.stack([vc[b, :, o:o + S] for b, o in enumerate(offs)])
    check_codes(k, Ck, dk, s, M, got_k, "dense encode_kv keys")
    check_codes(v, Cv, dv, None, False, got_v, "dense encode_kv values")


def attend_case(seed, B, Hq, Hkv, Sq, S_cap, lens, D=128, dk=8, dv=4, n_c=256, window=0):
    rng = np.random.default_rng(seed)
    return dict(B=B, H_q=Hq, H_kv=Hkv, S_q=Sq, D=D, dk=dk, dv=dv, S_cap=S_cap,
                q=synth.outlier_normal(rng, (B, Hq, Sq, D), 2),
                k_codes=rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dk), dtype=np.uint8),
                v_codes=rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dv), dtype=np.uint8),
                k_codebook=rng.standard_normal((n_c, dk)).astype(np.float32),
                v_codebook=rng.standard_normal((n_c, dv)).astype(np.float32),
                smooth=rng.uniform(0.5, 5, size=(Hkv, D)).astype(np.float32),
                kv_lens=np.array(lens, np.int32), scale=1 / math.sqrt(D), causal=True,
                window=window)


def run_dense(c, M):
    _, mi = mats(M)
    out = vq_attend(dev(c["q"]), dev(c["k_codes"]), dev(c["k_codebook"]), dev(c["v_codes"]),
                    dev(c["v_codebook"]), scale=c["scale"], smooth=dev(c["smooth"]),
                    kv_lens=dev(c["kv_lens"]), causal=True, sliding_window=c["window"], mat_inv=mi)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def dense_path(c):
    return vq_attend_path(c["B"], c["H_q"], c["S_q"], c["D"], c["dk"], c["dv"],
                          c["k_codebook"].shape[0], c["H_kv"], c["S_cap"], c["window"], transform=2)


@pytest.mark.parametrize("kind,B,Hq,Hkv,Sq,S_cap,lens,window,family", [
    ("orthogonal", 4, 32, 8, 1, 8192, [8192, 5000, 0, 77], 0, "stream"),
    ("general", 4, 16, 8, 3, 8192, [8192, 2, 4097, 8191], 0, "stream"),
    ("orthogonal", 3, 8, 2, 2, 600, [600, 257, 0], 0, "lut_valu"),
    ("general", 3, 4, 2, 100, 400, [400, 130, 100], 33, "lut_valu"),   # prefill-shaped
])
def test_attend_dense(kind, B, Hq, Hkv, Sq, S_cap, lens, window, family):
    """Attention with the query's dual transform (q * s) . (M^-1)^T computed
    from M^-1, on the streaming and the per-unit kernels, every output row
    against the oracle applying M."""
    rng = np.random.default_rng(2200 + Hq + Sq)
    M = random_orthogonal(rng, 128) if kind == "orthogonal" else general_matrix(rng, 128)
    c = attend_case(2300 + Hq + Sq, B, Hq, Hkv, Sq, S_cap, lens, window=window)
    assert dense_path(c) == family
    out = run_dense(c, M)
    check_attn(out, oracle_attend(dict(c, transform=M), c["k_codes"], c["v_codes"]),
               f"dense {kind} attend ({family}) Hq{Hq} Sq{Sq} W{window}")


def test_gqa_long_dense_full():
    """The long-context GQA decode (all 512 rows) with a random orthogonal
    transform matrix in place of the Walsh-Hadamard rotation."""
    rng = np.random.default_rng(2400)
    M = random_orthogonal(rng, 128)
    c = synth.gqa_long(0)
    assert dense_path(c) == "stream"
    out = run_dense(c, M)
    check_attn(out, oracle_attend(dict(c, transform=M), c["k_codes"], c["v_codes"]),
               "dense gqa_long W0")
