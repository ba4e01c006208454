"""GPU parity of 4-bit codes (two per byte, the even sub-vector in the low
nibble; the packing of rabitq_pack_values on the "Metal Kernels API" page)
through the C ABI against the CPU oracle, which unpacks the GPU's bytes with
its own nibble routine.  Bars as in test_gpu_parity: codes bit-exact except
at near-ties, reconstructions within 1e-3 (+ half an fp16 ulp for fp16),
attention within 2e-3 + 1e-2 |ref|."""
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import (synth, vq_attend, vq_attend_path, vq_decode, vq_encode,
                                     vq_encode_decode, vq_encode_kv)
from test_gpu_parity import (DEV, check_attn, check_codes, check_recon, dev, oracle_attend)

pytestmark = pytest.mark.gpu


def encode_case(seed, B, H, S, D, d, n_c, n_out=2):
    rng = np.random.default_rng(seed)
    k = synth.outlier_normal(rng, (B, H, S, D), n_out)
    s = synth.smooth_factors(k)
    C = synth.sample_rows(rng, O.forward_transform(k, s, True).reshape(-1, d), n_c)
    return k, s, C


@pytest.mark.parametrize("B,H,S,D,d,n_c", [
    (1, 2, 37, 128, 8, 16),      # short: codebook split across waves
    (2, 8, 600, 128, 8, 16),     # the 4-way split tier
    (1, 8, 4500, 128, 8, 16),    # long: one wave per token-heads group
    (2, 3, 301, 64, 4, 11),      # fewer centroids than 16
    (1, 2, 777, 32, 16, 16),     # two sub-vectors per token
    (1, 2, 129, 256, 8, 16),
])
def test_encode_4bit(B, H, S, D, d, n_c):
    k, s, C = encode_case(1500 + S + D + d, B, H, S, D, d, n_c)
    rec, packed = vq_encode_decode(dev(k), dev(C), d, smooth=dev(s), out_dtype=torch.float32,
                                   code_bits=4)
    only = vq_encode(dev(k), dev(C), d, smooth=dev(s), code_bits=4)
    torch.cuda.synchronize()
    packed = packed.cpu().numpy()
    assert packed.shape == (B, H, S, D // d // 2)
    assert np.array_equal(only.cpu().numpy(), packed)
    codes = O.unpack_nibbles(packed)
    check_codes(k, C, d, s, True, codes, f"4-bit D{D} d{d} n_c{n_c} S{S}")
    check_recon(rec.cpu().numpy(), O.decode(codes, C, s, True), "fp32", f"4-bit D{D} d{d}")
    # the packed bytes are the oracle's packing of the same codes
    assert np.array_equal(packed, O.pack_nibbles(codes))


def test_encode_4bit_append_and_decode():
    """4-bit codes written at S_off and at per-row offsets (other slots'
    bytes untouched), then decoded by vq_decode (fp32 and fp16)."""
    B, H, S, D, d, S_cap = 3, 4, 50, 128, 8, 200
    k, s, C = encode_case(1601, B, H, S, D, d, 16)
    ref, gap = O.encode(k, C, d, s, True)
    for offs in (None, [0, 150, 77]):
        buf = torch.full((B, H, S_cap, D // d // 2), 0xAB, dtype=torch.uint8, device=DEV)
        if offs is None:
            vq_encode(dev(k), dev(C), d, smooth=dev(s), codes=buf, S_off=120, code_bits=4)
            offs_b = [120] * B
        else:
            vq_encode(dev(k), dev(C), d, smooth=dev(s), codes=buf, row_offsets=offs, code_bits=4)
            offs_b = offs
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        for b, o in enumerate(offs_b):
            blk = O.unpack_nibbles(got[b, :, o:o + S])
            mis = blk != ref[b]
            assert np.all(gap[b][mis] < 1e-5), f"offs {offs}: mismatches away from near-ties"
            mask = np.ones(S_cap, bool)
            mask[o:o + S] = False
            assert np.all(got[b][:, mask] == 0xAB)
        # decode the written slots of row 0 back
        o0 = offs_b[0]
        out = vq_decode(buf[:1], dev(C), smooth=dev(s), S=S, S_off=o0, code_bits=4)
        out16 = vq_decode(buf[:1], dev(C), smooth=dev(s), S=S, S_off=o0, code_bits=4,
                          out_dtype=torch.float16)
        torch.cuda.synchronize()
        codes0 = O.unpack_nibbles(got[:1, :, o0:o0 + S])
        ref_rec = O.decode(codes0, C, s, True)
        check_recon(out.cpu().numpy(), ref_rec, "fp32", f"4-bit decode offs {offs}")
        check_recon(out16.cpu().numpy(), ref_rec, "fp16", f"4-bit decode fp16 offs {offs}")


def test_decode_4bit_random_codes():
    rng = np.random.default_rng(1602)
    B, H, S_cap, D, d = 2, 3, 40, 64, 4
    C = rng.standard_normal((16, d)).astype(np.float32)
    packed = rng.integers(0, 256, size=(B, H, S_cap, D // d // 2), dtype=np.uint8)
    out = vq_decode(dev(packed), dev(C), transform=False, S=30, S_off=5, code_bits=4)
    torch.cuda.synchronize()
    ref = O.pvq_decode(O.unpack_nibbles(packed[:, :, 5:35]), C)
    assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("B,H,S,S_cap,per_row", [(16, 8, 1, 64, True), (2, 4, 130, 400, False)])
def test_encode_kv_4bit(B, H, S, S_cap, per_row):
    rng = np.random.default_rng(1603 + S)
    D, dk, dv = 128, 8, 4
    k = synth.outlier_normal(rng, (B, H, S, D), 4)
    v = synth.outlier_normal(rng, (B, H, S, D), 4)
    s = synth.smooth_factors(k)
    Ck = synth.sample_rows(rng, O.forward_transform(k, s, True).reshape(-1, dk), 16)
    Cv = synth.sample_rows(rng, v.astype(np.float64).reshape(-1, dv), 16)
    kw = dict(row_offsets=[int(x) for x in rng.integers(0, S_cap - S + 1, size=B)]) if per_row \
        else dict(S_off=S_cap - S)
    fill = lambda n: torch.full((B, H, S_cap, D // n // 2), 0xCD, dtype=torch.uint8, device=DEV)
    kc, vc, kc2, vc2 = fill(dk), fill(dv), fill(dk), fill(dv)
    vq_encode_kv(dev(k), dev(v), dev(Ck), dk, dev(Cv), dv, smooth=dev(s), k_codes=kc, v_codes=vc,
                 code_bits=4, **kw)
    vq_encode(dev(k), dev(Ck), dk, smooth=dev(s), codes=kc2, code_bits=4, **kw)
    vq_encode(dev(v), dev(Cv), dv, transform=False, codes=vc2, code_bits=4, **kw)
    torch.cuda.synchronize()
    kc, vc = kc.cpu().numpy(), vc.cpu().numpy()
    assert np.array_equal(kc, kc2.cpu().numpy()) and np.array_equal(vc, vc2.cpu().numpy())
    offs = kw["row_offsets"] if per_row else [S_cap - S] * B
    got_k = np.stack([O.unpack_nibbles(kc[b, :, o:o + S]) for b, o in enumerate(offs)])
    got_v = np.stack([O.unpack_nibbles(vc[b, :, o:o + S]) for b, o in enumerate(offs)])
    check_codes(k, Ck, dk, s, True, got_k, f"4-bit encode_kv keys B{B} S{S}")
    check_codes(v, Cv, dv, None, False, got_v, f"4-bit encode_kv values B{B} S{S}")


def attend_case(seed, B, Hq, Hkv, Sq, S_cap, lens, D=128, dk=8, dv=4, n_c=16, window=0, causal=True):
    rng = np.random.default_rng(seed)
    return dict(B=B, H_q=Hq, H_kv=Hkv, S_q=Sq, D=D, dk=dk, dv=dv, S_cap=S_cap,
                q=synth.outlier_normal(rng, (B, Hq, Sq, D), 2),
                # codes uniform below n_c, packed by the oracle's nibble routine
                k_packed=O.pack_nibbles(rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dk))),
                v_packed=O.pack_nibbles(rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dv))),
                k_codebook=rng.standard_normal((n_c, dk)).astype(np.float32),
                v_codebook=rng.standard_normal((n_c, dv)).astype(np.float32),
                smooth=rng.uniform(0.5, 5, size=(Hkv, D)).astype(np.float32),
                kv_lens=np.array(lens, np.int32), scale=1 / math.sqrt(D), causal=causal,
                window=window)


def run_4bit(c, packed=True):
    """vq_attend on the packed codes (or, packed=False, on the unpacked codes
    with 8-bit rows: the same attention)."""
    if packed:
        kc, vc, bits = c["k_packed"], c["v_packed"], 4
    else:
        kc = O.unpack_nibbles(c["k_packed"]).astype(np.uint8)
        vc = O.unpack_nibbles(c["v_packed"]).astype(np.uint8)
        bits = 8
    out = vq_attend(dev(c["q"]), dev(kc), dev(c["k_codebook"]), dev(vc), dev(c["v_codebook"]),
                    scale=c["scale"], smooth=dev(c["smooth"]), kv_lens=dev(c["kv_lens"]),
                    causal=c["causal"], sliding_window=c["window"], code_bits=bits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def path_4bit(c):
    return vq_attend_path(c["B"], c["H_q"], c["S_q"], c["D"], c["dk"], c["dv"],
                          c["k_codebook"].shape[0], c["H_kv"], c["S_cap"], c["window"], code_bits=4)


def oracle_4bit(c):
    kc, vc = O.unpack_nibbles(c["k_packed"]), O.unpack_nibbles(c["v_packed"])
    return oracle_attend(dict(c, transform=True), kc, vc)


@pytest.mark.parametrize("Hq,Sq,lens,causal,window", [
    (32, 1, [8192, 5000, 0, 77], True, 0),
    (24, 1, [8192, 8000, 300, 64], True, 0),      # GQA-3: a partly filled 4-row unit
    (16, 3, [8192, 2, 4097, 8191], True, 0),      # several query positions per unit
    (32, 1, [8192, 7000, 6000, 100], False, 0),
    (8, 2, [8192, 8190, 5000, 2000], True, 8191),
])
def test_attend_4bit_stream(Hq, Sq, lens, causal, window):
    """Decode-shaped problems on the streaming kernel with nibble-packed key
    and value codes, every output row against the oracle and against the
    8-bit path on the same codes."""
    c = attend_case(1700 + Hq + Sq, 4, Hq, 8, Sq, 8192, lens, window=window, causal=causal)
    assert path_4bit(c) == "stream"
    out = run_4bit(c)
    ref = oracle_4bit(c)
    check_attn(out, ref, f"4-bit stream Hq{Hq} Sq{Sq} causal{causal} W{window}")
    out8 = run_4bit(c, packed=False)
    assert np.max(np.abs(out.astype(np.float64) - out8)) <= 2e-3


@pytest.mark.parametrize("D,dk,dv,Hq,Hkv,Sq,lens,window", [
    (128, 8, 4, 8, 2, 3, [700, 2, 333], 0),
    (128, 8, 4, 6, 2, 1, [300, 299, 1], 7),
    (64, 4, 4, 4, 4, 2, [500, 17, 250], 0),
    (128, 16, 8, 8, 8, 1, [1000, 999, 64], 0),
    (256, 8, 4, 2, 1, 64, [300, 200, 64], 0),     # many query rows: per-unit kernel
])
def test_attend_4bit_unit_kernel(D, dk, dv, Hq, Hkv, Sq, lens, window):
    """Smaller shapes (the per-unit VALU kernel) with nibble-packed codes,
    against the oracle."""
    c = attend_case(1800 + D + dk + Sq, 3, Hq, Hkv, Sq, max(lens) + 5, lens, D=D, dk=dk, dv=dv,
                    n_c=13, window=window)
    assert path_4bit(c) == "lut_valu"
    out = run_4bit(c)
    check_attn(out, oracle_4bit(c), f"4-bit unit kernel D{D} dk{dk} dv{dv} Sq{Sq} W{window}")


@pytest.mark.parametrize("window", [0, 4096])
def test_gqa_long_4bit_full(window):
    """The long-context GQA decode with 16-centroid codebooks and 4-bit codes
    (24 bytes per token and kv head), all 512 rows against the oracle."""
    c = synth.gqa_long(window, code_bits=4)
    c = dict(c, k_packed=c["k_codes"], v_packed=c["v_codes"])
    assert path_4bit(c) == "stream"
    out = run_4bit(c)
    check_attn(out, oracle_4bit(c), f"4-bit gqa_long W{window}")
