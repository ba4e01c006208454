"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (float tolerances follow the stated targets of the method's hot path):
  codes           bit-exact, except at near-ties where the oracle's top-2
                  distance gap is below 1e-5 relative; there the GPU's
                  choice must itself be a near-optimal centroid (its oracle
                  distance within 1e-5 * d2 of the minimum); mismatches are
                  counted and printed.
  reconstruction  fp32 output within 1e-3 absolute of the fp64 oracle;
                  fp16 output within 1e-3 + half an fp16 ulp of it.
  attention       fp16 output within 2e-3 absolute + 1e-2 relative of the
                  fp64 oracle (allclose form), fed the same codes.
Full-size workloads run on the GPU in the launch configuration the
benchmark times; the oracle checks sampled outputs computed one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import synth
from vector_quantized_kv_amd import (vq_attend, vq_attend_path, vq_decode, vq_encode,
                                     vq_encode_decode)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NEAR_TIE = 1e-5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def oracle_transform(keys, smooth):
    return O.forward_transform(keys, smooth, True)


# ----------------------------------------------------------------------------
# comparison helpers
# ----------------------------------------------------------------------------
def check_codes(keys, codebook, sub_dim, smooth, transform, gpu_codes, tag=""):
    """Compare GPU codes [B, H, S, n_sub] with the oracle under the near-tie
    rule; returns the number of (near-tie) mismatches, which is printed."""
    ref, gap = O.encode(keys, codebook, sub_dim, smooth, transform)
    gpu = np.asarray(gpu_codes).astype(np.int64)
    mism = gpu != ref
    n = int(mism.sum())
    if n:
        assert np.all(gap[mism] < NEAR_TIE), f"{tag}: {n} code mismatches, some not near-ties"
        # distances of the mismatched sub-vectors only: [n, 1, n_c]
        xt = O.forward_transform(keys, smooth, transform)
        sv = xt.reshape(*xt.shape[:-1], -1, sub_dim)[mism]
        dist = O.pvq_distances(sv, codebook, sub_dim)[:, 0]
        d_gpu = dist[np.arange(n), gpu[mism]]
        srt = np.sort(dist, -1)
        d1, d2 = srt[:, 0], srt[:, 1]
        assert np.all(d_gpu - d1 <= NEAR_TIE * d2), f"{tag}: GPU code not near-optimal"
    print(f"[codes] {tag}: {gpu.size} codes, {n} near-tie mismatches")
    return n


def fp16_ulp(x):
    """The fp16 unit in the last place of the binade holding |x|: 2^(e - 10)
    for 2^e <= |x| < 2^(e+1), and 2^-24 in the subnormal range.  (Not the
    spacing of the rounded value: -8.0034 rounds to -8.0, whose spacing
    toward zero is half the 2^-7 gap that -8.0034 sits in.)"""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - 10)


def check_recon(gpu, ref64, dtype, tag=""):
    gpu = np.asarray(gpu).astype(np.float64)
    if dtype == "fp32":
        tol = 1e-3
    else:
        tol = 1e-3 + 0.5 * fp16_ulp(ref64)
    err = np.abs(gpu - ref64)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{tag}: {int(bad.sum())} reconstruction elements out of tolerance; "
                             f"worst at {i}: gpu {gpu[i]!r} ref {ref64[i]!r} tol {tol[i] if np.ndim(tol) else tol:.3g}")
    print(f"[recon] {tag}: max abs err {err.max():.3g}")


def check_attn(gpu, ref, tag=""):
    gpu = np.asarray(gpu).astype(np.float64)
    err = np.abs(gpu - ref)
    bad = err > 2e-3 + 1e-2 * np.abs(ref)
    assert not np.any(np.isnan(gpu)), f"{tag}: NaN in output"
    assert not bad.any(), f"{tag}: {int(bad.sum())} elements out of tolerance, max err {err.max():.3g}"
    print(f"[attn] {tag}: max abs err {err.max():.3g}")


def run_attend(cfg, k_codes=None, v_codes=None, **over):
    p = dict(cfg, **over)
    kc = dev(p["k_codes"] if k_codes is None else k_codes)
    vc = dev(p["v_codes"] if v_codes is None else v_codes)
    lens = None if p.get("kv_lens") is None else dev(np.asarray(p["kv_lens"], np.int32))
    out = vq_attend(dev(p["q"]), kc, dev(p["k_codebook"]), vc, dev(p["v_codebook"]),
                    scale=p["scale"], smooth=None if p.get("smooth") is None else dev(p["smooth"]),
                    transform=p.get("transform", True), kv_lens=lens, causal=p["causal"],
                    sliding_window=p["window"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def path_of(c):
    """The kernel family vq_attend runs for a test case's shape."""
    return vq_attend_path(c["B"], c["H_q"], c["S_q"], c["D"], c["dk"], c["dv"],
                          c["k_codebook"].shape[0], c["H_kv"], c["k_codes"].shape[2], c["window"])


def oracle_attend(p, k_codes, v_codes, rows=None):
    return O.attend(p["q"], k_codes, p["k_codebook"], v_codes, p["v_codebook"], scale=p["scale"],
                    causal=p["causal"], sliding_window=p["window"], smooth=p.get("smooth"),
                    transform=p.get("transform", True), kv_lens=p.get("kv_lens"), rows=rows)


# ----------------------------------------------------------------------------
# tiny workload: encode keys and values, then attend from the GPU's codes
# ----------------------------------------------------------------------------
def test_tiny_end_to_end():
    c = synth.tiny(oracle_transform)
    k, v, s = c["keys"], c["values"], c["smooth"]
    rk, kc = vq_encode_decode(dev(k), dev(c["k_codebook"]), c["dk"], smooth=dev(s),
                              out_dtype=torch.float32)
    rv, vc = vq_encode_decode(dev(v), dev(c["v_codebook"]), c["dv"], transform=False,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    kc, vc = kc.cpu().numpy(), vc.cpu().numpy()
    check_codes(k, c["k_codebook"], c["dk"], s, True, kc, "tiny keys")
    check_codes(v, c["v_codebook"], c["dv"], None, False, vc, "tiny values")
    check_recon(rk.cpu().numpy(), O.decode(kc, c["k_codebook"], s, True), "fp32", "tiny keys")
    check_recon(rv.cpu().numpy(), O.decode(vc, c["v_codebook"]), "fp32", "tiny values")
    # fp16 reconstruction and the encode-only entry point give the same codes
    r16, kc16 = vq_encode_decode(dev(k), dev(c["k_codebook"]), c["dk"], smooth=dev(s))
    kc_only = vq_encode(dev(k), dev(c["k_codebook"]), c["dk"], smooth=dev(s))
    torch.cuda.synchronize()
    assert np.array_equal(kc16.cpu().numpy(), kc) and np.array_equal(kc_only.cpu().numpy(), kc)
    check_recon(r16.cpu().numpy(), O.decode(kc, c["k_codebook"], s, True), "fp16", "tiny keys fp16")
    # attention from the GPU's codes
    p = dict(c, k_codes=kc, v_codes=vc, kv_lens=None)
    out = run_attend(p)
    check_attn(out, oracle_attend(p, kc, vc), "tiny attend")


def test_identity_codebook_round_trip():
    """Codebook rows = transformed sub-vectors of 16 tokens: each sub-vector
    encodes to its own row and the fp16 reconstruction returns the keys.

    The reconstruction is computed in fp32: each element's rounding error is
    at most (log2 D + 3) * 2^-24 * |s_c| * ||x~||_1 (the rotation's adds over
    entries bounded by the transformed vector's 1-norm, the final scale and
    the smooth multiply).  Every element whose half fp16 ulp exceeds that
    bound must come back bit for bit; the others (keys within that bound of
    an fp16 rounding boundary, i.e. tiny elements next to x20 outliers) are
    held to the fp16 reconstruction bar."""
    c = synth.tiny()
    keys = np.ascontiguousarray(c["keys"][:, :1, :16])
    s = c["smooth"][:1]
    D = keys.shape[-1]
    xt = O.forward_transform(keys, s, True)
    C = xt.reshape(-1, c["dk"]).astype(np.float32)
    rec, codes = vq_encode_decode(dev(keys), dev(C), c["dk"], smooth=dev(s))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy().reshape(-1), np.arange(256))
    rec = rec.cpu().numpy()
    check_recon(rec, keys.astype(np.float64), "fp16", "identity codebook")
    bound = (math.log2(D) + 3) * 2.0 ** -24 * np.abs(s[0].astype(np.float64)) \
        * np.abs(xt).sum(-1, keepdims=True)
    k64 = keys.astype(np.float64)
    up = np.nextafter(keys, np.float16(np.inf)).astype(np.float64) - k64
    down = k64 - np.nextafter(keys, np.float16(-np.inf)).astype(np.float64)
    must = np.minimum(up, down) / 2 > bound       # half the gap to either fp16 neighbour
    same = rec.view(np.uint16) == keys.view(np.uint16)
    print(f"[identity] bit-identical fp16 elements: {same.mean():.4f}; "
          f"{int(must.sum())} of {must.size} must be, {int(same[must].sum())} are")
    assert np.all(same[must]), "an element far from an fp16 rounding boundary did not round-trip"


# ----------------------------------------------------------------------------
# key encode throughput workload at full size (sampled oracle)
# ----------------------------------------------------------------------------
def test_encode_full_size():
    """The key-encode workload [1, 8, 8192, 128] (d_k = 8, 256 centroids) in
    the launch configuration the benchmark times: every token-head's codes
    against the oracle (near-tie rule; the mismatch count is printed), and
    every element of the fp16 reconstruction against the oracle's decode of
    the GPU's codes."""
    c = synth.encode(oracle_transform)
    k, s, C = c["keys"], c["smooth"], c["k_codebook"]
    rec, codes = vq_encode_decode(dev(k), dev(C), c["dk"], smooth=dev(s))
    codes_only = vq_encode(dev(k), dev(C), c["dk"], smooth=dev(s))
    torch.cuda.synchronize()
    codes, rec = codes.cpu().numpy(), rec.cpu().numpy()
    assert np.array_equal(codes_only.cpu().numpy(), codes)
    check_codes(k, C, c["dk"], s, True, codes, "encode workload")
    check_recon(rec, O.decode(codes, C, s, True), "fp16", "encode workload")


def test_decode_entry_point():
    rng = np.random.default_rng(1)
    B, H, S_cap, D, d = 2, 3, 40, 128, 8
    C = rng.standard_normal((256, d)).astype(np.float32)
    s = rng.uniform(0.5, 4, size=(H, D)).astype(np.float32)
    codes = rng.integers(0, 256, size=(B, H, S_cap, D // d), dtype=np.uint8)
    out = vq_decode(dev(codes), dev(C), smooth=dev(s), S=25, S_off=7)
    out16 = vq_decode(dev(codes), dev(C), smooth=dev(s), S=25, S_off=7, out_dtype=torch.float16)
    torch.cuda.synchronize()
    ref = O.decode(codes[:, :, 7:32], C, s, True)
    check_recon(out.cpu().numpy(), ref, "fp32", "decode")
    check_recon(out16.cpu().numpy(), ref, "fp16", "decode fp16")
    out = vq_decode(dev(codes), dev(C), transform=False, S=10, S_off=0)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), O.pvq_decode(codes[:, :, :10], C).astype(np.float32))


@pytest.mark.parametrize("D,d,n_c", [(32, 1, 256), (32, 4, 7), (64, 16, 256), (128, 2, 256),
                                     (128, 16, 64), (256, 4, 256), (256, 8, 1)])
def test_encode_shapes(D, d, n_c):
    rng = np.random.default_rng(D * 100 + d)
    B, H, S = 2, 3, 37                       # ragged tail of token-heads
    k = synth.outlier_normal(rng, (B, H, S, D), 2)
    s = synth.smooth_factors(k)
    xt = O.forward_transform(k, s, True).reshape(-1, d)
    C = synth.sample_rows(rng, xt, n_c)
    rec, codes = vq_encode_decode(dev(k), dev(C), d, smooth=dev(s[0]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    check_codes(k, C, d, s[0], True, codes, f"D{D} d{d}")
    check_recon(rec.cpu().numpy(), O.decode(codes, C, s[0], True), "fp32", f"D{D} d{d}")


@pytest.mark.parametrize("S", [10, 200, 600])
def test_encode_codebook_split_tiers(S):
    """Short inputs split the codebook search across 16 or 4 waves of a
    workgroup; longer ones give each wave its own token-heads. All three
    give the oracle's codes (near-tie rule) and reconstructions."""
    rng = np.random.default_rng(300 + S)
    B, H, D, d = 2, 4, 128, 4                # 32 sub-vectors per token-head
    k = synth.outlier_normal(rng, (B, H, S, D), 2)
    s = synth.smooth_factors(k)
    xt = O.forward_transform(k, s, True).reshape(-1, d)
    C = synth.sample_rows(rng, xt, 256)
    rec, codes = vq_encode_decode(dev(k), dev(C), d, smooth=dev(s[0]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    check_codes(k, C, d, s[0], True, codes, f"tiers S{S}")
    check_recon(rec.cpu().numpy(), O.decode(codes, C, s[0], True), "fp32", f"tiers S{S}")


@pytest.mark.parametrize("D,d,n_c,B,H,S,transform,smooth", [
    (128, 8, 256, 1, 2, 2085, True, "per_head"),   # the key workload's head shape
    (128, 4, 256, 1, 3, 757, False, None),         # value encode: no transform, no smooth
    (64, 4, 100, 1, 1, 4097, True, "shared"),      # partial last tile of centroids
    (256, 16, 33, 1, 2, 2049, True, "per_head"),
    (32, 8, 7, 1, 1, 16385, True, None),           # 4 sub-vectors per head
])
def test_encode_matrix_core_shapes(D, d, n_c, B, H, S, transform, smooth):
    """Inputs of at least 65536 sub-vectors with sub_dim 4, 8 or 16 take the
    matrix-core nearest-centroid search; codes (near-tie rule) from vq_encode and
    vq_encode_decode agree with each other and the oracle, and the fp32
    reconstructions with the oracle's.  The last step of each shape is ragged."""
    rng = np.random.default_rng(700 + D + d + n_c)
    k = synth.outlier_normal(rng, (B, H, S, D), 2)
    s = None                                  # [H, D] per head, [D] shared
    if smooth == "per_head":
        s = synth.smooth_factors(k)
    elif smooth == "shared":
        s = np.ascontiguousarray(synth.smooth_factors(k)[0])
    xt = O.forward_transform(k, s, transform).reshape(-1, d)
    C = synth.sample_rows(rng, xt, n_c)
    ds = None if s is None else dev(s)
    rec, codes = vq_encode_decode(dev(k), dev(C), d, smooth=ds, transform=transform,
                                  out_dtype=torch.float32)
    codes_only = vq_encode(dev(k), dev(C), d, smooth=ds, transform=transform)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    assert np.array_equal(codes_only.cpu().numpy(), codes)
    check_codes(k, C, d, s, transform, codes, f"mfma D{D} d{d} n_c{n_c}")
    check_recon(rec.cpu().numpy(), O.decode(codes, C, s, transform), "fp32",
                f"mfma D{D} d{d} n_c{n_c}")


def test_encode_matrix_core_rescaled_steps():
    """Sub-vectors far larger than every centroid leave the fp16 range at the
    codebook's scale; the steps holding them take their own scale (and seeds),
    the others keep the codebook's.  Every 7th token is 64x larger and the
    codebook comes from the unscaled tokens, so both kinds of step occur."""
    rng = np.random.default_rng(811)
    B, H, S, D, d = 1, 2, 2085, 128, 8
    k = synth.outlier_normal(rng, (B, H, S, D), 2)
    C = synth.sample_rows(rng, O.forward_transform(k, None, True).reshape(-1, d), 256)
    k[:, :, ::7] = (k[:, :, ::7].astype(np.float32) * 64).astype(np.float16)
    rec, codes = vq_encode_decode(dev(k), dev(C), d, smooth=None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    check_codes(k, C, d, None, True, codes, "rescaled steps")
    check_recon(rec.cpu().numpy(), O.decode(codes, C, None, True), "fp32", "rescaled steps")


def test_encode_append_and_row_offsets():
    rng = np.random.default_rng(2)
    B, H, S, D, d, S_cap = 3, 2, 5, 64, 4, 20
    k = synth.outlier_normal(rng, (B, H, S, D), 2)
    C = rng.standard_normal((256, d)).astype(np.float32)
    buf = torch.full((B, H, S_cap, D // d), 0xAB, dtype=torch.uint8, device=DEV)
    vq_encode(dev(k), dev(C), d, transform=False, codes=buf, S_off=9)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    ref, _ = O.encode(k, C, d)
    assert np.array_equal(got[:, :, 9:14], ref)
    assert np.all(got[:, :, :9] == 0xAB) and np.all(got[:, :, 14:] == 0xAB)
    buf.fill_(0xAB)
    offs = [0, 15, 7]
    vq_encode(dev(k), dev(C), d, transform=False, codes=buf, row_offsets=offs)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    for b, o in enumerate(offs):
        assert np.array_equal(got[b, :, o:o + S], ref[b])
        mask = np.ones(S_cap, bool)
        mask[o:o + S] = False
        assert np.all(got[b][:, mask] == 0xAB)


@pytest.mark.parametrize("d", [8, 4])
def test_encode_matrix_core_append_offsets(d):
    """The matrix-core encode paths (>= 65536 sub-vectors) writing at S_off and
    at per-row offsets: codes land in the right slots, byte-exact with the
    oracle away from near-ties, and no other slot is touched."""
    rng = np.random.default_rng(900 + d)
    B, H, S, D, S_cap = 4, 8, 600, 128, 1600
    k = synth.outlier_normal(rng, (B, H, S, D), 2)
    s = synth.smooth_factors(k)
    C = synth.sample_rows(rng, O.forward_transform(k, s, True).reshape(-1, d), 256)
    ref, gap = O.encode(k, C, d, s, True)
    near = gap < NEAR_TIE
    for offs in (None, [0, 1000, 7, 419]):
        buf = torch.full((B, H, S_cap, D // d), 0xAB, dtype=torch.uint8, device=DEV)
        if offs is None:
            vq_encode(dev(k), dev(C), d, smooth=dev(s), codes=buf, S_off=333)
            offs_b = [333] * B
        else:
            vq_encode(dev(k), dev(C), d, smooth=dev(s), codes=buf, row_offsets=offs)
            offs_b = offs
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        n_mis = 0
        for b, o in enumerate(offs_b):
            blk = got[b, :, o:o + S].astype(np.int64)
            mis = blk != ref[b]
            assert np.all(near[b][mis]), f"d{d} offs {offs}: mismatches away from near-ties"
            n_mis += int(mis.sum())
            mask = np.ones(S_cap, bool)
            mask[o:o + S] = False
            assert np.all(got[b][:, mask] == 0xAB)
        print(f"[codes] append d{d} offs {offs}: {n_mis} near-tie mismatches")


# ----------------------------------------------------------------------------
# decode attention over random codes
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("S_kv", [512, 2048, 8192])
def test_decode_attend(S_kv):
    c = synth.decode(S_kv)
    out = run_attend(c)
    check_attn(out, oracle_attend(c, c["k_codes"], c["v_codes"]), f"decode S{S_kv}")


@pytest.mark.parametrize("window", [0, 4096])
def test_gqa_long_full(window):
    """The batched long-context GQA decode (B = 16, H_q = 32, H_kv = 8,
    32768-slot buffers, ragged lengths) on the streaming kernel the benchmark
    times: all 512 output rows against the oracle."""
    enc = synth.encode(oracle_transform)
    c = synth.gqa_long(window, k_codebook=enc["k_codebook"], smooth=enc["smooth"])
    assert path_of(c) == "stream"
    out = run_attend(c)
    check_attn(out, oracle_attend(c, c["k_codes"], c["v_codes"]), f"gqa_long W{window}")


def test_prefill_append_and_attend_full():
    """The prefill chunk: 512 new K/V tokens appended at slot 16384 of
    32768-slot buffers with vq_encode_kv (as the benchmark does; vq_encode of
    each half writes the same bytes), every appended code against the oracle,
    untouched slots checked, then all 32 (b, h) x 512 query rows of the causal
    attention over 16896 keys on the tile kernel against the oracle."""
    from vector_quantized_kv_amd import vq_encode_kv
    c = synth.prefill(oracle_transform)
    kbuf, vbuf = dev(c["k_codes"]), dev(c["v_codes"])
    vq_encode_kv(dev(c["keys"]), dev(c["values"]), dev(c["k_codebook"]), c["dk"],
                 dev(c["v_codebook"]), c["dv"], smooth=dev(c["smooth"]), k_codes=kbuf,
                 v_codes=vbuf, S_off=c["S_off"])
    kb2, vb2 = dev(c["k_codes"]), dev(c["v_codes"])
    vq_encode(dev(c["keys"]), dev(c["k_codebook"]), c["dk"], smooth=dev(c["smooth"]), codes=kb2,
              S_off=c["S_off"])
    vq_encode(dev(c["values"]), dev(c["v_codebook"]), c["dv"], transform=False, codes=vb2,
              S_off=c["S_off"])
    torch.cuda.synchronize()
    kc, vc = kbuf.cpu().numpy(), vbuf.cpu().numpy()
    assert np.array_equal(kc, kb2.cpu().numpy()) and np.array_equal(vc, vb2.cpu().numpy())
    lo, hi = c["S_off"], c["S_off"] + c["S_q"]
    assert np.array_equal(kc[:, :, :lo], c["k_codes"][:, :, :lo])
    assert np.array_equal(vc[:, :, :lo], c["v_codes"][:, :, :lo])
    assert np.all(kc[:, :, hi:] == 0) and np.all(vc[:, :, hi:] == 0)
    check_codes(c["keys"], c["k_codebook"], c["dk"], c["smooth"], True, kc[:, :, lo:hi],
                "prefill keys")
    check_codes(c["values"], c["v_codebook"], c["dv"], None, False, vc[:, :, lo:hi],
                "prefill values")
    assert path_of(c) == "tile"
    out = run_attend(c, k_codes=kc, v_codes=vc)
    check_attn(out, oracle_attend(c, kc, vc), "prefill attend")


@pytest.mark.parametrize("family", ["stream", "lut_mfma", "tile"])
def test_outlier_value_codebooks(family):
    """Value codebooks sampled from values with x20 outlier channels (entries
    up to |v| ~ 80) and key codebooks from the transformed outlier keys, with
    x20-outlier queries, so softmax rows are peaked and large value entries
    partly cancel: each kernel family's value path (fp16 value rows, fp16
    weights, fp32 accumulation) against the oracle on every output row."""
    rng = np.random.default_rng(1200 + len(family))
    D, dk, dv = 128, 8, 4
    if family == "stream":
        B, Hq, Hkv, Sq, S_cap, lens = 4, 32, 8, 1, 8192, [8192, 5000, 77, 8100]
    elif family == "lut_mfma":
        B, Hq, Hkv, Sq, S_cap, lens = 3, 8, 2, 2, 2000, [2000, 900, 33]
    else:
        B, Hq, Hkv, Sq, S_cap, lens = 2, 4, 2, 100, 600, [600, 250]
    keys = synth.outlier_normal(rng, (1, Hkv, 4096, D), 4)
    vals = synth.outlier_normal(rng, (1, Hkv, 4096, D), 4)
    s = synth.smooth_factors(keys)
    Ck = synth.sample_rows(rng, O.forward_transform(keys, s, True).reshape(-1, dk), 256)
    Cv = synth.sample_rows(rng, vals.astype(np.float64).reshape(-1, dv), 256)
    assert np.abs(Cv).max() > 20                # rows holding x20 outlier entries
    c = dict(B=B, H_q=Hq, H_kv=Hkv, S_q=Sq, D=D, dk=dk, dv=dv,
             q=synth.outlier_normal(rng, (B, Hq, Sq, D), 4),
             k_codes=synth.uniform_codes(rng, (B, Hkv, S_cap, D // dk)),
             v_codes=synth.uniform_codes(rng, (B, Hkv, S_cap, D // dv)),
             k_codebook=Ck, v_codebook=Cv, smooth=s, kv_lens=np.array(lens, np.int32),
             scale=1 / math.sqrt(D), causal=True, window=0)
    assert path_of(c) == family
    out = run_attend(c)
    ref = oracle_attend(c, c["k_codes"], c["v_codes"])
    check_attn(out, ref, f"outlier value codebooks ({family}), max |ref| {np.abs(ref).max():.1f}")


# ----------------------------------------------------------------------------
# edge cases and metamorphic checks
# ----------------------------------------------------------------------------
def small_case(seed, B=3, Hq=6, Hkv=2, Sq=3, D=64, dk=4, dv=4, n_c=256, S_cap=300):
    rng = np.random.default_rng(seed)
    return dict(B=B, H_q=Hq, H_kv=Hkv, S_q=Sq, D=D, dk=dk, dv=dv,
                q=synth.outlier_normal(rng, (B, Hq, Sq, D), 2),
                k_codes=rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dk), dtype=np.uint8),
                v_codes=rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dv), dtype=np.uint8),
                k_codebook=rng.standard_normal((n_c, dk)).astype(np.float32),
                v_codebook=rng.standard_normal((n_c, dv)).astype(np.float32),
                smooth=rng.uniform(0.5, 5, size=(Hkv, D)).astype(np.float32),
                kv_lens=np.array([S_cap, 1, 150][:B], np.int32), scale=1 / math.sqrt(D),
                causal=True, window=0)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 1), (True, 7), (False, 0),
                                           (False, 5), (True, 10000)])
def test_masks_gqa_multi_query(causal, window):
    c = small_case(10, S_cap=700)
    c["kv_lens"] = np.array([700, 2, 333], np.int32)
    p = dict(c, causal=causal, window=window)
    out = run_attend(p)
    check_attn(out, oracle_attend(p, c["k_codes"], c["v_codes"]), f"masks c{causal} W{window}")


def test_empty_and_short_rows():
    c = small_case(11, Sq=4)
    c["kv_lens"] = np.array([0, 2, 300], np.int32)      # empty row; causal row shorter than S_q
    out = run_attend(c)
    ref = oracle_attend(c, c["k_codes"], c["v_codes"])
    assert np.all(out[0] == 0) and np.all(out[1, :, :2] == 0)
    check_attn(out, ref, "empty/short")


@pytest.mark.parametrize("D,dk,dv,n_c", [(128, 8, 8, 256), (128, 4, 2, 256), (64, 16, 1, 16),
                                         (256, 4, 16, 256), (32, 2, 4, 200), (128, 8, 4, 1)])
def test_attend_shapes(D, dk, dv, n_c):
    c = small_case(D + dk + dv, D=D, dk=dk, dv=dv, n_c=n_c, Sq=1, Hq=8, Hkv=8)
    out = run_attend(c)
    check_attn(out, oracle_attend(c, c["k_codes"], c["v_codes"]), f"D{D} dk{dk} dv{dv} nc{n_c}")


def test_split_invariance_and_gqa_equivalence():
    """The same keys in a larger buffer (different split plan) and the GQA
    layout vs repeated kv heads give the same output."""
    c = small_case(12, B=2, Hq=8, Hkv=2, Sq=1, D=128, dk=8, S_cap=3000)
    c["kv_lens"] = np.array([2900, 1777], np.int32)
    a = run_attend(c)
    big = dict(c)
    pad = lambda x: np.concatenate([x, np.zeros((2, 2, 40000 - 3000, x.shape[3]), np.uint8)], 2)
    big["k_codes"], big["v_codes"] = pad(c["k_codes"]), pad(c["v_codes"])
    b = run_attend(big)
    assert np.max(np.abs(a.astype(np.float64) - b)) <= 2e-3
    rep = dict(c, H_kv=8, k_codes=np.repeat(c["k_codes"], 4, 1), v_codes=np.repeat(c["v_codes"], 4, 1),
               smooth=np.repeat(c["smooth"], 4, 0))
    m = run_attend(rep)
    assert np.max(np.abs(a.astype(np.float64) - m)) <= 2e-3
    check_attn(a, oracle_attend(c, c["k_codes"], c["v_codes"]), "split/gqa")


def test_stream_kernel_window_cuts():
    """A sliding window much shorter than the rows on the streaming kernel
    (B = 16, GQA-4, W = 2100 over ragged lengths up to 4096), every row."""
    c = small_case(95, B=16, Hq=32, Hkv=8, Sq=1, D=128, dk=8, dv=4, S_cap=4096)
    c["kv_lens"] = np.random.default_rng(96).integers(1, 4097, size=16).astype(np.int32)
    c["kv_lens"][:3] = [4096, 2100, 2099]
    c["causal"], c["window"] = True, 2100
    assert path_of(c) == "stream"
    out = run_attend(c)
    ref = oracle_attend(c, c["k_codes"], c["v_codes"])
    check_attn(out, ref, "stream window 2100")


def test_stream_kernel_short_ragged_units():
    """Many short ragged units (B = 16, GQA-4, lengths 1..2048, no window):
    the chunk plan charges every segment switch, so whole chunks fall on
    switch cost and carry no keys, and most chunks hold two or three unit
    segments; every row against the oracle."""
    c = small_case(97, B=16, Hq=32, Hkv=8, Sq=1, D=128, dk=8, dv=4, S_cap=2048)
    c["kv_lens"] = np.random.default_rng(98).integers(1, 2049, size=16).astype(np.int32)
    c["kv_lens"][:4] = [2048, 1, 0, 513]
    assert path_of(c) == "stream"
    out = run_attend(c)
    check_attn(out, oracle_attend(c, c["k_codes"], c["v_codes"]), "stream short ragged units")


@pytest.mark.parametrize("transform,smooth,n_c", [
    (False, "none", 256),     # no rotation, no smoothing
    (True, "shared", 256),    # one smooth row for every kv head
    (True, "per_head", 100),  # fewer centroids than codes the table holds
    (False, "per_head", 7),
])
def test_stream_kernel_options(transform, smooth, n_c):
    """The streaming kernel's query transform and codebook options, against
    the oracle on every output row (B = 4, GQA-4, ragged lengths)."""
    rng = np.random.default_rng(90 + n_c + 2 * int(transform))
    # B * H_kv * 8192 = 2^18 unit-keys: large enough for the streaming kernel
    c = small_case(91 + n_c, B=4, Hq=32, Hkv=8, Sq=1, D=128, dk=8, dv=4, n_c=n_c, S_cap=8192)
    c["kv_lens"] = np.array([8192, 6000, 77, 8000], np.int32)
    c["transform"] = transform
    assert path_of(c) == "stream"
    if smooth == "none":
        c["smooth"] = None
    elif smooth == "shared":
        c["smooth"] = rng.uniform(0.5, 5, size=128).astype(np.float32)  # [D]: one row
    out = run_attend(c)
    ref = oracle_attend(c, c["k_codes"], c["v_codes"])
    check_attn(out, ref, f"stream options transform{transform} smooth {smooth} n_c {n_c}")


@pytest.mark.parametrize("Hq,Hkv,Sq,lens,causal,window", [
    (4, 2, 100, [400, 130, 60], True, 0),     # GQA-2: 128-row tiles span two heads; len < S_q
    (2, 2, 64, [400, 64, 0], True, 0),        # one full row tile per kv head; an empty row
    (8, 2, 40, [400, 300, 41], True, 33),     # GQA-4 with a sliding window
    (2, 1, 129, [400, 200, 129], False, 0),   # non-causal, a 1-row last tile
    (2, 1, 96, [400, 390, 250], False, 50),   # non-causal window
])
def test_many_query_shapes(Hq, Hkv, Sq, lens, causal, window):
    """Shapes with at least 64 query rows per kv head (the prefill path):
    head dim 128, key sub_dim 8, value sub_dim 4, against the oracle."""
    c = small_case(50 + Sq, B=3, Hq=Hq, Hkv=Hkv, Sq=Sq, D=128, dk=8, dv=4, S_cap=400)
    c["kv_lens"] = np.array(lens, np.int32)
    c["causal"], c["window"] = causal, window
    assert path_of(c) == "tile"
    out = run_attend(c)
    ref = oracle_attend(c, c["k_codes"], c["v_codes"])
    check_attn(out, ref, f"many-query Hq{Hq} Hkv{Hkv} Sq{Sq} causal{causal} W{window}")


@pytest.mark.parametrize("Hq,Sq,lens,causal,window", [
    (32, 1, [8192, 5000, 0, 1], True, 0),       # GQA-4 decode, ragged with empty and 1-key rows
    (24, 1, [8192, 8000, 300, 64], True, 0),    # GQA-3: a 4-row unit is partly filled
    (16, 3, [8192, 2, 4097, 8191], True, 0),    # 2 query positions per row group; len < S_q
    (32, 1, [8192, 7000, 6000, 100], False, 0),
    (8, 2, [8192, 8190, 5000, 2000], True, 8191),  # a window as long as the buffer
])
def test_stream_kernel_cases(Hq, Sq, lens, causal, window):
    """Decode-shaped problems large enough for the persistent streaming path
    (head dim 128, key sub_dim 8, value sub_dim 4), every output row checked."""
    c = small_case(70 + Hq + Sq, B=4, Hq=Hq, Hkv=8, Sq=Sq, D=128, dk=8, dv=4, S_cap=8192)
    c["kv_lens"] = np.array(lens, np.int32)
    c["causal"], c["window"] = causal, window
    assert path_of(c) == "stream"
    out = run_attend(c)
    ref = oracle_attend(c, c["k_codes"], c["v_codes"])
    check_attn(out, ref, f"stream Hq{Hq} Sq{Sq} causal{causal} W{window}")


def test_stream_kernel_workspace_reuse():
    """The workspace's contents on entry are ignored: one workspace filled
    with random bytes, then reused by streaming-kernel calls of two shapes
    in turn (and by repeated calls), gives every call the oracle's result."""
    cases = []
    for seed, Hq, lens in [(301, 32, [8192, 5000, 0, 1]), (302, 24, [8000, 8192, 300, 64])]:
        c = small_case(seed, B=4, Hq=Hq, Hkv=8, Sq=1, D=128, dk=8, dv=4, S_cap=8192)
        c["kv_lens"] = np.array(lens, np.int32)
        c["causal"], c["window"] = True, 0
        assert path_of(c) == "stream"
        cases.append(c)
    n = max(api_workspace_bytes(c) for c in cases)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    refs = [oracle_attend(c, c["k_codes"], c["v_codes"]) for c in cases]
    args = [dict(q=dev(c["q"]), kc=dev(c["k_codes"]), kb=dev(c["k_codebook"]), vc=dev(c["v_codes"]),
                 vb=dev(c["v_codebook"]), sm=dev(c["smooth"]), lens=dev(c["kv_lens"])) for c in cases]
    for it, i in enumerate([0, 1, 0, 1, 1, 0, 0] + [0, 1] * 8):
        c, a = cases[i], args[i]
        out = vq_attend(a["q"], a["kc"], a["kb"], a["vc"], a["vb"], scale=c["scale"], smooth=a["sm"],
                        kv_lens=a["lens"], causal=True, sliding_window=0, workspace=ws)
        torch.cuda.synchronize()
        check_attn(out.cpu().numpy(), refs[i], f"workspace reuse call {it} (shape {i})")


def api_workspace_bytes(c):
    from vector_quantized_kv_amd import vq_attend_workspace_bytes
    return vq_attend_workspace_bytes(c["B"], c["H_q"], c["S_q"], c["D"], c["H_kv"],
                                     c["k_codes"].shape[2], c["window"])


# ----------------------------------------------------------------------------
# randomized Hadamard rotation M = diag(sigma) . H (sigma in {-1, +1}^D):
# the GPU path takes it as smooth factors s * sigma with the plain Hadamard
# transform; the oracle applies M itself as a dense matrix
# ----------------------------------------------------------------------------
def randomized_hadamard(rng, D):
    sigma = rng.choice([-1.0, 1.0], size=D)
    return sigma, sigma[:, None] * O.sylvester_hadamard(D)


@pytest.mark.parametrize("H,S", [(8, 37), (2, 4500)])   # per-lane search; matrix-core search
def test_randomized_hadamard_encode_decode(H, S):
    rng = np.random.default_rng(800 + S)
    B, D, d = 1, 128, 8
    k = synth.outlier_normal(rng, (B, H, S, D), 4)
    s = synth.smooth_factors(k).astype(np.float64)
    sigma, M = randomized_hadamard(rng, D)
    C = synth.sample_rows(rng, O.forward_transform(k, s, M).reshape(-1, d), 256)
    s_signed = (s * sigma).astype(np.float32)
    rec, codes = vq_encode_decode(dev(k), dev(C), d, smooth=dev(s_signed), out_dtype=torch.float32)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy()
    check_codes(k, C, d, s, M, codes, f"randomized Hadamard H{H} S{S}")
    ref = O.decode(codes, C, s, M)
    check_recon(rec.cpu().numpy(), ref, "fp32", f"randomized Hadamard H{H} S{S}")
    out = vq_decode(dev(codes), dev(C), smooth=dev(s_signed))
    torch.cuda.synchronize()
    check_recon(out.cpu().numpy(), ref, "fp32", f"randomized Hadamard decode H{H} S{S}")


@pytest.mark.parametrize("family", ["stream", "tile", "lut_mfma"])
def test_randomized_hadamard_attend(family):
    rng = np.random.default_rng(900 + len(family))
    if family == "stream":
        c = small_case(901, B=4, Hq=32, Hkv=8, Sq=1, D=128, dk=8, dv=4, S_cap=8192)
        c["kv_lens"] = np.array([8192, 5000, 77, 8100], np.int32)
    elif family == "tile":
        c = small_case(902, B=3, Hq=4, Hkv=2, Sq=100, D=128, dk=8, dv=4, S_cap=400)
        c["kv_lens"] = np.array([400, 130, 100], np.int32)
    else:
        c = small_case(903)                          # D = 64, GQA-3, 3 query positions
    assert path_of(c) == family
    sigma, M = randomized_hadamard(rng, c["D"])
    s = c["smooth"].astype(np.float64)
    out = run_attend(c, smooth=(s * sigma).astype(np.float32))
    ref = oracle_attend(dict(c, smooth=s, transform=M), c["k_codes"], c["v_codes"])
    check_attn(out, ref, f"randomized Hadamard attend ({family})")


# ----------------------------------------------------------------------------
# keys and values of one append in one call
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,S,D,dk,dv,S_cap,per_row", [
    (16, 8, 1, 128, 8, 4, 64, True),      # decode-step append: one launch, 16-way codebook split
    (3, 4, 125, 128, 8, 4, 300, False),   # one launch, 4-way split
    (2, 2, 3, 64, 4, 4, 16, True),        # head dim 64
    (2, 3, 100, 128, 8, 4, 128, False),   # the halves take different splits: two launches
    (1, 8, 2048, 128, 8, 4, 2048, False), # matrix-core search: two launches
])
def test_encode_kv(B, H, S, D, dk, dv, S_cap, per_row):
    """vq_encode_kv writes the same codes as vq_encode on the keys (smoothed,
    rotated) and on the values (neither), the oracle's codes under the
    near-tie rule, and leaves every other slot untouched."""
    from vector_quantized_kv_amd import vq_encode_kv
    rng = np.random.default_rng(1000 + B * H * S + D + dk)
    k = synth.outlier_normal(rng, (B, H, S, D), 4)
    v = synth.outlier_normal(rng, (B, H, S, D), 4)
    s = synth.smooth_factors(k)
    xk = O.forward_transform(k, s, True).reshape(-1, dk)
    xv = v.astype(np.float64).reshape(-1, dv)
    Ck = synth.sample_rows(rng, xk, min(256, len(xk)))
    # a value codebook of fewer centroids than the key codebook's 256
    Cv = synth.sample_rows(rng, xv, min(256 if per_row else 100, len(xv)))
    if per_row:
        offs = [int(x) for x in rng.integers(0, S_cap - S + 1, size=B)]
        kw = dict(row_offsets=offs)
    else:
        offs = [S_cap - S] * B
        kw = dict(S_off=S_cap - S)
    fill = lambda n: torch.full((B, H, S_cap, D // n), 0xAB, dtype=torch.uint8, device=DEV)
    kc, vc, kc2, vc2 = fill(dk), fill(dv), fill(dk), fill(dv)
    vq_encode_kv(dev(k), dev(v), dev(Ck), dk, dev(Cv), dv, smooth=dev(s), k_codes=kc, v_codes=vc, **kw)
    vq_encode(dev(k), dev(Ck), dk, smooth=dev(s), codes=kc2, **kw)
    vq_encode(dev(v), dev(Cv), dv, transform=False, codes=vc2, **kw)
    torch.cuda.synchronize()
    kc, vc, kc2, vc2 = (t.cpu().numpy() for t in (kc, vc, kc2, vc2))
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)
    for codes, x, C, d, sm, tr, tag in [(kc, k, Ck, dk, s, True, "keys"), (vc, v, Cv, dv, None, False, "values")]:
        mask = np.zeros(codes.shape[:3], bool)
        for b in range(B):
            mask[b, :, offs[b]:offs[b] + S] = True
        assert np.all(codes[~mask] == 0xAB), f"{tag}: a slot outside the append was written"
        got = np.stack([codes[b, :, offs[b]:offs[b] + S] for b in range(B)])
        check_codes(x, C, d, sm, tr, got, f"encode_kv {tag} B{B} H{H} S{S} D{D}")


def test_single_split_direct_output():
    """Key ranges up to 1024 run as one split per unit, whose workgroup
    writes the output rows itself (no merge launch): the same keys in a
    larger buffer (several splits and the merge) give the same rows, both
    match the oracle, including an empty row and a windowed range."""
    c = small_case(13, B=3, Hq=8, Hkv=2, Sq=2, D=128, dk=8, dv=4, S_cap=1000)
    c["kv_lens"] = np.array([1000, 517, 0], np.int32)
    assert path_of(c) == "lut_mfma"
    a = run_attend(c)
    big = dict(c)
    pad = lambda x: np.concatenate([x, np.zeros((3, 2, 1100 - 1000, x.shape[3]), np.uint8)], 2)
    big["k_codes"], big["v_codes"] = pad(c["k_codes"]), pad(c["v_codes"])
    b = run_attend(big)
    assert np.max(np.abs(a.astype(np.float64) - b)) <= 2e-3
    assert np.all(a[2] == 0)
    check_attn(a, oracle_attend(c, c["k_codes"], c["v_codes"]), "one split")
    check_attn(b, oracle_attend(big, big["k_codes"], big["v_codes"]), "several splits")
    w = small_case(14, B=3, Hq=8, Hkv=2, Sq=2, D=128, dk=8, dv=4, S_cap=6000)
    w["kv_lens"] = np.array([6000, 3000, 10], np.int32)
    w["window"] = 700                       # key range 701: one split
    check_attn(run_attend(w), oracle_attend(w, w["k_codes"], w["v_codes"]), "one split, window 700")


def test_graph_capture_decode_step():
    """The decode step (vq_encode_kv of one token per row, then vq_attend on
    the streaming kernel) captured in a HIP graph and replayed with new
    inputs, with eager calls between the replays: every replay writes the
    eager codes and matches the eager output and the oracle."""
    from vector_quantized_kv_amd import attend_workspace, vq_encode_kv
    c = small_case(401, B=4, Hq=32, Hkv=8, Sq=1, D=128, dk=8, dv=4, S_cap=8192)
    c["kv_lens"] = np.array([8192, 6000, 77, 8000], np.int32)
    assert path_of(c) == "stream"
    kc, vc = dev(c["k_codes"]), dev(c["v_codes"])
    kb, vb, sm, kl = dev(c["k_codebook"]), dev(c["v_codebook"]), dev(c["smooth"]), dev(c["kv_lens"])
    offs = [int(x) - 1 for x in c["kv_lens"]]
    q = torch.empty((4, 32, 1, 128), dtype=torch.float16, device=DEV)
    kn = torch.empty((4, 8, 1, 128), dtype=torch.float16, device=DEV)
    vn = torch.empty_like(kn)
    out = torch.empty_like(q)
    ws = attend_workspace(q, kc, 0)

    def new_inputs(seed):
        r = np.random.default_rng(seed)
        q.copy_(dev(synth.outlier_normal(r, (4, 32, 1, 128), 2)))
        kn.copy_(dev(synth.outlier_normal(r, (4, 8, 1, 128), 2)))
        vn.copy_(dev(synth.outlier_normal(r, (4, 8, 1, 128), 2)))

    def step():
        vq_encode_kv(kn, vn, kb, 8, vb, 4, smooth=sm, k_codes=kc, v_codes=vc, row_offsets=offs)
        vq_attend(q, kc, kb, vc, vb, scale=c["scale"], smooth=sm, kv_lens=kl, causal=True,
                  sliding_window=0, out=out, workspace=ws)

    new_inputs(0)
    step()                                   # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        new_inputs(10 + rep)
        g.replay()
        torch.cuda.synchronize()
        got, gk, gv = out.clone(), kc.clone(), vc.clone()
        step()                               # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(gk, kc) and torch.equal(gv, vc), f"replay {rep}: codes differ from eager"
        # the streaming kernel's waves claim blocks dynamically, so sums may
        # round differently between runs
        assert (got.float() - out.float()).abs().max().item() <= 2e-3, f"replay {rep}"
        p = dict(c, q=q.cpu().numpy())
        check_attn(got.cpu().numpy(), oracle_attend(p, kc.cpu().numpy(), vc.cpu().numpy()),
                   f"graph replay {rep}")


@pytest.mark.parametrize("S_cap,lens,window", [
    (8255, [8255, 8254, 4097, 63], 0),     # buffer length not a multiple of the 64-key block
    (8255, [8255, 8192, 8191, 1] + [2100 + 300 * i for i in range(12)], 2100),  # B = 16, a window
])
def test_stream_kernel_ragged_buffer(S_cap, lens, window):
    """The streaming kernel's blocks read past S_cap through range-checked
    loads (zeros there, always masked): a buffer whose length is not a
    multiple of 64, rows filling it, every output row against the oracle."""
    B = len(lens)
    c = small_case(700 + B + window, B=B, Hq=32, Hkv=8, Sq=1, D=128, dk=8, dv=4, S_cap=S_cap)
    c["kv_lens"] = np.array(lens, np.int32)
    c["window"] = window
    assert path_of(c) == "stream"
    out = run_attend(c)
    check_attn(out, oracle_attend(c, c["k_codes"], c["v_codes"]), f"stream S_cap {S_cap} W{window}")


@pytest.mark.parametrize("family", ["tile", "lut_mfma"])
@pytest.mark.parametrize("transform,smooth,n_c", [
    (False, "none", 256),     # no rotation, no smoothing
    (True, "shared", 100),    # one smooth row for every kv head; fewer centroids
    (False, "per_head", 7),
])
def test_tile_and_unit_kernel_options(family, transform, smooth, n_c):
    """The many-query (prefill) and per-unit kernels with the query-transform
    and codebook options, against the oracle on every output row."""
    rng = np.random.default_rng(80 + n_c + 2 * int(transform) + len(family))
    if family == "tile":
        c = small_case(81 + n_c, B=3, Hq=4, Hkv=2, Sq=100, D=128, dk=8, dv=4, n_c=n_c, S_cap=400)
        c["kv_lens"] = np.array([400, 130, 100], np.int32)
    else:
        c = small_case(82 + n_c, B=3, Hq=8, Hkv=2, Sq=2, D=128, dk=8, dv=4, n_c=n_c, S_cap=600)
        c["kv_lens"] = np.array([600, 257, 0], np.int32)
    c["transform"] = transform
    assert path_of(c) == family
    if smooth == "none":
        c["smooth"] = None
    elif smooth == "shared":
        c["smooth"] = rng.uniform(0.5, 5, size=128).astype(np.float32)
    out = run_attend(c)
    check_attn(out, oracle_attend(c, c["k_codes"], c["v_codes"]),
               f"{family} transform{transform} smooth {smooth} n_c {n_c}")
