"""The KV-cache layer on the GPU against the oracle ("veloxquant_mlx.cache.
vecinfer_cache module" page, VecInferKVCache): standard-mode update_and_fetch
returns the dequantized keys and values of every stored token; fused mode
keeps the code indices and attends from them; a ring keeps the last S_cap
tokens for decoding; trim rewinds the write position so no stale tail is
attended."""
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import VQKVCache, synth
from test_gpu_parity import DEV, check_attn, check_codes, check_recon, dev

pytestmark = pytest.mark.gpu

B, H, D, DK, DV = 2, 4, 128, 8, 4


def make_inputs(seed, S_total, bits=8):
    rng = np.random.default_rng(seed)
    k = synth.outlier_normal(rng, (B, H, S_total, D), 4)
    v = synth.outlier_normal(rng, (B, H, S_total, D), 4)
    s = synth.smooth_factors(k)
    n_c = 256 if bits == 8 else 16
    Ck = synth.sample_rows(rng, O.forward_transform(k, s, True).reshape(-1, DK), n_c)
    Cv = synth.sample_rows(rng, v.astype(np.float64).reshape(-1, DV), n_c)
    return k, v, s, Ck, Cv


def stored_codes(cache, bits):
    kc, vc = (t.cpu().numpy() for t in cache.state)
    if bits == 4:
        kc, vc = O.unpack_nibbles(kc), O.unpack_nibbles(vc)
    return kc.astype(np.int64), vc.astype(np.int64)


@pytest.mark.parametrize("bits", [8, 4])
def test_standard_mode(bits):
    """update_and_fetch over three appends returns, for every stored token,
    the oracle's decode of the oracle's codes (tokens holding a near-tie
    sub-vector are counted and checked against the decode of either code)."""
    k, v, s, Ck, Cv = make_inputs(3000 + bits, 300, bits)
    cache = VQKVCache(B, H, D, 512, dev(Ck), dev(Cv), smooth=dev(s), code_bits=bits,
                      mode="standard")
    for lo, hi in [(0, 200), (200, 201), (201, 300)]:
        khat, vhat = cache.update_and_fetch(dev(k[:, :, lo:hi]), dev(v[:, :, lo:hi]))
        assert khat.shape == (B, H, hi, D)
    torch.cuda.synchronize()
    kref_codes, kgap = O.encode(k, Ck, DK, s, True)
    vref_codes, vgap = O.encode(v, Cv, DV)
    for got, codes, gap, C, sm, tr, tag in [
            (khat, kref_codes, kgap, Ck, s, True, "keys"),
            (vhat, vref_codes, vgap, Cv, None, False, "values")]:
        got = got.cpu().numpy()
        ref = O.decode(codes, C, sm, tr)
        clean = np.all(gap >= 1e-5, axis=-1)           # tokens with no near-tie sub-vector
        print(f"[cache] standard {bits}-bit {tag}: {int((~clean).sum())} tokens hold a near-tie")
        check_recon(got[clean], ref[clean], "fp16", f"standard {bits}-bit {tag}")
    assert cache.size() == 300 and cache.compressed_key_bytes == B * H * 300 * (D // DK) * bits // 8


@pytest.mark.parametrize("bits", [8, 4])
def test_fused_mode_prefill_then_decode(bits):
    """A prefill chunk then single-token appends in fused mode: the stored
    indices are the oracle's codes, and fused_sdpa of raw queries equals the
    oracle's attention over them."""
    k, v, s, Ck, Cv = make_inputs(3100 + bits, 260, bits)
    cache = VQKVCache(B, H, D, 512, dev(Ck), dev(Cv), smooth=dev(s), code_bits=bits)
    rng = np.random.default_rng(3101)
    cache.update_and_fetch(dev(k[:, :, :256]), dev(v[:, :, :256]))
    for t in range(256, 260):
        cache.update_and_fetch(dev(k[:, :, t:t + 1]), dev(v[:, :, t:t + 1]))
    q = synth.outlier_normal(rng, (B, 2 * H, 1, D), 2)
    out = cache.fused_sdpa(dev(q), 1 / math.sqrt(D)).cpu().numpy()
    kc, vc = stored_codes(cache, bits)
    check_codes(k, Ck, DK, s, True, kc, f"fused {bits}-bit keys")
    check_codes(v, Cv, DV, None, False, vc, f"fused {bits}-bit values")
    ref = O.attend(q, kc, Ck, vc, Cv, scale=1 / math.sqrt(D), smooth=s, transform=True)
    check_attn(out, ref, f"fused {bits}-bit attend")


def test_ring_keeps_the_last_tokens():
    """A 64-slot ring fed 150 tokens (chunks that wrap) holds the last 64;
    decode attention over it equals the oracle's over those 64 tokens in
    token order."""
    S_cap = 64
    k, v, s, Ck, Cv = make_inputs(3200, 150)
    cache = VQKVCache(B, H, D, S_cap, dev(Ck), dev(Cv), smooth=dev(s), ring=True)
    for lo, hi in [(0, 40), (40, 100), (100, 101), (101, 150)]:
        cache.update_and_fetch(dev(k[:, :, lo:hi]), dev(v[:, :, lo:hi]))
    assert cache.size() == S_cap and not cache.is_trimmable() and cache.trim(5) == 0
    q = synth.outlier_normal(np.random.default_rng(3201), (B, H, 1, D), 2)
    out = cache.fused_sdpa(dev(q), 1 / math.sqrt(D)).cpu().numpy()
    kc, vc = stored_codes(cache, 8)
    order = [(p % S_cap) for p in range(150 - S_cap, 150)]      # slots in token order
    kc, vc = kc[:, :, order], vc[:, :, order]
    check_codes(k[:, :, 150 - S_cap:], Ck, DK, s, True, kc, "ring keys")
    ref = O.attend(q, kc, Ck, vc, Cv, scale=1 / math.sqrt(D), smooth=s, transform=True)
    check_attn(out, ref, "ring decode")
    with pytest.raises(ValueError, match="token order"):
        cache.fused_sdpa(dev(np.concatenate([q, q], 2)), 1 / math.sqrt(D))


@pytest.mark.parametrize("ring", [False, True])
def test_trim_rewinds_the_write_position(ring):
    """Append 50, trim 10, append 5 new tokens: the cache holds the first 40
    old tokens then the 5 new ones (the new codes overwrite the trimmed
    slots), and attention sees exactly those 45."""
    k, v, s, Ck, Cv = make_inputs(3300 + ring, 55)
    cache = VQKVCache(B, H, D, 64, dev(Ck), dev(Cv), smooth=dev(s), ring=ring)
    cache.update_and_fetch(dev(k[:, :, :50]), dev(v[:, :, :50]))
    assert cache.trim(10) == 10 and cache.size() == 40
    cache.update_and_fetch(dev(k[:, :, 50:55]), dev(v[:, :, 50:55]))
    assert cache.size() == 45
    keep = list(range(40)) + list(range(50, 55))
    kc, vc = stored_codes(cache, 8)
    check_codes(np.ascontiguousarray(k[:, :, keep]), Ck, DK, s, True, kc, f"trim ring={ring}")
    q = synth.outlier_normal(np.random.default_rng(3301), (B, H, 2, D), 2)
    out = cache.fused_sdpa(dev(q), 1 / math.sqrt(D)).cpu().numpy()
    ref = O.attend(q, kc, Ck, vc, Cv, scale=1 / math.sqrt(D), smooth=s, transform=True)
    check_attn(out, ref, f"attend after trim ring={ring}")


@pytest.mark.parametrize("S_cap,bits", [(32768, 8), (32768, 4), (512, 8)])
def test_decode_step(S_cap, bits):
    """decode_step on a fused-mode cache (one vq_decode_step launch when the
    shape runs on the streaming kernel, else update_and_fetch + fused_sdpa)
    stores the same codes as the two calls on a twin cache, and attends
    within the attention bar of them and of the oracle."""
    from vector_quantized_kv_amd import vq_attend_path
    k, v, s, Ck, Cv = make_inputs(3400 + bits + S_cap % 7, 303, bits)
    kw = dict(smooth=dev(s), code_bits=bits)
    a = VQKVCache(B, H, D, S_cap, dev(Ck), dev(Cv), **kw)
    b = VQKVCache(B, H, D, S_cap, dev(Ck), dev(Cv), **kw)
    for c in (a, b):
        c.update_and_fetch(dev(k[:, :, :300]), dev(v[:, :, :300]))
    rng = np.random.default_rng(3401)
    n_c = Ck.shape[0]
    print(f"[cache] decode_step S_cap={S_cap} {bits}-bit: path "
          f"{vq_attend_path(B, 2 * H, 1, D, DK, DV, n_c, H, S_cap, code_bits=bits)}")
    for t in range(300, 303):
        q = synth.outlier_normal(rng, (B, 2 * H, 1, D), 2)
        out_a = a.decode_step(dev(q), dev(k[:, :, t:t + 1]), dev(v[:, :, t:t + 1]), 1 / math.sqrt(D))
        b.update_and_fetch(dev(k[:, :, t:t + 1]), dev(v[:, :, t:t + 1]))
        out_b = b.fused_sdpa(dev(q), 1 / math.sqrt(D))
        torch.cuda.synchronize()
        assert a.size() == b.size() == t + 1
        for x, y in zip(a.state, b.state):
            assert torch.equal(x, y), "decode_step stored other codes than update_and_fetch"
        check_attn(out_a.cpu().numpy(), out_b.cpu().numpy().astype(np.float64),
                   f"decode_step S_cap={S_cap} {bits}-bit against the two calls")
    kc, vc = stored_codes(a, bits)
    check_codes(k, Ck, DK, s, True, kc, f"decode_step {bits}-bit keys")
    check_codes(v, Cv, DV, None, False, vc, f"decode_step {bits}-bit values")
    ref = O.attend(q, kc, Ck, vc, Cv, scale=1 / math.sqrt(D), smooth=s, transform=True)
    check_attn(out_a.cpu().numpy(), ref, f"decode_step S_cap={S_cap} {bits}-bit against the oracle")
