"""GPU parity of the fused decode step (vq_decode_step: the append of one new
token per row, then attention over the updated caches, in one launch of the
streaming kernel) through the C ABI.

The caches must equal those of its two-call form byte for byte: vq_encode_kv
of the new tokens at per-row offsets kv_lens - 1 (rows with kv_lens 0 get
nothing), then vq_attend.  The appended codes are also checked against the
oracle's encode (bit-exact except at near-ties), and the output against the
two-call output and, on sampled rows, the oracle's attention over the updated
caches, within the bar of the attention tests (2e-3 + 1e-2 |ref|).  The
outputs are not compared bit for bit: the streaming kernel's waves claim
blocks dynamically, so two runs of the same attention call can round the
softmax weights differently.  Half of the query heads point along their kv
head's new key (q = 4 k_new), so the new token dominates those rows and a
stale read of its codes would miss the bar by far."""
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import (attend_workspace, synth, vq_attend, vq_attend_path, vq_decode_step,
                                     vq_encode_kv)
from test_gpu_parity import DEV, check_attn, check_codes, dev

pytestmark = pytest.mark.gpu


def step_case(seed, B, Hq, Hkv, S_cap, lens, bits, n_c, smooth_rows, transform):
    D, dk, dv = 128, 8, 4
    rng = np.random.default_rng(seed)
    sample = synth.outlier_normal(rng, (1, Hkv, 64, D), 2)
    s = synth.smooth_factors(sample) if smooth_rows else None
    if s is not None and smooth_rows == 1:
        s = s[:1]
    sm_full = None if s is None else (np.repeat(s, Hkv, 0) if s.shape[0] == 1 else s)
    Ck = synth.sample_rows(rng, O.forward_transform(sample, sm_full, transform).reshape(-1, dk), n_c)
    Cv = synth.sample_rows(rng, synth.outlier_normal(rng, (1, Hkv, 64, D), 2).reshape(-1, dv), n_c)
    nk, nv = D // dk * bits // 8, D // dv * bits // 8
    q = synth.outlier_normal(rng, (B, Hq, 1, D), 2)
    k_new = synth.outlier_normal(rng, (B, Hkv, 1, D), 4)
    G = Hq // Hkv
    for h in range(0, Hq, 2):   # even heads: aligned with the new key of their kv head
        q[:, h] = (4 * k_new[:, h // G].astype(np.float32)).astype(np.float16)
    return dict(
        B=B, H_q=Hq, H_kv=Hkv, D=D, dk=dk, dv=dv, bits=bits, transform=transform,
        q=q, k_new=k_new,
        v_new=synth.outlier_normal(rng, (B, Hkv, 1, D), 4),
        k_codes=rng.integers(0, n_c, size=(B, Hkv, S_cap, nk), dtype=np.uint8)
        if bits == 8 else O.pack_nibbles(rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dk))),
        v_codes=rng.integers(0, n_c, size=(B, Hkv, S_cap, nv), dtype=np.uint8)
        if bits == 8 else O.pack_nibbles(rng.integers(0, n_c, size=(B, Hkv, S_cap, D // dv))),
        k_codebook=Ck, v_codebook=Cv, smooth=s, smooth_full=sm_full,
        kv_lens=np.asarray(lens, np.int32), scale=1 / math.sqrt(D))


def run_step(c, causal, window):
    """(fused caches, fused out, two-call caches, two-call out) as numpy."""
    kc, vc = dev(c["k_codes"]), dev(c["v_codes"])
    kc2, vc2 = kc.clone(), vc.clone()
    lens = dev(c["kv_lens"])
    Ck, Cv, q = dev(c["k_codebook"]), dev(c["v_codebook"]), dev(c["q"])
    sm = None if c["smooth"] is None else dev(c["smooth"])
    kn, vn = dev(c["k_new"]), dev(c["v_new"])
    kw = dict(scale=c["scale"], smooth=sm, transform=c["transform"], kv_lens=lens, causal=causal,
              sliding_window=window, code_bits=c["bits"])
    out = vq_decode_step(q, kn, vn, kc, Ck, vc, Cv, **kw)
    for b, L in enumerate(c["kv_lens"]):
        if L >= 1:
            vq_encode_kv(kn[b:b + 1], vn[b:b + 1], Ck, c["dk"], Cv, c["dv"], smooth=sm,
                         transform=c["transform"], k_codes=kc2[b:b + 1], v_codes=vc2[b:b + 1],
                         row_offsets=[int(L) - 1], code_bits=c["bits"])
    out2 = vq_attend(q, kc2, Ck, vc2, Cv, workspace=attend_workspace(q, kc2, window), **kw)
    out3 = vq_attend(q, kc2, Ck, vc2, Cv, workspace=attend_workspace(q, kc2, window), **kw)
    torch.cuda.synchronize()
    print(f"[step] two runs of vq_attend bit-identical: {torch.equal(out2, out3)}; "
          f"fused step bit-identical to the two calls: {torch.equal(out, out2)}")
    return (kc.cpu().numpy(), vc.cpu().numpy(), out.cpu().numpy(),
            kc2.cpu().numpy(), vc2.cpu().numpy(), out2.cpu().numpy())


def unpacked(codes, bits):
    return codes if bits == 8 else O.unpack_nibbles(codes)


@pytest.mark.parametrize("name,B,Hq,Hkv,S_cap,lens,bits,n_c,smooth_rows,transform,causal,window", [
    # the decode workload's shape family: GQA 4, ragged lengths, an empty row and a row
    # holding only the new token
    ("gqa4", 4, 8, 2, 32768, [32768, 1, 20001, 0], 8, 256, 2, True, True, 0),
    # 8 query heads per kv head: two units per (row, kv head), both holding the new key
    ("gqa8", 4, 16, 2, 32768, [30000, 17, 25000, 9999], 8, 256, 1, True, True, 0),
    # 4-bit codes, 16 centroids
    ("4bit", 4, 8, 2, 32768, [32768, 5, 12345, 32000], 4, 16, 2, True, True, 0),
    # sliding window (enough units for the streaming kernel), no rotation, no smoothing,
    # fewer centroids than 256
    ("window", 16, 32, 8, 32768, [32768, 2, 20001, 4097] + [30000] * 12, 8, 200, 0, False, True, 4096),
    # many short units: segments of fewer than 16 blocks hold the new key (their first
    # loads wait for its codes)
    ("short", 16, 32, 8, 4096, None, 8, 256, 8, True, False, 0),
])
def test_decode_step(name, B, Hq, Hkv, S_cap, lens, bits, n_c, smooth_rows, transform, causal, window):
    if lens is None:
        lens = np.random.default_rng(7).integers(1, 1500, size=B).tolist()
        lens[3] = S_cap
    c = step_case(sum(map(ord, name)), B, Hq, Hkv, S_cap, lens, bits, n_c, smooth_rows, transform)
    assert vq_attend_path(B, Hq, 1, 128, 8, 4, n_c, Hkv, S_cap, window, code_bits=bits,
                          transform=int(transform)) == "stream"
    kc, vc, out, kc2, vc2, out2 = run_step(c, causal, window)
    # the two-call form: every slot of both caches byte for byte, the output
    # within the attention bar
    assert np.array_equal(kc, kc2), f"{name}: key cache differs from vq_encode_kv's"
    assert np.array_equal(vc, vc2), f"{name}: value cache differs from vq_encode_kv's"
    check_attn(out, out2.astype(np.float64), f"step {name} against vq_encode_kv + vq_attend")
    # the appended codes against the oracle's encode
    rows = [b for b, L in enumerate(lens) if L >= 1]
    got_k = np.stack([unpacked(kc[b:b + 1, :, lens[b] - 1:lens[b]], bits)[0] for b in rows])
    got_v = np.stack([unpacked(vc[b:b + 1, :, lens[b] - 1:lens[b]], bits)[0] for b in rows])
    check_codes(c["k_new"][rows], c["k_codebook"], 8, c["smooth_full"], transform, got_k, f"step {name} keys")
    check_codes(c["v_new"][rows], c["v_codebook"], 4, None, False, got_v, f"step {name} values")
    # sampled output rows against the oracle over the updated caches
    sample = [(b, h) for b in range(B) for h in (0, Hq - 1)][:8]   # new-key aligned and random heads
    ref = O.attend(c["q"], unpacked(kc, bits), c["k_codebook"], unpacked(vc, bits), c["v_codebook"],
                   scale=c["scale"], causal=causal, sliding_window=window, smooth=c["smooth_full"],
                   transform=transform, kv_lens=c["kv_lens"], rows=sample)
    for b, h in sample:
        check_attn(out[b, h], ref[b, h], f"step {name} row ({b}, {h})")


def test_decode_step_unsupported_shape():
    """Shapes off the streaming kernel are rejected (the caller uses
    vq_encode_kv and vq_attend), and the caches are left untouched."""
    from vector_quantized_kv_amd import VQError
    c = step_case(3, 2, 8, 2, 64, [64, 10], 8, 256, 2, True)
    kc = dev(c["k_codes"])
    before = kc.cpu().numpy()
    with pytest.raises(VQError):
        vq_decode_step(dev(c["q"]), dev(c["k_new"]), dev(c["v_new"]), kc, dev(c["k_codebook"]),
                       dev(c["v_codes"]), dev(c["v_codebook"]), scale=c["scale"], smooth=dev(c["smooth"]),
                       kv_lens=dev(c["kv_lens"]))
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), before)


@pytest.mark.parametrize("seed", range(6))
def test_decode_step_random_shapes(seed):
    """Random shapes on the streaming kernel: batch size, kv heads, query
    heads per kv head (1, 2: padded units; 8: two units per kv head), 8- or
    4-bit codes, windows, causal or not, smoothing rows, ragged lengths with
    empty and one-token rows.  Caches byte-equal to the two calls, outputs
    within the attention bar of them and, on sampled rows, of the oracle."""
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(2, 7))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    bits = int(rng.choice([8, 4]))
    n_c = 16 if bits == 4 else int(rng.choice([256, 97]))
    U = B * Hkv * ((G + 3) // 4)
    need = -(-(1 << 18) // U)          # keys per unit for the streaming kernel
    S_cap = max(2048, 2 * need)
    # odd seeds: a sliding window, long enough for the streaming kernel
    window = int(rng.integers(need, S_cap)) if seed % 2 else 0
    causal = bool(rng.integers(0, 2))
    lens = rng.integers(0, S_cap + 1, size=B)
    lens[0] = S_cap
    lens[1] = int(rng.choice([0, 1]))
    smooth_rows = int(rng.choice([0, 1, Hkv]))
    transform = bool(rng.integers(0, 2))
    c = step_case(6000 + seed, B, G * Hkv, Hkv, S_cap, lens.tolist(), bits, n_c, smooth_rows, transform)
    print(f"[step] random {seed}: B={B} H_kv={Hkv} G={G} bits={bits} n_c={n_c} S_cap={S_cap} W={window} "
          f"causal={causal} smooth_rows={smooth_rows} transform={transform} lens={lens.tolist()}")
    assert vq_attend_path(B, G * Hkv, 1, 128, 8, 4, n_c, Hkv, S_cap, window, code_bits=bits,
                          transform=int(transform)) == "stream"
    kc, vc, out, kc2, vc2, out2 = run_step(c, causal, window)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2), "caches differ from vq_encode_kv's"
    check_attn(out, out2.astype(np.float64), f"random {seed} against the two calls")
    rows = [b for b, L in enumerate(lens) if L >= 1]
    got_k = np.stack([unpacked(kc[b:b + 1, :, lens[b] - 1:lens[b]], bits)[0] for b in rows])
    got_v = np.stack([unpacked(vc[b:b + 1, :, lens[b] - 1:lens[b]], bits)[0] for b in rows])
    check_codes(c["k_new"][rows], c["k_codebook"], 8, c["smooth_full"], transform, got_k, f"random {seed} keys")
    check_codes(c["v_new"][rows], c["v_codebook"], 4, None, False, got_v, f"random {seed} values")
    sample = [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 6), rng.integers(0, G * Hkv, 6))]
    ref = O.attend(c["q"], unpacked(kc, bits), c["k_codebook"], unpacked(vc, bits), c["v_codebook"],
                   scale=c["scale"], causal=causal, sliding_window=window, smooth=c["smooth_full"],
                   transform=transform, kv_lens=c["kv_lens"], rows=sample)
    for b, h in sample:
        check_attn(out[b, h], ref[b, h], f"random {seed} row ({b}, {h})")


def test_decode_step_graph_capture():
    """vq_decode_step captured in a HIP graph (one launch of the streaming
    kernel with the append, then the merge) and replayed with new inputs,
    eager calls between the replays: each replay writes the eager codes and
    matches the eager output (within the attention bar) and the oracle."""
    from test_gpu_parity import oracle_attend, small_case
    c = small_case(411, B=4, Hq=32, Hkv=8, Sq=1, D=128, dk=8, dv=4, S_cap=8192)
    c["kv_lens"] = np.array([8192, 6000, 77, 8000], np.int32)
    kc, vc = dev(c["k_codes"]), dev(c["v_codes"])
    kb, vb, sm, kl = dev(c["k_codebook"]), dev(c["v_codebook"]), dev(c["smooth"]), dev(c["kv_lens"])
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
        vq_decode_step(q, kn, vn, kc, kb, vc, vb, scale=c["scale"], smooth=sm, kv_lens=kl, causal=True,
                       out=out, workspace=ws)

    new_inputs(0)
    step()                                   # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        new_inputs(20 + rep)
        g.replay()
        torch.cuda.synchronize()
        got, gk, gv = out.clone(), kc.clone(), vc.clone()
        step()                               # eager, same inputs (rewrites the same slots)
        torch.cuda.synchronize()
        assert torch.equal(gk, kc) and torch.equal(gv, vc), f"replay {rep}: codes differ from eager"
        check_attn(got.cpu().numpy(), out.cpu().numpy().astype(np.float64), f"step graph replay {rep} vs eager")
        p = dict(c, q=q.cpu().numpy())
        check_attn(got.cpu().numpy(), oracle_attend(p, kc.cpu().numpy(), vc.cpu().numpy()),
                   f"step graph replay {rep}")
        # the appended slots hold the oracle's codes of this replay's tokens
        for b, L in enumerate(c["kv_lens"]):
            check_codes(kn[b:b + 1].cpu().numpy(), c["k_codebook"], 8, c["smooth"], True,
                        kc[b:b + 1, :, L - 1:L].cpu().numpy(), f"graph replay {rep} keys row {b}")
