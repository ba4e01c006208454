"""vq_attend_noalloc (split partials in the library's per-GPU scratch array)
against vq_attend with a caller's workspace and against the oracle, on
consecutive calls of decreasing size (the array keeps the previous call's
contents, which must not matter)."""
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import (VQError, synth, vq_attend, vq_attend_noalloc,
                                     vq_attend_path, vq_attend_workspace_bytes)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCRATCH_BYTES = 16 << 20


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def make_case(seed, B, Hq, Hkv, Sq, S_cap, lens, window=0):
    rng = np.random.default_rng(seed)
    D, dk, dv = 128, 8, 4
    return dict(B=B, H_q=Hq, H_kv=Hkv, S_q=Sq, D=D, dk=dk, dv=dv, S_cap=S_cap,
                q=synth.outlier_normal(rng, (B, Hq, Sq, D), 4),
                k_codes=synth.uniform_codes(rng, (B, Hkv, S_cap, D // dk)),
                v_codes=synth.uniform_codes(rng, (B, Hkv, S_cap, D // dv)),
                k_codebook=synth.normal_codebook(rng, 256, dk),
                v_codebook=synth.normal_codebook(rng, 256, dv),
                smooth=rng.uniform(0.5, 5, size=(Hkv, D)).astype(np.float32),
                kv_lens=np.array(lens, np.int32), scale=1 / math.sqrt(D), causal=True,
                window=window)


def close(a, ref):
    a = np.asarray(a, np.float64)
    err = np.abs(a - ref)
    return not np.isnan(a).any() and bool(np.all(err <= 2e-3 + 1e-2 * np.abs(ref))), err.max()


def test_noalloc_matches_vq_attend():
    cases = [
        make_case(501, 16, 32, 8, 1, 8192, np.random.default_rng(1).integers(1, 8193, 16)),  # stream
        make_case(502, 4, 32, 8, 1, 8192, [8192, 5000, 0, 77]),                               # smaller
        make_case(503, 1, 8, 8, 1, 2048, [2048]),                                             # per-unit
    ]
    paths = []
    for i, c in enumerate(cases):
        path = vq_attend_path(c["B"], c["H_q"], c["S_q"], c["D"], c["dk"], c["dv"], 256, c["H_kv"],
                              c["S_cap"], c["window"])
        paths.append(path)
        need = vq_attend_workspace_bytes(c["B"], c["H_q"], c["S_q"], c["D"], c["H_kv"], c["S_cap"],
                                         c["window"])
        assert 0 < need <= SCRATCH_BYTES
        args = (dev(c["q"]), dev(c["k_codes"]), dev(c["k_codebook"]), dev(c["v_codes"]),
                dev(c["v_codebook"]))
        kw = dict(scale=c["scale"], smooth=dev(c["smooth"]), kv_lens=dev(c["kv_lens"]),
                  causal=True, sliding_window=c["window"])
        with_ws = vq_attend(*args, **kw)
        out = torch.full_like(with_ws, float("nan"))
        vq_attend_noalloc(*args, out=out, **kw)
        torch.cuda.synchronize()
        got, base = out.cpu().numpy(), with_ws.cpu().numpy().astype(np.float64)
        ok, err = close(got, base)
        assert ok, f"call {i} ({path}): differs from vq_attend by up to {err:.3g}"
        ref = O.attend(c["q"], c["k_codes"], c["k_codebook"], c["v_codes"], c["v_codebook"],
                       scale=c["scale"], causal=True, sliding_window=c["window"], smooth=c["smooth"],
                       transform=True, kv_lens=c["kv_lens"])
        ok, err = close(got, ref)
        assert ok, f"call {i} ({path}): differs from the oracle by up to {err:.3g}"
        print(f"[noalloc] call {i} ({path}, {need} B of partials): max err vs oracle {err:.3g}")
    assert paths[0] == "stream" and paths[1] == "stream" and paths[2] == "lut_mfma"


def test_noalloc_rejects_shapes_beyond_the_scratch_array():
    p = synth.prefill()
    need = vq_attend_workspace_bytes(4, 8, 512, 128, 8, 32768, 0)
    assert need > SCRATCH_BYTES
    with pytest.raises(VQError, match="scratch"):
        vq_attend_noalloc(dev(p["q"]), dev(p["k_codes"]), dev(p["k_codebook"]), dev(p["v_codes"]),
                          dev(p["v_codebook"]), scale=p["scale"], smooth=dev(p["smooth"]),
                          kv_lens=dev(p["kv_lens"]))
