"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol declared in include/vq.h, and rejects invalid arguments before any
HIP call.  Valid calls on a host without a device return VQ_ERR_NO_DEVICE."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from vector_quantized_kv_amd import _lib, api
from vector_quantized_kv_amd.build import build_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vq.h")
OK, INVALID, UNSUPPORTED, NO_DEVICE, HIPERR, WORKSPACE = range(6)
P = ctypes.c_void_p(0x10000)          # a non-null, aligned pointer that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        build_library(verbose=False)
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vq_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = header_functions()
    for n in ["vq_encode", "vq_decode", "vq_encode_decode", "vq_encode_kv", "vq_attend",
              "vq_attend_workspace_bytes", "vq_supports_shape", "vq_status_string", "vq_last_error"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (vq_\w+)", out))
    for n in header_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(header_functions()) == set(_lib.SIGNATURES)


def test_status_strings(lib):
    assert lib.vq_status_string(OK) == b"ok"
    assert b"invalid" in lib.vq_status_string(INVALID)
    assert lib.vq_status_string(99) == b"unknown status"
    assert lib.vq_version() >= 100


@pytest.mark.parametrize("n_c,n_sub,D,ok", [
    (256, 16, 128, 1), (256, 16, 64, 1), (256, 32, 128, 1), (1, 64, 256, 1), (16, 32, 32, 1),
    (257, 16, 128, 0), (0, 16, 128, 0), (256, 16, 96, 0), (256, 128, 128, 0), (256, 5, 128, 0),
    (256, 4, 128, 0), (256, 16, 512, 0)])
def test_supports_shape(lib, n_c, n_sub, D, ok):
    assert lib.vq_supports_shape(n_c, n_sub, D) == ok


def enc(lib, B=1, H=2, S=8, D=64, n_c=256, dsub=4, smooth=P, srows=2, transform=1, S_cap=8,
        S_off=0, offs=None, keys=P, cb=P, codes=P, bits=8, mat=None, mat_inv=None):
    return lib.vq_encode(keys, B, H, S, D, cb, n_c, dsub, bits, smooth, srows, transform, mat, mat_inv,
                         codes, S_cap, S_off, offs, None)


def test_encode_validation(lib):
    assert enc(lib, keys=None) == INVALID
    assert enc(lib, codes=None) == INVALID
    assert enc(lib, D=64, dsub=3) == INVALID            # D % sub_dim
    assert enc(lib, n_c=300) == INVALID                 # does not fit uint8
    assert enc(lib, n_c=0) == INVALID
    assert enc(lib, srows=3) == INVALID                 # smooth rows not 1 or H
    assert enc(lib, transform=3) == INVALID
    assert enc(lib, transform=2) == INVALID            # the matrix is missing
    assert b"mat" in lib.vq_last_error()
    assert enc(lib, transform=2, mat=P, D=256, dsub=8, S=0) == UNSUPPORTED   # head dim above 128
    assert enc(lib, transform=2, mat=P, S=0) == OK
    assert enc(lib, S_off=4) == INVALID                 # 4 + 8 > 8
    assert enc(lib, S_off=-1) == INVALID
    assert enc(lib, H=0) == INVALID
    assert enc(lib, B=1 << 16, H=1 << 8, S=1 << 7, S_cap=1 << 7) == INVALID   # 2^31 token-heads
    assert b"2^31" in lib.vq_last_error()
    assert enc(lib, D=96, dsub=4) == UNSUPPORTED        # head dim cap
    assert enc(lib, D=128, dsub=1) == UNSUPPORTED       # 128 sub-vectors > 64
    offs = (ctypes.c_int32 * 2)(0, 5)
    assert enc(lib, B=2, S=4, offs=offs) == INVALID     # row 1 writes [5, 9)
    assert b"row 1" in lib.vq_last_error()
    assert enc(lib, B=257, offs=(ctypes.c_int32 * 257)()) == INVALID   # too many rows
    assert enc(lib, B=0) in (OK,)                       # empty: no-op
    assert enc(lib, S=0) in (OK,)
    # 4-bit codes: at most 16 centroids, an even number of sub-vectors
    assert enc(lib, bits=5) == INVALID
    assert enc(lib, bits=4, n_c=17) == INVALID
    assert b"16 centroids" in lib.vq_last_error()
    assert enc(lib, bits=4, n_c=16, D=32, dsub=16, S=0) == OK   # valid, empty: no launch


def test_decode_and_encode_decode_validation(lib):
    st = lib.vq_encode_decode(P, 1, 2, 8, 64, P, 256, 4, 8, P, 2, 1, None, None, P, 8, 0, None, None, 1,
                              None)
    assert st == INVALID                                # recon NULL
    st = lib.vq_encode_decode(P, 1, 2, 8, 64, P, 256, 4, 8, P, 2, 1, None, None, P, 8, 0, None, P, 7, None)
    assert st == INVALID                                # out_dtype
    st = lib.vq_encode_decode(P, 1, 2, 8, 64, P, 256, 4, 8, P, 2, 2, P, None, P, 8, 0, None, P, 1, None)
    assert st == INVALID                                # transform 2 needs mat_inv for the recon
    st = lib.vq_decode(P, 1, 2, 8, 8, 1, P, 256, 4, 8, None, 1, 1, None, None, 64, P, 0, None)
    assert st == INVALID                                # slots [1, 9) outside [0, 8)
    st = lib.vq_decode(P, 1, 2, 8, 8, 0, P, 256, 4, 8, None, 1, 1, None, None, 48, P, 0, None)
    assert st == UNSUPPORTED                            # D = 48
    st = lib.vq_decode(None, 1, 2, 8, 8, 0, P, 256, 4, 8, None, 1, 1, None, None, 64, P, 0, None)
    assert st == INVALID
    st = lib.vq_decode(P, 1, 2, 8, 8, 0, P, 32, 4, 4, None, 1, 1, None, None, 64, P, 0, None)
    assert st == INVALID                                # 4-bit codes, 32 centroids
    st = lib.vq_decode(P, 1, 2, 8, 8, 0, P, 256, 4, 8, None, 1, 2, P, None, 64, P, 0, None)
    assert st == INVALID                                # decode reads mat_inv
    st = lib.vq_decode(P, 1 << 16, 1 << 8, 1 << 7, 1 << 7, 0, P, 256, 4, 8, None, 1, 1, None, None, 64, P, 0,
                       None)
    assert st == INVALID and b"2^31" in lib.vq_last_error()   # 2^31 token-heads


def enc_kv(lib, B=1, H=2, S=8, D=128, dk=8, dv=4, nk=256, nv=256, S_cap=8, S_off=0, offs=None,
           keys=P, values=P, kcb=P, vcb=P, kc=P, vc=P, smooth=P, srows=2, transform=1, bits=8):
    return lib.vq_encode_kv(keys, values, B, H, S, D, kcb, nk, dk, smooth, srows, transform, None, None,
                            vcb, nv, dv, bits, kc, vc, S_cap, S_off, offs, None)


def test_encode_kv_validation(lib):
    assert enc_kv(lib, values=None) == INVALID
    assert enc_kv(lib, vc=None) == INVALID
    assert enc_kv(lib, dv=3) == INVALID                 # D % value sub_dim
    assert enc_kv(lib, nv=300) == INVALID               # value codes do not fit uint8
    assert enc_kv(lib, dk=1) == UNSUPPORTED             # 128 key sub-vectors
    assert enc_kv(lib, srows=3) == INVALID
    assert enc_kv(lib, S_off=1) == INVALID              # [1, 9) outside [0, 8)
    offs = (ctypes.c_int32 * 2)(0, 6)
    assert enc_kv(lib, B=2, S=4, offs=offs) == INVALID  # row 1 writes [6, 10)
    assert enc_kv(lib, S=0) == OK
    assert enc_kv(lib, B=0) == OK
    assert enc_kv(lib, bits=4, nk=16, nv=17) == INVALID  # value codebook too large for 4 bits
    if not torch.cuda.is_available():
        assert enc_kv(lib) == NO_DEVICE


def att(lib, B=2, Hq=8, Sq=1, D=128, dk=8, dv=4, n_c=256, Hkv=2, S_cap=64, W=0, causal=1,
        ws=P, ws_bytes=1 << 30, smooth=P, srows=2, scale=0.1, q=P, bits=8, transform=1, mat=None,
        mat_inv=None):
    return lib.vq_attend(q, B, Hq, Sq, D, P, P, dk, smooth, srows, transform, mat, mat_inv, P, P, dv, n_c,
                         bits, Hkv, S_cap, None, scale, causal, W, P, ws, ws_bytes, None)


def test_attend_validation(lib):
    assert att(lib, q=None) == INVALID
    assert att(lib, Hq=6, Hkv=4) == INVALID              # H_q % H_kv
    assert att(lib, dk=3) == INVALID                     # D % sub_dim
    assert att(lib, W=-1) == INVALID
    assert att(lib, causal=2) == INVALID
    assert att(lib, srows=3) == INVALID
    assert att(lib, scale=float("inf")) == INVALID
    assert att(lib, D=96) == UNSUPPORTED
    assert att(lib, D=32, dk=16) == UNSUPPORTED          # 2 key sub-vectors: not a multiple of 4
    assert att(lib, ws=None) == WORKSPACE
    assert att(lib, ws_bytes=16) == WORKSPACE
    assert b"workspace needs" in lib.vq_last_error()
    assert att(lib, B=0) == OK
    assert att(lib, bits=4) == INVALID                   # 256 centroids in 4 bits
    assert att(lib, bits=4, n_c=16, D=64, dk=16) == INVALID   # 4 key sub-vectors: not a multiple of 8
    assert att(lib, transform=2, mat=P) == INVALID       # the query needs mat_inv
    assert att(lib, transform=2, mat_inv=P, B=0) == OK


def step(lib, B=16, Hq=32, D=128, dk=8, dv=4, n_c=256, Hkv=8, S_cap=32768, W=0, causal=1, ws=P,
         ws_bytes=1 << 30, smooth=P, srows=8, bits=8, transform=1, kn=P, vn=P, lens=P):
    return lib.vq_decode_step(P, kn, vn, B, Hq, D, P, P, dk, smooth, srows, transform, P, P, dv, n_c, bits,
                              Hkv, S_cap, lens, 0.1, causal, W, P, ws, ws_bytes, None)


def test_decode_step_validation(lib):
    assert step(lib, kn=None) == INVALID
    assert step(lib, vn=None) == INVALID
    assert step(lib, lens=None) == INVALID                # the lengths after the append are required
    assert b"kv_lens" in lib.vq_last_error()
    assert step(lib, Hq=30) == INVALID                    # H_q % H_kv, as vq_attend
    assert step(lib, dk=4) == UNSUPPORTED                 # key sub_dim other than 8
    assert b"vq_encode_kv and vq_attend" in lib.vq_last_error()
    assert step(lib, S_cap=64) == UNSUPPORTED             # too few keys for the streaming kernel
    assert step(lib, D=64) == UNSUPPORTED
    assert step(lib, ws_bytes=16) == WORKSPACE
    assert step(lib, B=0) == OK
    if not torch.cuda.is_available():
        assert step(lib) == NO_DEVICE                     # valid: stops at the device check
        assert step(lib, bits=4, n_c=16, transform=0) == NO_DEVICE


@pytest.mark.skipif(torch.cuda.is_available(), reason="a device is visible")
def test_valid_calls_report_no_device(lib):
    assert enc(lib) == NO_DEVICE
    assert att(lib) == NO_DEVICE
    assert b"no HIP device" in lib.vq_last_error()


def test_workspace_bytes(lib):
    f = lib.vq_attend_workspace_bytes
    assert f(0, 8, 1, 128, 8, 1024, 0) == 0
    assert f(1, 6, 1, 128, 4, 1024, 0) == 0              # H_q % H_kv
    a = f(16, 32, 1, 128, 8, 32768, 0)
    b = f(16, 32, 1, 128, 8, 32768, 4096)
    assert a > 0 and b > 0
    # head dim 128 may run on the persistent kernel: one partial of 4 rows x
    # (128 + 2) floats per (chunk, unit) pair, 4096 chunks + 128 units here
    assert a >= (4096 + 16 * 8) * 4 * (128 + 2) * 4
    assert a == f(16, 32, 1, 128, 8, 32768, 0)            # a pure function of the shape
    # other head dims: (D + 2) floats per split partial, rows rounded up to 8,
    # then (256-byte aligned) the fp32 query rows an explicit transform matrix uses
    c = f(16, 32, 1, 64, 8, 32768, 0)
    q_rows = 16 * 32 * 1 * 64 * 4
    assert c > q_rows and (c - q_rows) % 256 == 0
    assert (c - q_rows) >= (64 + 2) * 4 * 16 * 8 * 8


def test_binding_rejects_host_tensors(lib):
    k = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    cb = torch.zeros(256, 4)
    with pytest.raises(ValueError, match="device tensor"):
        api.vq_encode(k, cb, 4)
    with pytest.raises(ValueError, match="fp16|float16"):
        api.vq_encode(k.float(), cb, 4)


@pytest.mark.parametrize("shape,path", [
    # (B, H_q, S_q, D, d_k, d_v, n_c, H_kv, S_cap, W): the benchmarked workloads
    ((16, 32, 1, 128, 8, 4, 256, 8, 32768, 0), "stream"),      # GQA decode step
    ((16, 32, 1, 128, 8, 4, 256, 8, 32768, 4096), "stream"),   # GQA decode, window 4096
    ((1, 8, 1, 128, 8, 4, 256, 8, 8192, 0), "lut_mfma"),       # single-query decode
    ((4, 8, 512, 128, 8, 4, 256, 8, 32768, 0), "tile"),        # prefill chunk
    # at the streaming threshold (2^18 unit-keys) and just below it
    ((4, 32, 1, 128, 8, 4, 256, 8, 8192, 0), "stream"),
    ((4, 8, 2, 128, 8, 4, 256, 8, 8192, 8191), "stream"),
    ((4, 8, 2, 128, 8, 4, 256, 8, 8192, 8190), "lut_mfma"),
    ((2, 32, 1, 128, 8, 4, 256, 8, 8192, 0), "lut_mfma"),
    # 64 query rows per kv head start the tile kernel
    ((3, 2, 64, 128, 8, 4, 256, 2, 400, 0), "tile"),
    ((3, 2, 63, 128, 8, 4, 256, 2, 400, 0), "lut_mfma"),
    # other sub-vector sizes and head dims
    ((1, 8, 1, 128, 8, 8, 256, 8, 300, 0), "lut_valu"),
    ((1, 8, 1, 64, 4, 4, 256, 8, 300, 0), "lut_mfma"),
    ((1, 8, 1, 64, 16, 4, 16, 8, 300, 0), "lut_valu"),         # 4 key sub-vectors
    ((1, 8, 1, 256, 4, 16, 256, 8, 300, 0), "lut_valu"),
])
def test_attend_path_routing(lib, shape, path):
    """vq_attend's kernel choice depends on the shape only; these pins keep
    the benchmarked and tested shapes on the kernels they are meant for."""
    assert api.vq_attend_path(*shape) == path


def test_attend_path_rejects_what_attend_rejects(lib):
    with pytest.raises(api.VQError):
        api.vq_attend_path(1, 6, 1, 128, 8, 4, 256, 4, 100)      # H_q % H_kv != 0
    with pytest.raises(api.VQError):
        api.vq_attend_path(1, 8, 1, 128, 6, 4, 256, 8, 100)      # D % d_k != 0
    with pytest.raises(api.VQError):
        api.vq_attend_path(1, 8, 1, 128, 8, 4, 257, 8, 100)      # more than 256 centroids
    assert lib.vq_attend_path(0, 8, 1, 128, 8, 4, 256, 8, 1, 8, 100, 0) == 0
    # explicit transform matrices: the streaming and per-unit VALU kernels only
    assert api.vq_attend_path(4, 8, 512, 128, 8, 4, 256, 8, 32768, transform=2) == "lut_valu"
    assert api.vq_attend_path(16, 32, 1, 128, 8, 4, 256, 8, 32768, transform=2) == "stream"
    with pytest.raises(api.VQError):
        api.vq_attend_path(1, 8, 1, 256, 8, 4, 256, 8, 300, transform=2)
    with pytest.raises(api.VQError):
        api.vq_attend_path(1, 8, 1, 128, 8, 4, 17, 8, 100, code_bits=4)    # 17 centroids in 4 bits


def test_binding_rejects_wrong_shapes(lib):
    """The C ABI receives bare pointers and sizes, so the binding checks every
    buffer's shape against the others before any call (host tensors here:
    the shape checks come before the device check)."""
    f16, f32, u8, i32 = torch.float16, torch.float32, torch.uint8, torch.int32
    k = torch.zeros(2, 3, 8, 64, dtype=f16)
    cb = torch.zeros(256, 4)
    cases = [
        (lambda: api.vq_encode(k, cb, 4, codes=torch.zeros(2, 3, 8, 8, dtype=u8)), "codes"),
        (lambda: api.vq_encode(k, cb, 4, codes=torch.zeros(1, 3, 8, 16, dtype=u8)), "codes"),
        (lambda: api.vq_encode(k, cb, 4, codes=torch.zeros(2, 3, 8, 16, dtype=u8), S_cap=9), "codes"),
        (lambda: api.vq_encode(k, torch.zeros(256, 8), 4), "codebook"),
        (lambda: api.vq_encode(k, cb, 3), "divide"),
        (lambda: api.vq_encode(k, cb, 4, smooth=torch.zeros(3, 32)), "smooth"),
        (lambda: api.vq_encode(k, cb, 4, smooth=torch.zeros(2, 64)), "smooth"),
        (lambda: api.vq_encode(k, cb, 4, row_offsets=[0]), "row_offsets"),
        (lambda: api.vq_encode_decode(k, cb, 4, recon=torch.zeros(2, 3, 7, 64, dtype=f16)), "recon"),
        (lambda: api.vq_encode_decode(k, cb, 4, recon=torch.zeros(2, 3, 8, 64, dtype=torch.float64)),
         "recon"),
        (lambda: api.vq_decode(torch.zeros(2, 3, 8, 16, dtype=u8), cb, S=4,
                               out=torch.zeros(2, 3, 5, 64)), "out"),
        (lambda: api.vq_decode(torch.zeros(2, 3, 8, 16, dtype=u8), cb,
                               out=torch.zeros(2, 3, 64, 8).transpose(2, 3)), "out"),
        (lambda: api.vq_encode_kv(k, torch.zeros(2, 3, 8, 32, dtype=f16), cb, 4, cb, 4), "values"),
        (lambda: api.vq_encode_kv(k, k, cb, 4, cb, 4, k_codes=torch.zeros(2, 3, 8, 16, dtype=u8),
                                  v_codes=torch.zeros(2, 3, 9, 16, dtype=u8)), "v_codes"),
    ]
    q = torch.zeros(2, 8, 1, 64, dtype=f16)
    kc = torch.zeros(2, 4, 100, 16, dtype=u8)
    att_kw = dict(scale=0.1)
    cases += [
        (lambda: api.vq_attend(q, torch.zeros(3, 4, 100, 16, dtype=u8), cb, kc, cb, **att_kw), "k_codes"),
        (lambda: api.vq_attend(q, torch.zeros(2, 4, 100, 8, dtype=u8), cb, kc, cb, **att_kw), "k_codes"),
        (lambda: api.vq_attend(q, kc, cb, torch.zeros(2, 4, 99, 16, dtype=u8), cb, **att_kw), "v_codes"),
        (lambda: api.vq_attend(q, kc, cb, kc, cb, kv_lens=torch.zeros(3, dtype=i32), **att_kw),
         "kv_lens"),
        (lambda: api.vq_attend(q, kc, cb, kc, cb, out=torch.zeros(2, 8, 1, 32, dtype=f16), **att_kw),
         "out"),
        (lambda: api.vq_attend(q, kc, cb, kc, cb, smooth=torch.zeros(4, 65), **att_kw), "smooth"),
        (lambda: api.vq_attend(q, kc, cb, kc, torch.zeros(100, 4), **att_kw), "n_centroids"),
        (lambda: api.vq_attend(q, kc, cb, kc, cb, workspace=torch.zeros(4, 4, dtype=u8), **att_kw),
         "workspace"),
    ]
    for i, (fn, what) in enumerate(cases):
        with pytest.raises(ValueError, match=what):
            fn()
    # consistent shapes get as far as the device check
    with pytest.raises(ValueError, match="device tensor"):
        api.vq_attend(q, kc, cb, kc, cb, kv_lens=torch.zeros(2, dtype=i32),
                      out=torch.zeros(2, 8, 1, 64, dtype=f16), workspace=torch.zeros(16, dtype=u8),
                      smooth=torch.zeros(4, 64), **att_kw)
    # the fused decode step: new tokens [B, H_kv, 1, D], one query position, lengths required
    kn = torch.zeros(2, 4, 1, 64, dtype=f16)
    lens = torch.zeros(2, dtype=i32)
    step_cases = [
        (lambda: api.vq_decode_step(q, torch.zeros(2, 4, 2, 64, dtype=f16), kn, kc, cb, kc, cb, kv_lens=lens,
                                    **att_kw), "k_new"),
        (lambda: api.vq_decode_step(q, kn, torch.zeros(2, 3, 1, 64, dtype=f16), kc, cb, kc, cb, kv_lens=lens,
                                    **att_kw), "v_new"),
        (lambda: api.vq_decode_step(q, kn, kn.float(), kc, cb, kc, cb, kv_lens=lens, **att_kw), "v_new"),
        (lambda: api.vq_decode_step(q, kn, kn, kc, cb, kc, cb, kv_lens=None, **att_kw), "kv_lens"),
        (lambda: api.vq_decode_step(torch.zeros(2, 8, 2, 64, dtype=f16), kn, kn, kc, cb, kc, cb, kv_lens=lens,
                                    **att_kw), "S_q"),
        (lambda: api.vq_decode_step(q, kn, kn, kc, cb, torch.zeros(2, 4, 99, 16, dtype=u8), cb,
                                    kv_lens=lens, **att_kw), "v_codes"),
    ]
    for fn, what in step_cases:
        with pytest.raises(ValueError, match=what):
            fn()
    with pytest.raises(ValueError, match="device tensor"):
        api.vq_decode_step(q, kn, kn, kc, cb, kc, cb, kv_lens=lens, workspace=torch.zeros(16, dtype=u8),
                           **att_kw)


def test_attend_noalloc_validation(lib):
    """vq_attend_noalloc validates like vq_attend, and rejects shapes whose
    partials exceed its device scratch array before touching a device."""
    f = lib.vq_attend_noalloc
    args = lambda B=2, Hq=8, Sq=1, q=P: (q, B, Hq, Sq, 128, P, P, 8, P, 2, 1, None, None, P, P, 4, 256, 8,
                                         2, 64, None, 0.1, 1, 0, P, None)
    assert f(*args(q=None)) == INVALID
    assert f(*args(Hq=7)) == INVALID                     # H_q % H_kv
    assert f(*args(B=0)) == OK
    st = f(P, 4, 8, 512, 128, P, P, 8, P, 8, 1, None, None, P, P, 4, 256, 8, 8, 32768, None, 0.1, 1, 0, P,
           None)
    assert st == WORKSPACE and b"scratch" in lib.vq_last_error()
    if not torch.cuda.is_available():
        assert f(*args()) == NO_DEVICE


def test_transform_validation(lib):
    f = lib.vq_transform
    args = lambda B=1, H=2, S=4, D=128, smooth=None, rows=1, tr=1, mat=None, keys=P, out=P: (
        keys, B, H, S, D, smooth, rows, tr, mat, out, None)
    assert f(*args(keys=None)) == INVALID
    assert f(*args(out=None)) == INVALID
    assert f(*args(H=0)) == INVALID
    assert f(*args(S=-1)) == INVALID
    assert f(*args(D=96)) == UNSUPPORTED
    assert f(*args(smooth=P, rows=3)) == INVALID                     # smooth_rows not in {1, H}
    assert f(*args(tr=2)) == INVALID and b"mat" in lib.vq_last_error()
    assert f(*args(tr=2, D=256, mat=P)) == UNSUPPORTED
    assert f(*args(tr=3)) == INVALID
    assert f(*args(out=ctypes.c_void_p(0x10004))) == INVALID        # misaligned
    assert f(*args(S=0)) == OK and f(*args(B=0)) == OK
    if not torch.cuda.is_available():
        assert f(*args()) == NO_DEVICE


def test_kmeans_validation(lib):
    f = lib.vq_kmeans
    need = lib.vq_kmeans_workspace_bytes(1 << 20, 8, 256)
    args = lambda v=P, N=1 << 20, d=8, C=P, n_c=256, it=4, ws=P, wsb=need: (
        v, N, d, C, n_c, it, None, None, ws, wsb, None)
    assert f(*args(N=-1)) == INVALID
    assert f(*args(d=3)) == UNSUPPORTED and f(*args(d=32)) == UNSUPPORTED
    assert f(*args(n_c=0)) == INVALID and f(*args(n_c=257)) == INVALID
    assert f(*args(it=-1)) == INVALID
    assert f(*args(C=None)) == INVALID and f(*args(v=None)) == INVALID
    assert f(*args(ws=ctypes.c_void_p(0x10008))) == INVALID         # misaligned
    assert f(*args(wsb=need - 1)) == WORKSPACE and b"workspace" in lib.vq_last_error()
    assert f(*args(ws=None)) == WORKSPACE
    assert f(*args(it=0)) == OK                                      # no-op
    if not torch.cuda.is_available():
        assert f(*args()) == NO_DEVICE
        assert f(*args(v=None, N=0, wsb=lib.vq_kmeans_workspace_bytes(0, 8, 256))) == NO_DEVICE


def test_kmeans_workspace_bytes(lib):
    """One fp64 row of n_c * (d + 1) + 1 accumulators per assignment
    workgroup: one workgroup per 4096 vectors, at most 256."""
    f = lib.vq_kmeans_workspace_bytes
    row = lambda d, n_c: (n_c * (d + 1) + 1) * 8
    assert f(0, 8, 256) == row(8, 256)
    assert f(4096, 8, 256) == row(8, 256)
    assert f(4097, 8, 256) == 2 * row(8, 256)
    assert f(1 << 20, 8, 256) == 256 * row(8, 256)
    assert f(1 << 30, 16, 16) == 256 * row(16, 16)
    assert f(-1, 8, 256) == 0 and f(10, 3, 256) == 0 and f(10, 8, 0) == 0 and f(10, 8, 257) == 0


def test_kmeans_binding_checks_shapes(lib):
    C = torch.zeros(16, 8)
    with pytest.raises(ValueError, match="vectors must be"):
        api.vq_kmeans(torch.zeros(100, 4), C, 1)
    with pytest.raises(ValueError, match="centroids must be"):
        api.vq_kmeans(torch.zeros(100, 8), torch.zeros(16, 8, dtype=torch.float64), 1)
    with pytest.raises(ValueError, match="labels must have shape"):
        api.vq_kmeans(torch.zeros(100, 8), C, 1, labels=torch.zeros(99, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor"):
        api.vq_kmeans(torch.zeros(100, 8), C, 1)
    with pytest.raises(ValueError, match="out must have shape"):
        api.vq_transform(torch.zeros(1, 2, 3, 64, dtype=torch.float16), out=torch.zeros(1, 2, 3, 32))
