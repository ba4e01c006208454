"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each `pin_*` checks the oracle against something the pages or mathematics
fix: hand-worked examples (tests/golden), closed forms, brute force on tiny
inputs, invariants, and special cases that reduce to a library routine
(torch's scaled_dot_product_attention on CPU in float64).  The mutation tests
at the end plant plausible mistakes in the oracle (on the CPU) and check
that at least one pin fails for each.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import synth
from conftest import read_golden


# ----------------------------------------------------------------------------
# Independent helpers (closed forms written here, not taken from the oracle)
# ----------------------------------------------------------------------------
def closed_form_hadamard(D):
    i = np.arange(D)[:, None]
    j = np.arange(D)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1.0, -1.0) / math.sqrt(D)


# ----------------------------------------------------------------------------
# Pins
# ----------------------------------------------------------------------------
def pin_hadamard_closed_form(o):
    for D in [1, 2, 4, 8, 16, 32, 64, 128, 256]:
        H = o.sylvester_hadamard(D)
        assert np.max(np.abs(H - closed_form_hadamard(D))) < 1e-15, D


def pin_hadamard_golden(o):
    g = read_golden("hadamard_sylvester_8.txt")["H8"].reshape(8, 8)
    assert np.array_equal(o.sylvester_hadamard(8) * math.sqrt(8), g)


def pin_hadamard_orthonormal(o):
    for D in [2, 16, 64, 128, 256]:
        H = o.sylvester_hadamard(D)
        assert np.allclose(H, H.T, atol=0, rtol=0)
        assert np.max(np.abs(H @ H - np.eye(D))) < 1e-12
        e0 = np.zeros((1, 1, 1, D))
        e0[..., 0] = 1
        assert np.allclose(o.forward_transform(e0, None, True), 1 / math.sqrt(D), atol=1e-15)


def pin_storage(o):
    rows = read_golden("storage_bytes.txt")[None].reshape(-1, 5).astype(int)
    for D, d, b, nbytes, entries in rows:
        assert o.code_bytes_per_token(D, d, b) == nbytes
        assert o.codebook_bytes(b, d, 1) == entries


def _golden_encode_inputs():
    g = read_golden("encode_worked_d4.txt")
    D, d = int(g["D"][0]), int(g["sub_dim"][0])
    keys = g["keys"].reshape(1, 1, -1, D)
    return g, D, d, keys, g["smooth"], g["codebook"].reshape(-1, d)


def pin_encode_golden(o):
    g, D, d, keys, s, C = _golden_encode_inputs()
    xt = o.forward_transform(keys, s, True)
    assert np.array_equal(xt.reshape(-1), g["transformed"])
    codes, _ = o.encode(keys, C, d, s, True)
    assert np.array_equal(codes.reshape(-1), g["codes"])
    rec = o.decode(codes, C, s, True)
    assert np.array_equal(rec.reshape(-1), g["recon"])
    # per-head smooth [H, D] gives the same result as the shared [D] form
    codes2, _ = o.encode(keys, C, d, s[None, :], True)
    assert np.array_equal(codes2, codes)


def pin_distances_and_gap_golden(o):
    """The squared-distance table and the near-tie gap against the hand-worked
    example: every sub-vector's distance to each centroid, and (d2 - d1) / d2
    from its two smallest distances (one exact tie, gaps of 0.8 and 8/13)."""
    g, D, d, keys, s, C = _golden_encode_inputs()
    xt = o.forward_transform(keys, s, True)
    dist = o.pvq_distances(xt, C, d)                              # [1, 1, 4, 2, 4]
    assert dist.shape == (1, 1, 4, 2, 4)
    assert np.array_equal(dist.reshape(-1), g["distances"])
    _, gap = o.encode(keys, C, d, s, True)
    want = g["gap_num"] / g["gap_den"]
    assert np.max(np.abs(gap.reshape(-1) - want)) < 1e-15


def pin_gap_bruteforce(o):
    """pvq_distances and the gap of pvq_encode against pure-Python loops on
    tiny inputs: every squared distance written out term by term, the two
    smallest found by a full sort, gap = (d2 - d1) / d2."""
    rng = np.random.default_rng(17)
    for D, d, nc in [(8, 2, 5), (12, 4, 7), (6, 3, 2)]:
        x = rng.standard_normal((1, 2, 3, D))
        C = rng.standard_normal((nc, d))
        dist = o.pvq_distances(x, C, d)
        _, gap = o.pvq_encode(x, C, d)
        for h in range(2):
            for t in range(3):
                for j in range(D // d):
                    ds = [sum((float(x[0, h, t, j * d + e]) - float(C[c, e])) ** 2 for e in range(d))
                          for c in range(nc)]
                    assert max(abs(a - b) for a, b in zip(ds, dist[0, h, t, j])) < 1e-12
                    srt = sorted(ds)
                    assert abs(gap[0, h, t, j] - (srt[1] - srt[0]) / srt[1]) < 1e-12


def pin_nibbles(o):
    """Nibble packing against the hand-worked bytes (low nibble = even
    element, masked to 4 bits), its inverse, and the storage formula at
    b = 4: D = 128, d = 8 gives 16 codes in 8 bytes per token and head."""
    g = read_golden("nibble_pack.txt")
    codes = g["codes"].astype(np.int64)
    packed = o.pack_nibbles(codes)
    assert packed.dtype == np.uint8 and packed.tolist() == g["packed"].astype(int).tolist()
    assert o.unpack_nibbles(packed).tolist() == g["unpacked"].astype(int).tolist()
    rng = np.random.default_rng(23)
    c = rng.integers(0, 16, size=(2, 3, 5, 16))
    p2 = o.pack_nibbles(c)
    assert p2.shape == (2, 3, 5, 8) and np.array_equal(o.unpack_nibbles(p2), c)
    assert p2.shape[-1] == o.code_bytes_per_token(128, 8, 4)


def pin_bruteforce(o):
    """Exhaustive search over whole code tuples equals the per-sub-vector
    argmin (product-VQ separability), with the rotation and smoothing
    computed here from the closed form."""
    rng = np.random.default_rng(7)
    for D, d, nc, transform in [(4, 2, 4, False), (4, 2, 4, True), (8, 4, 3, True), (6, 2, 3, False)]:
        keys = rng.standard_normal((1, 2, 12, D))
        s = rng.uniform(0.5, 2.0, size=(2, D))
        C = rng.standard_normal((nc, d))
        n_sub = D // d
        x = keys / s[None, :, None, :]
        if transform:
            x = x @ closed_form_hadamard(D)
        tuples = list(itertools.product(range(nc), repeat=n_sub))
        full = np.stack([np.concatenate([C[c] for c in t]) for t in tuples])   # [T, D]
        dist = ((x[..., None, :] - full) ** 2).sum(-1)                          # [..., T]
        best = np.array(tuples)[dist.argmin(-1)]
        codes, _ = o.encode(keys, C, d, s, transform)
        assert np.array_equal(codes, best), (D, d, nc, transform)


def pin_ties(o):
    # duplicated centroid rows -> the lower index
    C = np.array([[1.0, 1.0], [0.0, 0.0], [0.0, 0.0], [5.0, 5.0]])
    codes, gap = o.pvq_encode(np.zeros((1, 2)), C, 2)
    assert codes.tolist() == [[1]] and gap[0, 0] == 0.0
    # equidistant point -> the lower index
    C2 = np.array([[1.0, 1.0], [0.0, 0.0]])
    codes, _ = o.pvq_encode(np.full((1, 2), 0.5), C2, 2)
    assert codes.tolist() == [[0]]


def pin_identity_codebook(o):
    """Codebook rows = the transformed sub-vectors of 16 tokens: encode
    returns each row's own index and the fp16 reconstruction equals the
    original fp16 keys bit for bit."""
    cfg = synth.tiny()
    keys = cfg["keys"][:, :1, :16]                    # [1, 1, 16, 64]
    s = cfg["smooth"][:1]
    d = cfg["dk"]
    xt = o.forward_transform(keys, s, True)
    C = xt.reshape(-1, d)                             # 256 rows, float64
    codes, _ = o.encode(keys, C, d, s, True)
    assert np.array_equal(codes.reshape(-1), np.arange(C.shape[0]))
    rec = o.decode(codes, C, s, True)
    assert np.array_equal(rec.astype(np.float16).view(np.uint16), keys.view(np.uint16))


def pin_idempotent_and_permutation(o):
    rng = np.random.default_rng(3)
    D, d, nc = 32, 4, 64
    C = rng.standard_normal((nc, d))
    s = rng.uniform(0.5, 3, size=(2, D))
    codes = rng.integers(0, nc, size=(1, 2, 20, D // d))
    rec = o.decode(codes, C, s, True)
    again, _ = o.encode(rec, C, d, s, True)
    assert np.array_equal(again, codes)
    perm = rng.permutation(nc)
    inv = np.argsort(perm)
    C2 = C[perm]                                      # row r of C2 is row perm[r] of C
    rec2 = o.decode(inv[codes], C2, s, True)
    assert np.allclose(rec2, rec, atol=1e-12)


def _golden_attend_inputs():
    g = read_golden("attend_worked.txt")
    kc = g["k_codes"].reshape(1, 1, 3, 2).astype(np.int64)
    vc = g["v_codes"].reshape(1, 1, 3, 2).astype(np.int64)
    Ck = np.array([[0, 0], [np.float32(np.log(3.0)), 0], [np.float32(np.log(4.0)), 0], [1, 1]])
    Cv = g["v_codebook"].reshape(4, 2)
    q = g["q"].reshape(1, 1, 2, 4)
    return g, q, kc, Ck, vc, Cv


def pin_attend_golden(o):
    g, q, kc, Ck, vc, Cv = _golden_attend_inputs()
    for key, causal, W in [("out_causal_w0", True, 0), ("out_causal_w1", True, 1),
                           ("out_causal_w2", True, 2), ("out_full_w0", False, 0),
                           ("out_full_w1", False, 1)]:
        out = o.attend(q, kc, Ck, vc, Cv, scale=1.0, causal=causal, sliding_window=W)
        assert np.max(np.abs(out.reshape(-1) - g[key])) < 1e-6, key


def _exact_codebook_case(rng, B, Hkv, S, D, dk, dv):
    """Codebooks whose rows are exactly the sub-vectors of K and V, so the
    decoded keys and values equal K and V (no smooth, no rotation)."""
    K = rng.standard_normal((B, Hkv, S, D))
    V = rng.standard_normal((B, Hkv, S, D))
    Ck = K.reshape(-1, dk)
    Cv = V.reshape(-1, dv)
    kc = np.arange(Ck.shape[0]).reshape(B, Hkv, S, D // dk)
    vc = np.arange(Cv.shape[0]).reshape(B, Hkv, S, D // dv)
    return K, V, Ck, Cv, kc, vc


def _torch_sdpa(q, K, V, lens, scale, causal, W, G):
    B, Hq, Sq, D = q.shape
    out = np.zeros(q.shape)
    for b in range(B):
        L = int(lens[b])
        qq = torch.from_numpy(q[b])                                    # [Hq, Sq, D]
        kk = torch.from_numpy(K[b, :, :L]).repeat_interleave(G, dim=0)
        vv = torch.from_numpy(V[b, :, :L]).repeat_interleave(G, dim=0)
        m = torch.ones(Sq, L, dtype=torch.bool)
        if causal:
            m = m.tril(diagonal=L - Sq)
        if W > 0:
            m = m & ~torch.ones(Sq, L, dtype=torch.bool).tril(diagonal=L - Sq - W)
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=scale)
        out[b] = o.numpy()
    return out


def pin_attend_sdpa(o):
    rng = np.random.default_rng(11)
    B, Hkv, G, S, D, Sq = 2, 2, 2, 40, 8, 3
    K, V, Ck, Cv, kc, vc = _exact_codebook_case(rng, B, Hkv, S, D, 2, 4)
    q = rng.standard_normal((B, Hkv * G, Sq, D))
    lens = np.array([40, 23])
    for causal, W in [(True, 0), (True, 5), (False, 0), (False, 7), (True, 100)]:
        ref = _torch_sdpa(q, K, V, lens, 0.37, causal, W, G)
        out = o.attend(q, kc, Ck, vc, Cv, scale=0.37, causal=causal, sliding_window=W, kv_lens=lens)
        assert np.max(np.abs(out - ref)) < 1e-12, (causal, W)


def pin_attend_closed_forms(o):
    rng = np.random.default_rng(5)
    B, Hkv, S, D = 1, 1, 30, 8
    K, V, Ck, Cv, kc, vc = _exact_codebook_case(rng, B, Hkv, S, D, 4, 4)
    q = rng.standard_normal((1, 1, 4, D))
    lens = np.array([25])
    # W = 1 -> the value at the query's own slot q_abs = len - S_q + i
    out = o.attend(q, kc, Ck, vc, Cv, scale=1.0, causal=True, sliding_window=1, kv_lens=lens)
    for i in range(4):
        assert np.allclose(out[0, 0, i], V[0, 0, 25 - 4 + i], atol=1e-12)
    # all key codes equal -> uniform weights -> mean of the valid values
    kc_same = np.zeros_like(kc)
    out = o.attend(q, kc_same, Ck, vc, Cv, scale=1.0, causal=True, kv_lens=lens)
    for i in range(4):
        assert np.allclose(out[0, 0, i], V[0, 0, :25 - 4 + i + 1].mean(0), atol=1e-12)
    # one key -> that value
    out = o.attend(q[:, :, :1], kc, Ck, vc, Cv, scale=1.0, causal=True, kv_lens=np.array([1]))
    assert np.allclose(out[0, 0, 0], V[0, 0, 0], atol=1e-12)
    # fully masked rows (causal, more queries than keys) -> zeros
    out = o.attend(q, kc, Ck, vc, Cv, scale=1.0, causal=True, kv_lens=np.array([2]))
    assert np.all(out[0, 0, :2] == 0) and np.allclose(out[0, 0, 2], V[0, 0, 0])


def pin_gqa_and_window(o):
    rng = np.random.default_rng(9)
    B, Hkv, G, S, D = 2, 2, 3, 50, 16
    kc = rng.integers(0, 32, size=(B, Hkv, S, D // 4))
    vc = rng.integers(0, 32, size=(B, Hkv, S, D // 4))
    Ck = rng.standard_normal((32, 4))
    Cv = rng.standard_normal((32, 4))
    s = rng.uniform(0.5, 2, size=(Hkv, D))
    q = rng.standard_normal((B, Hkv * G, 2, D))
    lens = np.array([50, 31])
    gqa = o.attend(q, kc, Ck, vc, Cv, scale=0.3, smooth=s, transform=True, kv_lens=lens)
    rep = lambda a: np.repeat(a, G, axis=1)
    mha = o.attend(q, rep(kc), Ck, rep(vc), Cv, scale=0.3, smooth=np.repeat(s, G, axis=0),
                   transform=True, kv_lens=lens)
    assert np.allclose(gqa, mha, atol=1e-12)
    big_w = o.attend(q, kc, Ck, vc, Cv, scale=0.3, smooth=s, transform=True, kv_lens=lens,
                     sliding_window=60)
    assert np.allclose(big_w, gqa, atol=1e-12)


def pin_dual_transform(o):
    """LUT scores of the transformed query equal q . K_hat (dual identity)."""
    g, D, d, keys, s, C = _golden_encode_inputs()
    codes, _ = o.encode(keys, C, d, s, True)
    q = np.array([1.0, 1.0, 0.0, 0.0])
    sc = o.lut_scores(q, codes[0, 0], C, d, smooth_row=s, transform=True)
    assert sc[0] == 6.0          # q . [4, 2, 2, 0], derived by hand
    rng = np.random.default_rng(13)
    D, d, nc = 64, 4, 256
    C = rng.standard_normal((nc, d))
    s = rng.uniform(0.3, 9.0, size=D)
    codes = rng.integers(0, nc, size=(1, 1, 300, D // d))
    q = rng.standard_normal(D) * rng.uniform(0.1, 20, size=D)
    K = o.decode(codes, C, s, True)[0, 0]
    ref = K @ q
    sc = o.lut_scores(q, codes[0, 0], C, d, smooth_row=s, transform=True)
    assert np.max(np.abs(sc - ref)) <= 1e-10 * np.max(np.abs(ref))


def random_orthogonal(rng, D):
    """A random orthogonal matrix (QR of a Gaussian), not symmetric."""
    qm, r = np.linalg.qr(rng.standard_normal((D, D)))
    return qm * np.sign(np.diag(r))[None, :]


def pin_dense_transform(o):
    """An explicit transform matrix M (the H_mat argument of the fused
    encode-decode kernel): encode applies x . M, decode x~ . M^-1, the query
    LUT (q * s) . (M^-1)^T.  Pinned with a non-symmetric orthogonal M, where
    M, M^T and M^-1 differ, and with M = the Sylvester matrix itself."""
    rng = np.random.default_rng(21)
    D, d, nc = 32, 4, 64
    M = random_orthogonal(rng, D)
    assert np.max(np.abs(M @ M.T - np.eye(D))) < 1e-12 and np.max(np.abs(M - M.T)) > 0.1
    x = rng.standard_normal((1, 2, 40, D)) * rng.uniform(0.5, 20, size=D)
    s = rng.uniform(0.3, 9.0, size=(2, D))
    # round trip without quantization returns the input
    back = o.inverse_transform(o.forward_transform(x, s, M), s, M)
    assert np.max(np.abs(back - x)) <= 1e-12 * np.max(np.abs(x))
    # forward is (x / s) . M, written out element by element for one vector
    xt = o.forward_transform(x, s, M)
    v = x[0, 1, 7] / s[1]
    assert np.max(np.abs(xt[0, 1, 7] - np.array([sum(v[i] * M[i, j] for i in range(D))
                                                  for j in range(D)]))) < 1e-12
    # dual identity: LUT scores equal q . K_hat with K_hat decoded through M^-1
    C = rng.standard_normal((nc, d))
    codes = rng.integers(0, nc, size=(1, 1, 200, D // d))
    q = rng.standard_normal(D) * rng.uniform(0.1, 20, size=D)
    K = o.decode(codes, C, s[:1], M)[0, 0]
    sc = o.lut_scores(q, codes[0, 0], C, d, smooth_row=s[0], transform=M)
    assert np.max(np.abs(sc - K @ q)) <= 1e-10 * np.max(np.abs(K @ q))
    # M = the Sylvester matrix reproduces transform=True
    H = closed_form_hadamard(D)
    c1, _ = o.encode(x, C, d, s, H)
    c2, _ = o.encode(x, C, d, s, True)
    assert np.array_equal(c1, c2)
    assert np.max(np.abs(o.decode(c1, C, s, H) - o.decode(c2, C, s, True))) < 1e-12


def pin_randomized_hadamard(o):
    """M = diag(sigma) . H with sigma in {-1, +1}^D (a randomized Hadamard
    rotation) is orthonormal, and transforming with smooth s and M equals
    transforming with smooth s * sigma and the plain Hadamard matrix: the
    divided vector's signs flip before the rotation, decode's multiply flips
    them back, and the query's smooth multiply carries them to the LUT."""
    rng = np.random.default_rng(22)
    D, d, nc, S = 64, 8, 128, 60
    sigma = rng.choice([-1.0, 1.0], size=D)
    M = sigma[:, None] * closed_form_hadamard(D)
    assert np.max(np.abs(M @ M.T - np.eye(D))) < 1e-12
    s = rng.uniform(0.3, 9.0, size=(2, D))
    x = rng.standard_normal((1, 2, S, D)) * rng.uniform(0.5, 20, size=D)
    C = rng.standard_normal((nc, d))
    c1, g1 = o.encode(x, C, d, s, M)
    c2, g2 = o.encode(x, C, d, s * sigma, True)
    assert np.array_equal(c1, c2)
    assert np.max(np.abs(o.decode(c1, C, s, M) - o.decode(c1, C, s * sigma, True))) < 1e-12
    q = rng.standard_normal((1, 4, 3, D))
    vc = rng.integers(0, nc, size=(1, 2, S, D // 4))
    Cv = rng.standard_normal((nc, 4))
    a1 = o.attend(q, c1, C, vc, Cv, scale=0.2, smooth=s, transform=M, kv_lens=[50])
    a2 = o.attend(q, c1, C, vc, Cv, scale=0.2, smooth=s * sigma, transform=True, kv_lens=[50])
    assert np.max(np.abs(a1 - a2)) < 1e-12


def pin_kmeans_golden(o):
    """Two Lloyd runs worked by hand (tests/golden/kmeans_worked.txt): a 1-D
    one whose second step moves a point, a 2-D one with an exact tie and a
    centroid that never gets a member."""
    g = read_golden("kmeans_worked.txt")
    for tag, d, steps in [("a", 1, 3), ("b", 2, 2)]:
        x = g[f"{tag}_points"].reshape(-1, d)
        C = g[f"{tag}_init"].reshape(-1, d)
        for it in range(1, steps + 1):
            C, labels, inertia, _ = o.lloyd_step(x, C)
            if f"{tag}_labels_{it}" in g:
                assert np.array_equal(labels, g[f"{tag}_labels_{it}"]), (tag, it)
            assert abs(inertia - g[f"{tag}_inertia_{it}"][0]) < 1e-12, (tag, it, inertia)
            assert np.max(np.abs(C.ravel() - g[f"{tag}_centroids_{it}"])) < 1e-12, (tag, it)
        Ck, lk, ek, _ = o.kmeans(x, g[f"{tag}_init"].reshape(-1, d), steps)
        assert np.allclose(ek, [g[f"{tag}_inertia_{i}"][0] for i in range(1, steps + 1)], rtol=0, atol=1e-12)
        assert np.max(np.abs(Ck.ravel() - g[f"{tag}_centroids_{steps}"])) < 1e-12


def pin_kmeans_single_cluster(o):
    """k = 1 in closed form: one step moves the centroid to the mean; the
    first inertia is N (sum of variances + |mean - init|^2) (parallel axis),
    the second N * sum of variances."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((500, 6)) * rng.uniform(0.5, 4, size=6) + rng.uniform(-3, 3, size=6)
    init = rng.standard_normal((1, 6)) * 5
    C, labels, inertia, _ = o.kmeans(x, init, 2)
    mean, var = x.mean(axis=0), x.var(axis=0)
    assert np.max(np.abs(C[0] - mean)) < 1e-12 and not labels.any()
    n = x.shape[0]
    assert abs(inertia[0] - n * (var.sum() + np.sum((mean - init[0]) ** 2))) < 1e-8 * inertia[0]
    assert abs(inertia[1] - n * var.sum()) < 1e-9 * inertia[1]


def pin_kmeans_separated(o):
    """Blobs far apart relative to their spread, each started from one of its
    own points (in a shuffled order): every label is the blob's start index
    and every centroid the blob's mean, from the first step on."""
    rng = np.random.default_rng(32)
    k, n, d = 12, 40, 8
    centres = rng.standard_normal((k, d)) * 100
    x = np.concatenate([c + rng.standard_normal((n, d)) for c in centres])
    order = rng.permutation(k)                      # centroid i starts in blob order[i]
    init = x[order * n]
    C, labels, inertia, _ = o.kmeans(x, init, 3)
    blob_of_centroid = np.empty(k, dtype=np.int64)
    blob_of_centroid[order] = np.arange(k)          # blob b is centroid blob_of_centroid[b]
    assert np.array_equal(labels, np.repeat(blob_of_centroid, n))
    for b in range(k):
        assert np.max(np.abs(C[blob_of_centroid[b]] - x[b * n:(b + 1) * n].mean(axis=0))) < 1e-9
    assert inertia[1] == pytest.approx(inertia[2], rel=1e-12) and inertia[0] > inertia[1]


def pin_kmeans_fixed_point_bruteforce(o):
    """Run to convergence on a tiny random set; then, checked with plain
    loops, every label is the nearest centroid (lowest index on ties), every
    centroid the mean of its members, and the inertia never rose."""
    rng = np.random.default_rng(33)
    N, k, d = 60, 5, 3
    x = rng.standard_normal((N, d)) * np.array([1.0, 3.0, 0.5])
    C, labels, inertia, _ = o.kmeans(x, x[:k] + 0.01, 60)
    for i in range(1, len(inertia)):
        assert inertia[i] <= inertia[i - 1] * (1 + 1e-12)
    for i in range(N):
        best, arg = None, None
        for c in range(k):
            dist = sum((float(x[i][e]) - float(C[c][e])) ** 2 for e in range(d))
            if best is None or dist < best:
                best, arg = dist, c
        assert labels[i] == arg
    for c in range(k):
        members = [i for i in range(N) if labels[i] == c]
        if members:
            for e in range(d):
                assert abs(C[c][e] - sum(float(x[i][e]) for i in members) / len(members)) < 1e-12
    # the training vectors are the transformed keys' sub-vectors, in order
    keys = rng.standard_normal((1, 2, 3, 8))
    tv = o.training_vectors(keys, 4)
    for h in range(2):
        for t in range(3):
            for j in range(2):
                assert np.array_equal(tv[(h * 3 + t) * 2 + j], keys[0, h, t, 4 * j:4 * j + 4])


ALL_PINS = [pin_hadamard_closed_form, pin_hadamard_golden, pin_hadamard_orthonormal,
            pin_storage, pin_encode_golden, pin_distances_and_gap_golden, pin_gap_bruteforce,
            pin_bruteforce, pin_nibbles, pin_ties, pin_identity_codebook,
            pin_idempotent_and_permutation, pin_attend_golden, pin_attend_sdpa,
            pin_attend_closed_forms, pin_gqa_and_window, pin_dual_transform,
            pin_dense_transform, pin_randomized_hadamard, pin_kmeans_golden,
            pin_kmeans_single_cluster, pin_kmeans_separated, pin_kmeans_fixed_point_bruteforce]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)


# ----------------------------------------------------------------------------
# Fixture sanity and generator determinism
# ----------------------------------------------------------------------------
def test_golden_wrong_direction_differs():
    g, D, d, keys, s, C = _golden_encode_inputs()
    xt = (keys * s) @ closed_form_hadamard(D)
    codes, _ = O.pvq_encode(xt, C, d)
    assert np.array_equal(codes[0, 0, 0], g["wrong_direction_codes_token0"])
    assert not np.array_equal(codes[0, 0, 0], g["codes"][:2])


def test_storage_matches_workloads():
    # 16 B/token/head key codes at D=128, d_k=8, 8-bit codes; 32 B for d_v=4
    assert O.code_bytes_per_token(128, 8, 8) == 16
    assert O.code_bytes_per_token(128, 4, 8) == 32


def test_generator_deterministic():
    a, b = synth.tiny(), synth.tiny()
    for k in ["keys", "values", "q", "smooth", "k_codebook", "v_codebook"]:
        assert np.array_equal(a[k], b[k])
    g1, g2 = synth.gqa_long(0), synth.gqa_long(4096)
    assert np.array_equal(g1["kv_lens"], g2["kv_lens"])
    assert g1["kv_lens"].min() >= 16384 and g1["kv_lens"].max() <= 32768
    # outlier channels: per head, exactly n channels carry the x20 scale
    k = synth.tiny()["keys"].astype(np.float32)
    big = (np.abs(k).max(axis=2) > 8).sum(-1)
    assert big.tolist() == [[2, 2]]


# ----------------------------------------------------------------------------
# Planted mistakes: every mutation must make at least one pin fail
# ----------------------------------------------------------------------------
def _mut_smooth_direction(mp):
    orig = O._smooth_rows
    mp.setattr(O, "_smooth_rows", lambda s, h, d: None if s is None else 1.0 / orig(s, h, d))


def _mut_unnormalized_hadamard(mp):
    orig = O.sylvester_hadamard
    mp.setattr(O, "sylvester_hadamard", lambda D: orig(D) * math.sqrt(D))


def _mut_no_inverse_rotation(mp):
    orig = O.inverse_transform
    mp.setattr(O, "inverse_transform", lambda xt, s=None, t=False: orig(xt, s, False))


def _mut_ties_high(mp):
    orig = O.pvq_encode

    def enc(x, C, d, chunk_rows=1 << 15):
        C = np.asarray(C)
        c, g = orig(x, C[::-1], d, chunk_rows)
        return C.shape[0] - 1 - c, g
    mp.setattr(O, "pvq_encode", enc)


def _mut_strided_split(mp):
    enc0, dec0 = O.pvq_encode, O.pvq_decode

    def perm(D, d):
        n = D // d
        return np.arange(D).reshape(d, n).T.reshape(-1)   # sub-vector j = dims j, j+n, ...

    def enc(x, C, d, chunk_rows=1 << 15):
        x = np.asarray(x)
        return enc0(x[..., perm(x.shape[-1], d)], C, d, chunk_rows)

    def dec(codes, C):
        y = dec0(codes, C)
        D, d = y.shape[-1], np.asarray(C).shape[1]
        return y[..., np.argsort(perm(D, d))]
    mp.setattr(O, "pvq_encode", enc)
    mp.setattr(O, "pvq_decode", dec)


def _mut_head_aligned_causal(mp):
    def mask(L, Sq, causal, W):
        i = np.arange(Sq)[:, None]
        t = np.arange(L)[None, :]
        v = np.ones((Sq, L), bool)
        if causal:
            v &= t <= i
        if W > 0:
            v &= t > i - W
        return v
    mp.setattr(O, "attention_mask", mask)


def _mut_window_off_by_one(mp):
    orig = O.attention_mask
    mp.setattr(O, "attention_mask", lambda L, Sq, c, W: orig(L, Sq, c, W + 1 if W > 0 else 0))


def _mut_window_needs_causal(mp):
    orig = O.attention_mask
    mp.setattr(O, "attention_mask", lambda L, Sq, c, W: orig(L, Sq, c, W if c else 0))


def _mut_gqa_modulo(mp):
    orig = O.attend

    def att(q, kc, Ck, vc, Cv, **kw):
        Hq, Hkv = q.shape[1], kc.shape[1]
        G = Hq // Hkv
        # query head h reads kv head h % H_kv: reorder heads so that the
        # contiguous mapping of the original produces the modulo mapping
        order = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
        inv = np.argsort(order)
        out = orig(q[:, inv], kc, Ck, vc, Cv, **kw)
        return out[:, order]
    mp.setattr(O, "attend", att)


def _mut_lut_divides(mp):
    orig = O.query_lut
    mp.setattr(O, "query_lut", lambda q, C, d, s=None, t=False:
               orig(q, C, d, None if s is None else 1.0 / np.asarray(s), t))


def _mut_missing_scale(mp):
    orig = O.attend
    mp.setattr(O, "attend", lambda *a, **kw: orig(*a, **{**kw, "scale": 1.0}))


def _mut_value_transposed(mp):
    orig = O.pvq_decode

    def dec(codes, C):
        C = np.asarray(C)
        g = C[np.asarray(codes).astype(np.int64)]                # [..., n_sub, d]
        g = np.swapaxes(g, -1, -2)
        return g.reshape(*np.asarray(codes).shape[:-1], -1)
    mp.setattr(O, "pvq_decode", dec)


def _mut_matrix_involutory(mp):
    # every explicit transform matrix treated as its own inverse, as the
    # Sylvester matrix is
    orig = O._rotation

    def rot(t, D):
        m, mi = orig(t, D)
        return (m, m) if isinstance(t, np.ndarray) else (m, mi)
    mp.setattr(O, "_rotation", rot)


def _mut_dual_untransposed(mp):
    # the query rotated by M^-1 instead of (M^-1)^T
    orig = O._rotation
    mp.setattr(O, "query_lut", lambda q, C, d, s=None, t=False: _lut_with(orig, q, C, d, s, t))


def _lut_with(rot, q, C, d, s, t):
    qt = np.asarray(q, dtype=np.float64)
    if s is not None:
        qt = qt * np.asarray(s, dtype=np.float64)
    _, mi = rot(t, qt.shape[-1])
    if mi is not None:
        qt = qt @ mi
    return qt.reshape(-1, d) @ np.asarray(C, dtype=np.float64).T


def _mut_gap_relative_to_d1(mp):
    # the near-tie gap taken relative to the smaller distance: (d2 - d1) / d1
    orig = O.pvq_encode

    def enc(x, C, d, chunk_rows=1 << 15):
        c, g = orig(x, C, d, chunk_rows)
        with np.errstate(divide="ignore", invalid="ignore"):
            return c, np.where(g < 1, g / (1 - g), np.inf)
    mp.setattr(O, "pvq_encode", enc)


def _mut_gap_third_smallest(mp):
    # the gap from the smallest and the third-smallest distance
    orig = O.pvq_encode

    def enc(x, C, d, chunk_rows=1 << 15):
        c, _ = orig(x, C, d, chunk_rows)
        dist = O.pvq_distances(np.asarray(x, dtype=np.float64), C, d)
        srt = np.sort(dist, -1)
        k = min(2, srt.shape[-1] - 1)
        with np.errstate(divide="ignore", invalid="ignore"):
            return c, np.where(srt[..., k] > 0, (srt[..., k] - srt[..., 0]) / srt[..., k], 0.0)
    mp.setattr(O, "pvq_encode", enc)


def _mut_distances_transposed(mp):
    # the distance table built from a transposed reshape of the sub-vectors
    def dist(x, C, sub_dim):
        x = np.asarray(x, dtype=np.float64)
        C = np.asarray(C, dtype=np.float64)
        n_sub = x.shape[-1] // sub_dim
        r = np.swapaxes(x.reshape(*x.shape[:-1], sub_dim, n_sub), -1, -2)[..., None, :]
        return np.sum((r - C) ** 2, axis=-1)
    mp.setattr(O, "pvq_distances", dist)


def _mut_nibble_order(mp):
    # the even element in the high nibble
    def pack(codes):
        c = np.asarray(codes).astype(np.int64)
        return (((c[..., 0::2] & 0xF) << 4) | (c[..., 1::2] & 0xF)).astype(np.uint8)

    def unpack(packed):
        b = np.asarray(packed).astype(np.int64)
        out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
        out[..., 0::2], out[..., 1::2] = b >> 4, b & 0xF
        return out
    mp.setattr(O, "pack_nibbles", pack)
    mp.setattr(O, "unpack_nibbles", unpack)


def _mut_kmeans_sum_update(mp):
    # the update keeps the members' sum instead of their mean
    orig = O.lloyd_step

    def step(x, C):
        new, labels, e, gap = orig(x, C)
        counts = np.bincount(labels, minlength=np.asarray(C).shape[0])
        has = counts > 0
        new[has] *= counts[has, None]
        return new, labels, e, gap
    mp.setattr(O, "lloyd_step", step)


def _mut_kmeans_empty_to_zero(mp):
    # a centroid with no member is reset to the origin
    orig = O.lloyd_step

    def step(x, C):
        new, labels, e, gap = orig(x, C)
        counts = np.bincount(labels, minlength=np.asarray(C).shape[0])
        new[counts == 0] = 0.0
        return new, labels, e, gap
    mp.setattr(O, "lloyd_step", step)


def _mut_kmeans_inertia_after_update(mp):
    # the inertia measured against the updated centroids
    orig = O.lloyd_step

    def step(x, C):
        new, labels, e, gap = orig(x, C)
        diff = np.asarray(x, dtype=np.float64) - new[labels]
        return new, labels, float(np.sum(diff * diff)), gap
    mp.setattr(O, "lloyd_step", step)


def _mut_kmeans_split_strided(mp):
    # training vectors taken with a strided split of D
    def tv(x, sub_dim, smooth=None, transform=False):
        xt = O.forward_transform(x, smooth, transform)
        D = xt.shape[-1]
        return np.swapaxes(xt.reshape(*xt.shape[:-1], sub_dim, D // sub_dim), -1, -2).reshape(-1, sub_dim)
    mp.setattr(O, "training_vectors", tv)


MUTATIONS = [_mut_matrix_involutory, _mut_dual_untransposed, _mut_smooth_direction, _mut_unnormalized_hadamard, _mut_no_inverse_rotation,
             _mut_ties_high, _mut_strided_split, _mut_head_aligned_causal,
             _mut_window_off_by_one, _mut_window_needs_causal, _mut_gqa_modulo,
             _mut_lut_divides, _mut_missing_scale, _mut_value_transposed,
             _mut_gap_relative_to_d1, _mut_gap_third_smallest, _mut_distances_transposed,
             _mut_nibble_order, _mut_kmeans_sum_update, _mut_kmeans_empty_to_zero,
             _mut_kmeans_inertia_after_update, _mut_kmeans_split_strided]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda m: m.__name__)
def test_planted_mistake_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"{mutation.__name__} went unnoticed by every pin"
