"""GPU parity of codebook training: vq_transform (the vectors the encode
searches) and vq_kmeans (Lloyd iterations) against the oracle's
forward_transform and lloyd_step / kmeans (reading R25 of the oracle: the
pages encode against a pre-trained codebook and say no more about how it is
trained).

Bars, derived from the arithmetic (fp32 on the GPU, fp64 in the oracle):
  transform   |gpu - ref| <= gamma_n * (|x / s| . |M|) elementwise, n the
              roundings on the path (division, log2 D butterfly stages and
              the final scale), gamma_n = n u / (1 - n u), u = 2^-24
              (Higham's bound for sums).  A dense matrix runs on the matrix
              cores as three split-fp16 products per term (each within
              3 * 2^-22 of the exact product: two split roundings and the
              dropped lo.lo part) summed in fp32 in an unspecified order:
              n = 3 D + 14.
  labels      equal, except at near-ties (the oracle's top-2 gap below 1e-5
              relative), where the GPU's centroid must be within 1e-5 d2 of
              the nearest (as for codes).
  centroids   clusters with the same members on both sides: within the
              largest transform bound of any vector (the members differ by
              at most that) plus one fp32 rounding of the mean.  Clusters a
              near-tie moved a vector into or out of: the GPU centroid is the
              mean of the GPU's own members (a property of the step).
  inertia     within 2 t sqrt(d N E) + (d + 2) u E + N d t^2 of the oracle's
              E, t the transform bound (Cauchy-Schwarz over the per-vector
              distance errors).
Full size (the encode workload's 1,048,576 key sub-vectors) checks sampled
labels against the oracle one by one and the update as a property: every
trained centroid is the mean of its members, the inertia never rises.
"""
import math

import numpy as np
import pytest
import torch

import oracle.vq_oracle as O
from vector_quantized_kv_amd import synth, vq_kmeans, vq_transform
from test_gpu_parity import DEV, NEAR_TIE, dev

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def transform_bound(keys, smooth, transform):
    """Elementwise bound on |fp32 transform - exact| for keys [B, H, S, D]."""
    B, H, S, D = keys.shape
    x = np.abs(keys.astype(np.float64))
    if smooth is not None:
        s = np.abs(np.asarray(smooth, np.float64).reshape(-1, D))
        x = x / np.broadcast_to(s, (H, D))[None, :, None, :]
    if transform is True:
        return gamma(int(math.log2(D)) + 3) * (x.sum(-1, keepdims=True) / math.sqrt(D)) * np.ones(D)
    if transform is False:
        return gamma(1) * x
    return gamma(3 * D + 14) * (x @ np.abs(np.asarray(transform, np.float64)))


def mats(M):
    return dev(np.asarray(M, np.float32))


def run_transform(keys, smooth, transform):
    m = None
    if transform is not True and transform is not False:
        m = mats(transform)
    out = vq_transform(dev(keys), smooth=None if smooth is None else dev(smooth),
                       transform=transform if m is None else 2, mat=m)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B,H,S,D,smooth_kind,transform", [
    (1, 2, 37, 32, None, True),
    (2, 3, 129, 64, "shared", True),
    (1, 8, 300, 128, "per_head", True),
    (1, 2, 65, 256, "per_head", True),
    (2, 4, 50, 128, None, False),
    (1, 3, 77, 64, "per_head", "dense"),
    (1, 2, 40, 128, "shared", "dense"),
])
def test_transform(B, H, S, D, smooth_kind, transform):
    rng = np.random.default_rng(5000 + D + S)
    k = synth.outlier_normal(rng, (B, H, S, D), 4)
    s = synth.smooth_factors(k)
    smooth = None if smooth_kind is None else (s if smooth_kind == "per_head" else s[0])
    if transform == "dense":
        transform = np.eye(D) + 0.3 * rng.standard_normal((D, D)) / math.sqrt(D)
    got = run_transform(k, smooth, transform)
    ref = O.forward_transform(k, smooth, transform)
    bound = transform_bound(k, smooth, transform)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"worst excess {np.max(err - bound):.3g}"
    print(f"[transform] D{D} {smooth_kind} max err {err.max():.3g} (bound max {bound.max():.3g})")


# ----------------------------------------------------------------------------
# one Lloyd step against the oracle
# ----------------------------------------------------------------------------
def check_labels(vec_ref, C, lab_gpu, lab_ref, gap, tag):
    mism = lab_gpu != lab_ref
    n = int(mism.sum())
    if n:
        assert np.all(gap[mism] < NEAR_TIE), f"{tag}: {n} label mismatches, some not near-ties"
        dist = O.pvq_distances(vec_ref[mism], C, C.shape[1])[:, 0]
        srt = np.sort(dist, -1)
        assert np.all(dist[np.arange(n), lab_gpu[mism]] - srt[:, 0] <= NEAR_TIE * srt[:, 1]), \
            f"{tag}: a GPU label is not near-optimal"
    print(f"[kmeans] {tag}: {lab_gpu.size} labels, {n} near-tie mismatches")
    return mism


def check_step(tag, vec_ref, vec_gpu, tbound, init, C_gpu, lab_gpu, e_gpu):
    """One Lloyd step of the GPU (from init) against the oracle's."""
    C_ref, lab_ref, e_ref, gap = O.lloyd_step(vec_ref, init)
    lab_gpu = lab_gpu.astype(np.int64)
    mism = check_labels(vec_ref, init, lab_gpu, lab_ref, gap, tag)
    touched = np.zeros(init.shape[0], dtype=bool)
    touched[lab_ref[mism]] = True
    touched[lab_gpu[mism]] = True
    same = ~touched
    bar = tbound + 2 * U * np.abs(C_ref[same]) + 1e-12
    err = np.abs(C_gpu[same].astype(np.float64) - C_ref[same])
    assert np.all(err <= bar), f"{tag}: centroid error {np.max(err - bar):.3g} over the bar"
    for c in np.nonzero(touched)[0]:
        members = vec_gpu[lab_gpu == c].astype(np.float64)
        want = members.mean(axis=0) if len(members) else init[c]
        assert np.all(np.abs(C_gpu[c] - want) <= 2 * U * np.abs(want) + 1e-12), f"{tag}: centroid {c}"
    N, d = vec_ref.shape
    ebar = 2 * tbound * math.sqrt(d * N * e_ref) + (d + 2) * U * e_ref + N * d * tbound ** 2
    assert abs(e_gpu - e_ref) <= ebar, f"{tag}: inertia {e_gpu} vs {e_ref} (bar {ebar:.3g})"
    print(f"[kmeans] {tag}: centroid max err {err.max() if err.size else 0:.3g}, "
          f"{int(touched.sum())} clusters touched by near-ties, inertia rel err "
          f"{abs(e_gpu - e_ref) / max(e_ref, 1e-300):.3g}")
    return C_ref


@pytest.mark.parametrize("B,H,S,D,d,n_c,kind", [
    (1, 4, 512, 128, 8, 256, "keys"),
    (1, 4, 512, 128, 4, 256, "values"),
    (2, 2, 333, 128, 8, 16, "keys"),
    (1, 4, 257, 128, 16, 64, "keys"),
    (1, 2, 100, 64, 2, 32, "values"),
    (1, 1, 70, 32, 1, 8, "keys"),
    (1, 1, 3, 32, 8, 256, "keys"),          # fewer vectors (12) than centroids
    (1, 8, 600, 128, 8, 256, "keys"),       # 76,800 sub-vectors of 8: the matrix-core search
    (2, 2, 1100, 128, 8, 16, "keys"),       # 70,400 of 8, a 16-centroid codebook
])
def test_lloyd_step(B, H, S, D, d, n_c, kind):
    """vq_transform then one vq_kmeans iteration, from centroids sampled from
    the oracle's transformed vectors (n_c > N: the extra centroids are the
    sampled ones repeated, so some keep their value)."""
    rng = np.random.default_rng(5100 + S + d + n_c)
    x = synth.outlier_normal(rng, (B, H, S, D), 4)
    keys = kind == "keys"
    s = synth.smooth_factors(x) if keys else None
    vec_ref = O.training_vectors(x, d, s, keys)
    N = vec_ref.shape[0]
    init = synth.sample_rows(rng, vec_ref, min(n_c, N))
    if n_c > N:
        init = np.concatenate([init] * (n_c // N + 1))[:n_c]
    vt = vq_transform(dev(x), smooth=None if s is None else dev(s), transform=keys)
    C = dev(init)
    _, labels, inertia = vq_kmeans(vt.view(-1, d), C, 1, with_labels=True)
    torch.cuda.synchronize()
    tb = float(transform_bound(x, s, keys).max())
    check_step(f"{kind} D{D} d{d} n_c{n_c} N{N}", vec_ref, vt.view(-1, d).cpu().numpy(), tb,
               init.astype(np.float64), C.cpu().numpy(), labels.cpu().numpy(),
               float(inertia.cpu().numpy()[0]))


@pytest.mark.parametrize("n", [300, 1100])
def test_separated_blobs_many_iterations(n):
    """Blobs far apart: ten GPU iterations land on the oracle's centroids,
    labels equal throughout (no near-ties exist), and the inertia sequence
    matches (64 x 1100 vectors run the matrix-core search)."""
    rng = np.random.default_rng(5200 + n)
    k, d = 64, 8
    centres = rng.standard_normal((k, d)) * 50
    x = np.concatenate([c + rng.standard_normal((n, d)) for c in centres]).astype(np.float32)
    blob = np.repeat(np.arange(k), n)
    perm = rng.permutation(x.shape[0])
    x, blob = x[perm], blob[perm]
    # one start per blob, in a shuffled blob order, off its first point
    first = np.array([np.nonzero(blob == b)[0][0] for b in rng.permutation(k)])
    init = x[first] + rng.standard_normal((k, d)).astype(np.float32) * 0.5
    C_ref, lab_ref, e_ref, gap = O.kmeans(x, init, 10)
    assert gap.min() > 1e-3
    C = dev(init)
    _, labels, inertia = vq_kmeans(dev(x), C, 10, with_labels=True)
    torch.cuda.synchronize()
    assert np.array_equal(labels.cpu().numpy().astype(np.int64), lab_ref)
    err = np.abs(C.cpu().numpy() - C_ref)
    assert np.all(err <= 4 * U * np.abs(C_ref) + 1e-6), err.max()
    e = inertia.cpu().numpy()
    assert np.allclose(e, e_ref, rtol=1e-6, atol=0), (e, e_ref)
    print(f"[kmeans] blobs: centroid max err {err.max():.3g}, inertia {e[0]:.6g} -> {e[-1]:.6g}")


def test_empty_and_duplicate_centroids():
    """A centroid far from every vector and an exact duplicate of another get
    no member and keep their values; ties go to the lower index."""
    rng = np.random.default_rng(5300)
    x = rng.standard_normal((5000, 4)).astype(np.float32)
    init = x[:16].copy()
    init[3] = 1e4
    init[9] = init[2]                      # exact duplicate of centroid 2
    C_ref, lab_ref, e_ref, _ = O.lloyd_step(x, init)
    C = dev(init)
    _, labels, inertia = vq_kmeans(dev(x), C, 1, with_labels=True)
    torch.cuda.synchronize()
    lab = labels.cpu().numpy().astype(np.int64)
    assert not np.any(lab == 3) and not np.any(lab == 9) and np.any(lab == 2)
    got = C.cpu().numpy()
    assert np.array_equal(got[3], init[3]) and np.array_equal(got[9], init[9])
    check_labels(x.astype(np.float64), init.astype(np.float64), lab, lab_ref,
                 O.lloyd_step(x, init)[3], "empty/duplicate")


def test_degenerate_sizes():
    """N = 0 keeps every centroid and reports zero inertia; one centroid
    becomes the mean; a single vector pulls its nearest centroid onto it."""
    C = dev(np.arange(8, dtype=np.float32).reshape(2, 4))
    before = C.clone()
    _, _, inertia = vq_kmeans(torch.empty((0, 4), dtype=torch.float32, device=DEV), C, 2)
    torch.cuda.synchronize()
    assert torch.equal(C, before) and inertia.cpu().tolist() == [0.0, 0.0]
    rng = np.random.default_rng(5400)
    x = rng.standard_normal((10007, 8)).astype(np.float32)
    C1 = dev(np.zeros((1, 8), np.float32))
    vq_kmeans(dev(x), C1, 1)
    torch.cuda.synchronize()
    mean = x.astype(np.float64).mean(axis=0)
    assert np.all(np.abs(C1.cpu().numpy()[0] - mean) <= 2 * U * np.abs(mean) + 1e-12)
    C2 = dev(np.array([[0, 0], [5, 5]], np.float32))
    _, lab, e = vq_kmeans(dev(np.array([[4.0, 4.5]], np.float32)), C2, 1, with_labels=True)
    torch.cuda.synchronize()
    assert C2.cpu().tolist() == [[0, 0], [4.0, 4.5]] and lab.item() == 1
    assert e.item() == pytest.approx(1.0 + 0.25, rel=1e-12)


def test_full_size_training():
    """The encode workload's keys (1,048,576 sub-vectors of 8, 256
    centroids): one GPU step's labels on a sample equal the oracle's from the
    same start; eight more iterations never raise the inertia and leave every
    centroid at the mean of its members."""
    w = synth.encode()
    x, d, n_c = w["keys"], w["dk"], 256
    s = w["smooth"]
    rng = np.random.default_rng(5500)
    vec_ref = O.training_vectors(x, d, s, True)
    N = vec_ref.shape[0]
    init = synth.sample_rows(rng, vec_ref, n_c)
    vt = vq_transform(dev(x), smooth=dev(s)).view(-1, d)
    C = dev(init)
    _, labels, inertia = vq_kmeans(vt, C, 1, with_labels=True)
    torch.cuda.synchronize()
    sample = rng.choice(N, size=4096, replace=False)
    lab_ref, gap = O.pvq_encode(vec_ref[sample], init, d)
    check_labels(vec_ref[sample], init.astype(np.float64), labels.cpu().numpy()[sample].astype(np.int64),
                 lab_ref[:, 0], gap[:, 0], "full-size sample")
    e_sample = O.lloyd_step(vec_ref[sample], init)[2]
    e0 = float(inertia.cpu().numpy()[0])
    assert 0.8 * e_sample * N / 4096 < e0 < 1.25 * e_sample * N / 4096   # same scale as the sample

    _, labels, inertia = vq_kmeans(vt, C, 8, with_labels=True)
    torch.cuda.synchronize()
    e = inertia.cpu().numpy()
    assert e[0] <= e0 * (1 + 1e-6) and np.all(np.diff(e) <= 1e-6 * e[:-1]), e
    v = vt.cpu().numpy().astype(np.float64)
    lab = labels.cpu().numpy().astype(np.int64)
    counts = np.bincount(lab, minlength=n_c)
    sums = np.zeros((n_c, d))
    np.add.at(sums, lab, v)
    got = C.cpu().numpy()
    has = counts > 0
    mean = sums[has] / counts[has, None]
    assert np.all(np.abs(got[has] - mean) <= 2 * U * np.abs(mean) + 1e-12)
    print(f"[kmeans] full size: N={N}, inertia {e0:.6g} -> {e[-1]:.6g}, {int((~has).sum())} empty")
