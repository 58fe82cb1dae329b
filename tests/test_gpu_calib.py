"""GPU parity of the on-device calibration (covariance and eigenbasis)
against the CPU oracle's float64 definitions, and the rotated pipeline run
on a device-computed basis against the oracle given that same basis."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import bf16_dev, dev, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    need_gpu()
    from sparse_attention_key_amd import fathom

    fathom.lib()
    return fathom


def _cov_def(x):
    x = np.asarray(x, np.float64)
    xc = x - x.mean(axis=0)
    return xc.T @ xc / x.shape[0]


COV_CASES = [("klt_sample", 8192, 128), ("offset_ragged", 5000, 128), ("m1", 1, 128), ("m3_d97", 3, 97),
             ("d64", 2049, 64)]


def _cov_keys(case, m, D, P=3):
    g = np.random.default_rng(m * 131 + D)
    if case == "klt_sample":
        w = wl.WORKLOADS["host1m_klt"]
        xs = np.stack([wl.calibration_sample(w, p) for p in range(P)])
        return xs, bf16_dev(xs)
    xs = (g.standard_normal((P, m, D)) * np.exp(0.8 * g.standard_normal(D)) + 7.0).astype(np.float32)
    return xs, dev(xs)


@pytest.mark.parametrize("case,m,D", COV_CASES)
def test_covariance_matches_definition(F, orc, case, m, D):
    P = 3
    xs, keys = _cov_keys(case, m, D, P)
    say("calib covariance", case, P, m, D)
    cov, var = F.calib_covariance(keys)
    cov, var = cov.cpu().numpy(), var.cpu().numpy()
    for p in range(P):
        ref = _cov_def(xs[p])
        scale = max(np.abs(ref).max(), 1e-300)
        assert np.max(np.abs(cov[p] - ref)) <= 1e-11 * scale, p
        rv = orc.calib.channel_variance(xs[p])
        # the same float64 value up to summation order, rounded once to float32
        assert np.all(np.abs(var[p].astype(np.float64) - rv) <= np.spacing(np.abs(rv)) + 1e-30), p


@pytest.mark.parametrize("case,m,D", COV_CASES)
def test_variances_alone_equal_the_covariance_diagonal(F, case, m, D):
    """Asked for variances only, the library skips the covariance and sums
    the centred squares per channel in the covariance diagonal's own order:
    the variances must equal those of the full call bit for bit."""
    _, keys = _cov_keys(case, m, D)
    say("calib variances alone", case, m, D)
    _, var_full = F.calib_covariance(keys)
    cov, var_only = F.calib_covariance(keys, with_cov=False)
    assert cov is None
    assert torch.equal(var_only.view(torch.int32), var_full.view(torch.int32))


def _basis_checks(U, lam, C, ref_U, ref_lam):
    D = C.shape[0]
    lmax = max(float(ref_lam.max()), 1e-30)
    assert np.all(np.diff(lam) <= 0)
    assert np.max(np.abs(lam - ref_lam)) <= 2e-6 * lmax
    Ud = U.astype(np.float64)
    assert np.max(np.abs(Ud.T @ Ud - np.eye(D))) <= 2e-5
    assert np.max(np.abs(C @ Ud - Ud * lam.astype(np.float64))) <= 2e-5 * lmax
    # eigenvectors of well-separated eigenvalues agree with the oracle's up to sign
    gaps = np.minimum(np.abs(np.diff(ref_lam, prepend=np.inf)), np.abs(np.diff(ref_lam, append=-np.inf)))
    sep = gaps > 1e-3 * lmax
    dots = np.abs(np.sum(Ud * ref_U.astype(np.float64), axis=0))
    assert np.all(dots[sep] >= 1 - 1e-4)
    # sign convention: the largest-magnitude component of each column is positive
    idx = np.argmax(np.abs(U), axis=0)
    assert np.all(U[idx, np.arange(D)] > 0)


BASIS_CASES = ["klt_sample", "constructed", "identity", "d97", "d2"]


@pytest.mark.parametrize("case", BASIS_CASES)
def test_basis_matches_eigh(F, orc, case):
    g = np.random.default_rng(len(case) * 17)
    if case == "klt_sample":
        w = wl.WORKLOADS["host1m_klt"]
        samples = [wl.calibration_sample(w, p) for p in range(2)]
        covs = [_cov_def(x) for x in samples]
    elif case == "constructed":
        D = 128
        Q = np.linalg.qr(g.standard_normal((D, D)))[0]
        s2 = np.exp(np.linspace(2.0, -4.0, D))
        covs = [(Q * s2) @ Q.T]
    elif case == "identity":
        covs = [np.eye(128) * 2.5]
    elif case == "d97":
        x = g.standard_normal((4000, 97)) * np.exp(0.5 * g.standard_normal(97))
        covs = [_cov_def(x)]
    else:
        covs = [np.array([[2.0, 1.0], [1.0, 2.0]])]
    C = np.stack([(c + c.T) / 2 for c in covs])
    say("calib basis", case, C.shape)
    U, lam = F.calib_basis(dev(C))
    U, lam = U.cpu().numpy(), lam.cpu().numpy()
    for p in range(C.shape[0]):
        vals, vecs = np.linalg.eigh(C[p])
        order = np.argsort(-vals, kind="stable")
        _basis_checks(U[p], lam[p], C[p], vecs[:, order], np.clip(vals[order], 0, None))


def test_device_basis_drives_the_rotated_pipeline(F, orc):
    # the device basis and the oracle's agree to float32 accuracy, so the
    # rotated pipeline on either finds (nearly) the same winners; both runs
    # are on the GPU and the oracle only supplies its own basis
    w = wl.WORKLOADS["host1m_klt"]
    P, n = 2, 4000
    xs = bf16_dev(np.stack([wl.keys_host(w, p, n=n) for p in range(P)]))
    q = dev(np.stack([wl.queries(w, p) for p in range(P)]))
    samples = [wl.calibration_sample(w, p) for p in range(P)]
    say("rotated pipeline on a device basis")
    cov, _ = F.calib_covariance(bf16_dev(np.stack(samples)))
    U, lam = F.calib_basis(cov)
    refU, reflam = zip(*(orc.calib.klt_basis(x) for x in samples))
    results = []
    for rot, s2 in ((U, lam), (dev(np.stack(refU)), dev(np.stack(reflam)))):
        planes, scales = F.pack(xs, rot=rot)
        pl = F.plan(q, s2, w.budget, rot=rot)
        results.append(F.scan_topk(planes, scales, n, pl, w.k).idx.cpu().numpy())
    for p in range(P):
        for h in range(w.G):
            common = len(set(results[0][p, h]) & set(results[1][p, h]))
            assert common >= 0.98 * w.k, (p, h, common)
