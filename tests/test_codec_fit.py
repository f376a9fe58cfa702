"""The library's codebook fit (xattn_codec_fit, host C++) against the oracle's
fit (oracle/codec.py), and its host validation.  No GPU is needed: the fit is
offline calibration on the host.

The two share no code: the library runs its own Jacobi eigensolver in fp64
and writes fp32 codebooks; the oracle calls numpy's symmetric eigensolver.
An eigenvector's sign is arbitrary, so rotation columns and centres are
compared up to each column's sign; bit tables must be identical, half-ranges
and centres equal to fp32 rounding, and the library's rotation orthogonal.
The codebooks are then used the same way: encode/decode of held-out rows with
the oracle's quantiser gives the same reconstruction error under both."""
import ctypes

import numpy as np
import pytest

from oracle import codec as OC
from shared_history_candidate_amd import workloads as W
from shared_history_candidate_amd import xattn as X


def _sample(dh, heads, mode, seed):
    wl = W.custom("fit", [1500, 700, 3], [2, 1, 1], q=1, d=dh * heads, heads=heads,
                  dtype="bf16", kv_mode=mode, seed=seed)
    K, V = W.anisotropic_memory(wl, seed + 1)
    return K if V is None else V


@pytest.mark.parametrize("dh,heads,bpc", [(32, 4, 4), (64, 4, 4.5), (128, 2, 3), (64, 2, 8),
                                          (64, 2, 0.5)])
def test_fit_matches_oracle(dh, heads, bpc):
    Xs = _sample(dh, heads, "separate", dh + int(bpc * 2))
    budget = int(round(bpc * dh / 32.0)) * 32
    lib = X.codec_fit(Xs, heads, budget)
    orc = OC.fit(Xs, heads, budget)
    assert lib["bits"].shape == (heads, dh)
    assert np.array_equal(lib["bits"].astype(np.int64), orc["bits"])
    assert np.all(lib["bits"].sum(axis=1) == budget)
    np.testing.assert_allclose(lib["half"], orc["half"], rtol=2e-6, atol=1e-7)
    E = lib["rot"].astype(np.float64)
    for h in range(heads):
        np.testing.assert_allclose(E[h].T @ E[h], np.eye(dh), atol=2e-6)
        sg = np.sign(np.sum(E[h] * orc["rot"][h], axis=0))
        np.testing.assert_allclose(E[h] * sg[None, :], orc["rot"][h], atol=2e-5)
        np.testing.assert_allclose(lib["center"][h] * sg, orc["center"][h], atol=2e-6)
        # the library's sign convention: largest-magnitude entry positive
        idx = np.argmax(np.abs(E[h]), axis=0)
        assert np.all(E[h][idx, np.arange(dh)] > 0)


def test_fitted_codebooks_reconstruct_alike():
    """Held-out rows encoded and decoded (oracle quantiser) with either fit:
    the same mean reconstruction error."""
    heads, dh = 4, 64
    fit_rows = _sample(dh, heads, "shared", 3)
    held = _sample(dh, heads, "shared", 4)
    lib = X.codec_fit(fit_rows, heads, 288)
    orc = OC.fit(fit_rows, heads, 288)
    libd = {k: (np.asarray(v, dtype=np.float64) if k != "bits" else v.astype(np.int64))
            for k, v in lib.items() if k != "budget"}
    errs = []
    for cb in (libd, orc):
        n, c = OC.encode(held, cb)
        errs.append(np.mean((OC.decode(n, c, cb) - held) ** 2))
    assert abs(errs[0] - errs[1]) <= 1e-3 * errs[1], errs


def test_fit_host_validation():
    L = X.lib()
    Xs = np.ones((4, 128), dtype=np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    bits = np.zeros((2, 64), dtype=np.uint8)
    f = np.zeros((2, 64), dtype=np.float32)
    rot = np.zeros((2, 64, 64), dtype=np.float32)

    def fit(d=128, heads=2, Xp=p(Xs), n=4, budget=256, b=p(bits)):
        return L.xattn_codec_fit(d, heads, Xp, n, budget, b, p(f), p(f), p(rot))

    assert fit() == X.XATTN_OK
    assert fit(Xp=None) == X.XATTN_EINVAL
    assert fit(b=None) == X.XATTN_EINVAL
    assert fit(heads=3) == X.XATTN_EINVAL
    assert fit(n=0) == X.XATTN_EINVAL
    assert fit(budget=8 * 64 + 1) == X.XATTN_EUNSUPPORTED
    Z = np.zeros((4, 128), dtype=np.float32)
    assert fit(Xp=p(Z)) == X.XATTN_EINVAL          # a head with no usable row
