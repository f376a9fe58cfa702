"""Pins for the fp64 oracle of the TransX memory codec (oracle/codec.py).

The page (TransX report s.3) fixes the structure - norm apart, direction
rotated by the full eigenvector basis of its covariance, bits by energy under
a fixed total - but not the quantiser, the allocation rule's integer form or
the rounding, so those parts are pinned to their own definitions written out
(stated in the module) and to what the mathematics fixes:
  * the rotation is orthogonal and diagonalises the sample covariance;
  * the integer allocation meets the budget, the cap and the energy order,
    and equals the reverse water-filling closed form where that is integral;
  * a coordinate inside the quantiser's range is reconstructed within half a
    step, a cell centre is its own reconstruction, out-of-range values clamp;
  * packing round-trips and matches a hand-packed word;
  * the decoded vector keeps the stored norm and direction to the
    quantisation bound.
A mutation test plants plausible mistakes in copies of the module and checks
that these pins catch each of them.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle import codec as C0

HERE = os.path.dirname(os.path.abspath(__file__))


def _sample(rng, n=4000, d=32, heads=2, decay=0.7):
    """Directions with a decaying spectrum (most energy in few coordinates),
    norms spread over [0.5, 3]."""
    dh = d // heads
    scales = decay ** np.arange(dh)
    X = np.zeros((n, d))
    for h in range(heads):
        B = np.linalg.qr(rng.normal(size=(dh, dh)))[0]
        X[:, h * dh:(h + 1) * dh] = (rng.normal(size=(n, dh)) * scales + 0.3) @ B.T
    return X * rng.uniform(0.5, 3.0, size=(n, 1))


def _check_rotation(C, seed):
    rng = np.random.default_rng(seed)
    X = _sample(rng)
    cb = C.fit(X, heads=2, budget=64)
    err = 0.0
    for h in range(2):
        E = cb["rot"][h]
        err = max(err, np.max(np.abs(E.T @ E - np.eye(E.shape[0]))))
        x = X[:, h * 16:(h + 1) * 16]
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        xr = u @ E
        cov = np.cov(xr.T, bias=True)
        err = max(err, np.max(np.abs(cov - np.diag(cb["lam"][h]))))
        err = max(err, np.max(np.abs(xr.mean(axis=0) - cb["center"][h])))
        assert np.all(np.diff(cb["lam"][h]) <= 1e-15)
    return err


def test_rotation_is_orthogonal_and_diagonalises():
    assert _check_rotation(C0, 0) < 1e-12


def _check_alloc_closed_form(C):
    # reverse water-filling: b_i = b + log2(lam_i / geomean) / 2 is integral here
    b = C.allocate_bits([64.0, 16.0, 4.0, 1.0], 10)
    return list(b) == [4, 3, 2, 1]


def _check_alloc_properties(C, seed):
    rng = np.random.default_rng(seed)
    ok = True
    for _ in range(20):
        n = int(rng.integers(2, 40))
        lam = np.sort(rng.exponential(size=n))[::-1] * rng.uniform(0.1, 10)
        budget = int(rng.integers(0, n * 8 + 1))
        b = C.allocate_bits(lam, budget, 8)
        ok &= int(b.sum()) == budget and b.max(initial=0) <= 8 and b.min(initial=0) >= 0
        ok &= bool(np.all(np.diff(b) <= 0))           # more energy, never fewer bits
    ok &= list(C.allocate_bits(np.ones(6), 18)) == [3] * 6
    ok &= list(C.allocate_bits([1.0, 0.0, 0.0], 3)) == [3, 0, 0]
    return ok


def test_allocation_closed_form():
    assert _check_alloc_closed_form(C0)


def test_allocation_properties():
    assert _check_alloc_properties(C0, 1)


def _check_quantizer(C, seed):
    """Returns the largest (error / half step) over in-range values; cell
    centres and clamping checked exactly."""
    rng = np.random.default_rng(seed)
    center = rng.normal(size=8)
    half = rng.uniform(0.1, 2.0, size=8)
    bits = np.array([8, 6, 5, 4, 3, 2, 1, 0])
    x = center + half * rng.uniform(-0.999, 0.999, size=(5000, 8))
    codes = C.quantize(x, center, half, bits)
    xr = C.dequantize(codes, center, half, bits)
    step = 2 * half / 2.0 ** bits
    worst = float(np.max((np.abs(xr - x) / (step / 2))[:, :7]))
    assert np.all(xr[:, 7] == center[7]) and np.all(codes[:, 7] == 0)
    # centres map to themselves
    cc = np.arange(2 ** 4)
    xc = center[3] - half[3] + (cc + 0.5) * step[3]
    assert np.array_equal(C.quantize(xc[:, None], center[3:4], half[3:4], bits[3:4])[:, 0], cc)
    # clamping
    far = np.array([[center[0] - 10 * half[0]], [center[0] + 10 * half[0]]])
    assert list(C.quantize(far, center[:1], half[:1], bits[:1])[:, 0]) == [0, 255]
    return worst


def test_quantizer_half_step_bound():
    assert _check_quantizer(C0, 2) <= 1.0 + 1e-9


def _check_pack(C):
    bits = np.array([[3, 5, 8, 8, 8, 0]])            # 32 bits
    codes = np.array([[[5, 17, 200, 1, 255, 0]]])
    words = C.pack(codes, bits)
    # hand-packed, least-significant bit first: 5 | 17<<3 | 200<<8 | 1<<16 | 255<<24
    want = 5 | (17 << 3) | (200 << 8) | (1 << 16) | (255 << 24)
    ok = int(words[0, 0, 0]) == want
    rng = np.random.default_rng(3)
    bits2 = np.array([[7, 7, 6, 5, 4, 3, 0, 0, 0], [8, 8, 8, 8, 0, 0, 0, 0, 0]])
    codes2 = np.stack([rng.integers(0, 2 ** bits2[h], size=(50, 9)) for h in range(2)], axis=1)
    ok &= np.array_equal(C.unpack(C.pack(codes2, bits2), bits2), codes2)
    return ok


def test_pack_layout_and_round_trip():
    assert _check_pack(C0)


def _check_round_trip(C, seed):
    """Decoded vector vs the original: per head, the error of the rotated
    direction is at most half a step per coordinate wherever no coordinate
    was clipped; norms are kept exactly.  Returns the worst ratio."""
    rng = np.random.default_rng(seed)
    X = _sample(rng, n=3000)
    cb = C.fit(X, heads=2, budget=96)
    norms, codes = C.encode(X, cb)
    Y = C.decode(norms, codes, cb)
    worst = 0.0
    for h in range(2):
        x = X[:, h * 16:(h + 1) * 16]
        nrm = np.linalg.norm(x, axis=1)
        assert np.allclose(norms[:, h], nrm, rtol=0, atol=1e-12)
        xr = (x / nrm[:, None]) @ cb["rot"][h]
        yr = (Y[:, h * 16:(h + 1) * 16] / nrm[:, None]) @ cb["rot"][h]
        inside = np.all(np.abs(xr - cb["center"][h]) < cb["half"][h], axis=1)
        step = 2 * cb["half"][h] / 2.0 ** cb["bits"][h]
        coded = cb["bits"][h] > 0
        ratio = np.abs(yr - xr)[inside][:, coded] / (step[coded] / 2)
        worst = max(worst, float(ratio.max()))
        # zero-bit coordinates are reconstructed at the mean
        assert np.allclose(yr[:, ~coded], cb["center"][h][~coded], atol=1e-12)
    return worst


def test_round_trip_bound():
    assert _check_round_trip(C0, 4) <= 1.0 + 1e-9


def test_zero_vector_decodes_to_zero():
    rng = np.random.default_rng(5)
    X = _sample(rng, n=500)
    cb = C0.fit(X, heads=2, budget=64)
    Z = np.zeros((3, 32))
    n, c = C0.encode(Z, cb)
    assert np.all(n == 0) and np.all(C0.decode(n, c, cb) == 0)


def test_size_accounting_matches_page_scale():
    """The page's sizes (28 KiB of bf16 memory to 8.5 KiB) correspond to about
    4.5 bits per coordinate with a 32-bit norm per 64-wide vector; check the
    accounting of this layout at that budget."""
    dh, budget = 64, 256 + 32    # 4.5 bits per coordinate
    bf16 = dh * 2
    coded = budget // 8 + 4
    assert abs(bf16 / coded - 28 / 8.5) / (28 / 8.5) < 0.05


MUTANTS = {
    "encode_rotation_transposed": ("xr = u @ cb[\"rot\"][h]\n        norms", "xr = u @ cb[\"rot\"][h].T\n        norms"),
    "alloc_wrong_exponent": ("v = lam[i] * 4.0 ** (-b[i])", "v = lam[i] * 2.0 ** (-b[i])"),
    "reconstruct_cell_start": ("center - half + (np.asarray(codes) + 0.5) * step", "center - half + np.asarray(codes) * step"),
    "center_not_subtracted": ("t = np.floor((xr - center + half)", "t = np.floor((xr + half)"),
    "pack_msb_first": ("words[:, h, pos // 32] |= bit.astype(np.uint64) << np.uint64(pos % 32)",
                       "words[:, h, pos // 32] |= bit.astype(np.uint64) << np.uint64(31 - pos % 32)"),
    "range_uses_variance": ("out[\"half\"][h] = RANGE_SIGMAS * np.sqrt(lam)", "out[\"half\"][h] = RANGE_SIGMAS * lam"),
    "eigen_order_ascending": ("order = np.argsort(-lam, kind=\"stable\")", "order = np.argsort(lam, kind=\"stable\")"),
}


def _load_mutant(tmp_path, name, old, new):
    src = open(C0.__file__).read()
    assert old in src, "mutation anchor for %s not found" % name
    path = tmp_path / ("codec_mut_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("codec_mut_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _all_pins(C):
    checks = {
        "rotation": lambda: _check_rotation(C, 0) < 1e-12,
        "alloc_closed": lambda: _check_alloc_closed_form(C),
        "alloc_props": lambda: _check_alloc_properties(C, 1),
        "quantizer": lambda: _check_quantizer(C, 2) <= 1.0 + 1e-9,
        "pack": lambda: _check_pack(C),
        "round_trip": lambda: _check_round_trip(C, 4) <= 1.0 + 1e-9,
    }
    fails = []
    for k, fn in checks.items():
        try:
            ok = bool(fn())
        except Exception:
            ok = False
        if not ok:
            fails.append(k)
    return fails


def test_unmutated_codec_passes_all_pins():
    assert _all_pins(C0) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_codec_mistake_is_caught(tmp_path, name):
    mod = _load_mutant(tmp_path, name, *MUTANTS[name])
    assert _all_pins(mod), "mutant %s passed every pin" % name
