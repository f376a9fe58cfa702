"""fp64 oracle of the TransX memory codec.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and the CPU-baseline leg of
``bench.py``); the product path never imports it.

Source: TransX technical report (paper-daily), s.3 (memory published to the
online cache): each key or value vector is split into its length and its
direction; the length is stored apart and only the direction is compressed.
The direction vectors' covariance is estimated from a sample, eigendecomposed,
and every direction is rotated by the full orthogonal matrix of eigenvectors
(no dimension is dropped); rotated coordinate i then has variance lambda_i
(its "energy"), and bits are handed out by energy under a fixed total.

Readings where the page is silent (each one is an assumption, listed with the
others in the design notes):
  * the vector is the per-head slice (d_h values) of a key or value row;
    each head has its own rotation and bit table;
  * covariance is the centred sample covariance of the unit directions; the
    rotation's columns are eigenvectors sorted by eigenvalue, largest first;
  * bit allocation: integers b_i in [0, b_max], sum_i b_i = budget, built
    greedily by handing one bit at a time to the coordinate with the largest
    lambda_i * 4^(-b_i) (ties to the lower index) - the integer form of the
    reverse water-filling rule b_i = b + log2(lambda_i / geomean(lambda)) / 2;
  * quantiser: uniform, mid-rise, on [m_i - a_i, m_i + a_i] with m_i the mean
    of rotated coordinate i and a_i = 3 sqrt(lambda_i); code =
    clamp(floor((x - m_i + a_i) / (2 a_i) * 2^b_i), 0, 2^b_i - 1),
    reconstruction at the cell centre; a coordinate with b_i = 0 is
    reconstructed as m_i;
  * the decoded vector is norm * E x_hat (not renormalised); a zero vector
    has norm 0 and decodes to zero;
  * storage: norm as fp32, codes packed least-significant bit first into
    32-bit words, coordinate 0 first, budget / 32 words per vector.
Parity pins: tests/test_oracle_codec.py.
"""
from __future__ import annotations

import numpy as np

RANGE_SIGMAS = 3.0


def allocate_bits(lam, budget: int, b_max: int = 8) -> np.ndarray:
    """Greedy integer bit allocation by energy (see the module notes)."""
    lam = np.asarray(lam, dtype=np.float64)
    n = lam.shape[0]
    if budget < 0 or budget > n * b_max:
        raise ValueError("budget must lie in [0, n * b_max]")
    b = np.zeros(n, dtype=np.int64)
    for _ in range(budget):
        best, best_v = -1, -1.0
        for i in range(n):
            if b[i] >= b_max:
                continue
            v = lam[i] * 4.0 ** (-b[i])
            if v > best_v:
                best, best_v = i, v
        b[best] += 1
    return b


def fit(X, heads: int, budget: int, b_max: int = 8) -> dict:
    """Codebook from a calibration sample X [n, d]: per head h the rotation
    rot[h] (d_h x d_h, column i = i-th eigenvector), energies lam[h], bits[h],
    centres[h] and half-ranges[h] of the rotated coordinates."""
    X = np.asarray(X, dtype=np.float64)
    n, d = X.shape
    dh = d // heads
    out = {"rot": np.zeros((heads, dh, dh)), "lam": np.zeros((heads, dh)),
           "bits": np.zeros((heads, dh), dtype=np.int64), "center": np.zeros((heads, dh)),
           "half": np.zeros((heads, dh)), "budget": int(budget)}
    for h in range(heads):
        x = X[:, h * dh:(h + 1) * dh]
        nrm = np.linalg.norm(x, axis=1)
        keep = nrm > 0
        u = x[keep] / nrm[keep, None]
        mu = u.mean(axis=0)
        cov = (u - mu).T @ (u - mu) / u.shape[0]
        lam, E = np.linalg.eigh(cov)
        order = np.argsort(-lam, kind="stable")
        lam = np.maximum(lam[order], 0.0)
        E = E[:, order]
        out["rot"][h] = E
        out["lam"][h] = lam
        out["bits"][h] = allocate_bits(lam, budget, b_max)
        out["center"][h] = E.T @ mu
        out["half"][h] = RANGE_SIGMAS * np.sqrt(lam)
    return out


def quantize(xr, center, half, bits) -> np.ndarray:
    """Codes of rotated coordinates xr [..., d_h] (0 where bits == 0)."""
    xr = np.asarray(xr, dtype=np.float64)
    levels = 2.0 ** bits
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.floor((xr - center + half) / (2.0 * half) * levels)
    t = np.where(bits > 0, t, 0.0)
    return np.clip(np.nan_to_num(t), 0, levels - 1).astype(np.int64)


def dequantize(codes, center, half, bits) -> np.ndarray:
    """Cell centres of the codes (the centre m_i where bits == 0)."""
    levels = 2.0 ** bits
    step = 2.0 * half / levels
    return np.where(bits > 0, center - half + (np.asarray(codes) + 0.5) * step, center)


def encode(X, cb: dict):
    """X [n, d] -> (norms [n, heads] fp64, codes [n, heads, d_h] int)."""
    X = np.asarray(X, dtype=np.float64)
    heads, dh = cb["bits"].shape
    n = X.shape[0]
    norms = np.zeros((n, heads))
    codes = np.zeros((n, heads, dh), dtype=np.int64)
    for h in range(heads):
        x = X[:, h * dh:(h + 1) * dh]
        nrm = np.linalg.norm(x, axis=1)
        u = np.divide(x, nrm[:, None], out=np.zeros_like(x), where=nrm[:, None] > 0)
        xr = u @ cb["rot"][h]
        norms[:, h] = nrm
        codes[:, h] = quantize(xr, cb["center"][h], cb["half"][h], cb["bits"][h])
    return norms, codes


def rotated_values(X, cb: dict) -> np.ndarray:
    """Rotated unit-direction coordinates [n, heads, d_h] before quantisation
    (for tests that check which codes lie near a decision boundary)."""
    X = np.asarray(X, dtype=np.float64)
    heads, dh = cb["bits"].shape
    out = np.zeros((X.shape[0], heads, dh))
    for h in range(heads):
        x = X[:, h * dh:(h + 1) * dh]
        nrm = np.linalg.norm(x, axis=1)
        u = np.divide(x, nrm[:, None], out=np.zeros_like(x), where=nrm[:, None] > 0)
        out[:, h] = u @ cb["rot"][h]
    return out


def decode(norms, codes, cb: dict) -> np.ndarray:
    """(norms, codes) -> vectors [n, d]: norm * E x_hat per head."""
    heads, dh = cb["bits"].shape
    n = np.asarray(norms).shape[0]
    out = np.zeros((n, heads * dh))
    for h in range(heads):
        xh = dequantize(codes[:, h], cb["center"][h], cb["half"][h], cb["bits"][h])
        out[:, h * dh:(h + 1) * dh] = np.asarray(norms)[:, h, None] * (xh @ cb["rot"][h].T)
    return out


def pack(codes, bits) -> np.ndarray:
    """codes [n, heads, d_h], bits [heads, d_h] -> words [n, heads, budget/32]
    uint32 (least-significant bit first, coordinate 0 first)."""
    codes = np.asarray(codes, dtype=np.int64)
    n, heads, dh = codes.shape
    budget = int(np.sum(bits[0]))
    assert all(int(np.sum(bits[h])) == budget for h in range(heads)) and budget % 32 == 0
    words = np.zeros((n, heads, budget // 32), dtype=np.uint64)
    for h in range(heads):
        off = 0
        for i in range(dh):
            b = int(bits[h, i])
            for k in range(b):
                bit = (codes[:, h, i] >> k) & 1
                pos = off + k
                words[:, h, pos // 32] |= bit.astype(np.uint64) << np.uint64(pos % 32)
            off += b
    return words.astype(np.uint32)


def unpack(words, bits) -> np.ndarray:
    """Inverse of pack."""
    words = np.asarray(words, dtype=np.uint64)
    n, heads, _ = words.shape
    dh = bits.shape[1]
    codes = np.zeros((n, heads, dh), dtype=np.int64)
    for h in range(heads):
        off = 0
        for i in range(dh):
            b = int(bits[h, i])
            v = np.zeros(n, dtype=np.int64)
            for k in range(b):
                pos = off + k
                v |= (((words[:, h, pos // 32] >> np.uint64(pos % 32)) & np.uint64(1))
                      .astype(np.int64) << k)
            codes[:, h, i] = v
            off += b
    return codes
