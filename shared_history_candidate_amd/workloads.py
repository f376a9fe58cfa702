"""Seeded synthetic inputs for shared-history cross-attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the GPU path's tests/bench and the CPU oracle read
the arrays it returns, so the two sides always see identical inputs.

Shapes and distributions follow the workloads the pages describe:
  * ReST-like serving (ReST reading note, s.3.3 and s.5.3): d = 256, q = 3
    token-specific query tokens ([CLS]/ad/user), memory = encoder output H used
    as both K and V, ragged history lengths;
  * long history (ReST reading note s.5.3, length axis up to 16k, width 512);
  * TransX-like memory (TransX report s.2): 64 recent + 32 chunk-summary slots
    with separate K and V, one query per candidate, ~1000 candidates per
    request (EST article s.1: thousands of candidates per request);
  * ragged shared-prefix training batch (ReST reading note s.3.5 ULT; TransX
    report s.2 trajectory packing): lognormal history lengths, 1..64
    candidates per user.

Draw order (numpy PCG64, ``default_rng(seed)``): memory lengths, candidate
counts, H (or K then V), Z, W_Q slots in order.  Values are standard normal
(float32 draws); W_Q has variance 1/d.  In bf16 mode every array is rounded to
the nearest bf16 value (round-to-nearest-even) and kept as float32 holding
that exact value, so converting it to bf16 on the device is exact and the
oracle reads the same numbers upcast to fp64.

W_Q is returned output-major: ``wt[s][o][i]`` is W_Q[s] of Eq. (7) at (i, o).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

__all__ = ["Workload", "CONFIGS", "make", "custom", "round_bf16", "output_weights",
           "attention_like", "prefix_lengths", "output_grad", "anisotropic_memory"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    arrays whose low 16 mantissa bits are zero.  Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    q: int
    d: int
    heads: int
    dtype: str                 # "bf16" or "fp32"
    kv_mode: str               # "shared" (K = V = H) or "separate"
    cu_kv: np.ndarray          # int32 [R+1]
    cu_cand: np.ndarray        # int32 [R+1]
    Z: np.ndarray              # float32 [total_cand, q, d]
    wt: np.ndarray             # float32 [q, d, d]  output-major W_Q
    K: np.ndarray              # float32 [total_kv, d]  (= H in shared mode)
    V: Optional[np.ndarray]    # float32 [total_kv, d] or None in shared mode
    seed: int = 0
    info: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return len(self.cu_kv) - 1

    @property
    def total_cand(self) -> int:
        return int(self.cu_cand[-1])

    @property
    def total_kv(self) -> int:
        return int(self.cu_kv[-1])

    @property
    def rows(self) -> int:
        return self.total_cand * self.q

    @property
    def d_h(self) -> int:
        return self.d // self.heads

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_kv)

    @property
    def cands(self) -> np.ndarray:
        return np.diff(self.cu_cand)

    def flops(self) -> float:
        """Algorithmic FLOPs of one pass: projection 2*rows*d*d plus
        QK^T and PV, 4 * sum_r M_r * L_r * d."""
        m = self.cands.astype(np.float64) * self.q
        return 2.0 * self.rows * self.d * self.d + 4.0 * float(np.sum(m * self.lengths)) * self.d

    def bytes(self) -> float:
        """Algorithmic HBM bytes of one pass: K (and V), Z, W_Q, O, each once."""
        b = 2 if self.dtype == "bf16" else 4
        kv = (1 if self.kv_mode == "shared" else 2) * self.total_kv * self.d
        return float(b * (kv + 2 * self.rows * self.d + self.q * self.d * self.d))

    def flops_projection(self) -> float:
        """FLOPs of the TSP projection alone: 2 * rows * d * d."""
        return 2.0 * self.rows * self.d * self.d

    def bytes_projection(self) -> float:
        """Bytes the projection must move: Z and W_Q in, Q out."""
        b = 2 if self.dtype == "bf16" else 4
        return float(b * (2 * self.rows * self.d + self.q * self.d * self.d))

    def flops_attention(self, kv_len: Optional[np.ndarray] = None) -> float:
        """FLOPs of QK^T and PV: 4 * sum_r M_r * L_r * d; with per-candidate
        prefix lengths, 4 * q * d * sum_c clamp(kv_len[c], 0, L_r)."""
        if kv_len is not None:
            return 4.0 * self.q * self.d * float(np.sum(self._visible(kv_len)))
        m = self.cands.astype(np.float64) * self.q
        return 4.0 * float(np.sum(m * self.lengths)) * self.d

    def _visible(self, kv_len: np.ndarray) -> np.ndarray:
        """Memory rows each candidate sees under a prefix length."""
        L = np.repeat(self.lengths, self.cands)
        return np.clip(np.asarray(kv_len, dtype=np.int64), 0, L)

    def flops_backward(self, kv_len: Optional[np.ndarray] = None) -> float:
        """Algorithmic FLOPs of the backward pass: scores recomputed, dP, dQ,
        dK and dV (10 * sum_r M_r * L_r * d, or 10 * q * d * sum_c n_c with
        per-candidate prefix lengths), dZ and dW_Q (4 * rows * d * d)."""
        if kv_len is not None:
            att = 10.0 * self.q * self.d * float(np.sum(self._visible(kv_len)))
        else:
            m = self.cands.astype(np.float64) * self.q
            att = 10.0 * float(np.sum(m * self.lengths)) * self.d
        return att + 4.0 * self.rows * self.d * self.d

    def bytes_backward(self) -> float:
        """Algorithmic bytes of the backward pass: Z, W_Q, K (and V), dO in;
        dZ, dK (and dV) out, dW_Q out in fp32."""
        b = 2 if self.dtype == "bf16" else 4
        kv = (1 if self.kv_mode == "shared" else 2) * self.total_kv * self.d
        return float(b * (3 * self.rows * self.d + self.q * self.d * self.d + 2 * kv)
                     + 4 * self.q * self.d * self.d)

    def flops_output(self) -> float:
        """FLOPs of the gate and output projections of Eq. (7): 4 * rows * d * d."""
        return 4.0 * self.rows * self.d * self.d

    def bytes_output(self) -> float:
        """Bytes the output stage must move: Z, O in, Y out, W_go and W_o."""
        b = 2 if self.dtype == "bf16" else 4
        return float(b * (3 * self.rows * self.d + (self.q + 1) * self.d * self.d))

    def bytes_attention(self, kv_len: Optional[np.ndarray] = None) -> float:
        """Bytes the attention over projected queries must move: K (and V), Q, O.
        With per-candidate prefix lengths only the rows some candidate of the
        request sees (the longest prefix) count, plus the lengths themselves."""
        b = 2 if self.dtype == "bf16" else 4
        rows_kv = self.total_kv
        extra = 0
        if kv_len is not None:
            vis = self._visible(kv_len)
            rows_kv = sum(int(vis[a:c].max()) if c > a else 0
                          for a, c in zip(self.cu_cand[:-1], self.cu_cand[1:]))
            extra = 4 * self.total_cand
        kv = (1 if self.kv_mode == "shared" else 2) * rows_kv * self.d
        return float(b * (kv + 2 * self.rows * self.d) + extra)


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def custom(name: str, lengths: Sequence[int], cands: Sequence[int], q: int, d: int,
           heads: int, dtype: str = "bf16", kv_mode: str = "shared", seed: int = 0,
           wq_std: Optional[float] = None, rng=None, info=None) -> Workload:
    """Build a workload with the given per-request memory lengths and candidate
    counts.  Draws H (or K then V), Z, then W_Q slots from ``rng`` (or from
    ``default_rng(seed)``)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    cands = np.asarray(cands, dtype=np.int64)
    assert lengths.shape == cands.shape
    cu_kv = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu_kv[1:] = np.cumsum(lengths)
    cu_cand = np.zeros(len(cands) + 1, dtype=np.int32)
    cu_cand[1:] = np.cumsum(cands)
    total_kv, total_cand = int(cu_kv[-1]), int(cu_cand[-1])
    K = _normal(rng, (total_kv, d))
    V = _normal(rng, (total_kv, d)) if kv_mode == "separate" else None
    Z = _normal(rng, (total_cand, q, d))
    wt = _normal(rng, (q, d, d), std=(wq_std if wq_std is not None else 1.0 / np.sqrt(d)))
    if dtype == "bf16":
        K = round_bf16(K)
        V = round_bf16(V) if V is not None else None
        Z = round_bf16(Z)
        wt = round_bf16(wt)
    elif dtype != "fp32":
        raise ValueError("dtype must be bf16 or fp32")
    return Workload(name=name, q=q, d=d, heads=heads, dtype=dtype, kv_mode=kv_mode,
                    cu_kv=cu_kv, cu_cand=cu_cand, Z=Z, wt=wt, K=K, V=V, seed=seed,
                    info=dict(info or {}))


def _tiny(seed):
    # 1 request, L = 64, d = 64 (2 heads x 32), K = V = H, 4 candidates x 3
    # query tokens, W_Q ~ N(0, 1/64) per slot, fp32.
    return custom("tiny_fp32", [64], [4], q=3, d=64, heads=2, dtype="fp32",
                  kv_mode="shared", seed=seed)


def _rest(seed):
    # 8 requests, L ~ U{512..1024}, d = 256 (4 x 64), K = V = H, 256
    # candidates x 3 TSP query tokens per request.
    rng = np.random.default_rng(seed)
    R = 8
    lengths = rng.integers(512, 1025, size=R)
    cands = np.full(R, 256)
    return custom("rest_bf16", lengths, cands, q=3, d=256, heads=4, dtype="bf16",
                  kv_mode="shared", seed=seed, rng=rng)


def _long(seed):
    # 4 requests, L = 16384, d = 512 (8 x 64), K = V = H, 512 candidates x 3.
    rng = np.random.default_rng(seed)
    R = 4
    return custom("long_bf16", np.full(R, 16384), np.full(R, 512), q=3, d=512, heads=8,
                  dtype="bf16", kv_mode="shared", seed=seed, rng=rng)


def _transx(seed):
    # 256 requests, 96 memory slots (64 recent + 32 chunk summaries), separate
    # K and V, d = 256 (4 x 64), 1024 candidates x 1 query token.
    rng = np.random.default_rng(seed)
    R = 256
    return custom("transx_bf16", np.full(R, 96), np.full(R, 1024), q=1, d=256, heads=4,
                  dtype="bf16", kv_mode="separate", seed=seed, rng=rng,
                  info={"recent": 64, "summaries": 32})


def _ragged(seed):
    # 64 users, L = clip(rint(exp(N(7.5, 0.6^2))), 256, 4096), candidates per
    # user ~ U{1..64}, d = 256 (8 x 32), K = V = H, 3 TSP query tokens.
    rng = np.random.default_rng(seed)
    R = 64
    lengths = np.clip(np.rint(np.exp(rng.normal(7.5, 0.6, size=R))), 256, 4096).astype(np.int64)
    cands = rng.integers(1, 65, size=R)
    return custom("ragged_bf16", lengths, cands, q=3, d=256, heads=8, dtype="bf16",
                  kv_mode="shared", seed=seed, rng=rng)


def output_weights(wl: Workload, seed: int = 0):
    """Gate and output weights of Eq. (7) for a workload: W_go [q][d][d] (one
    set per query slot, output-major) and W_o [d][d] (output-major), each
    N(0, 1/d) like W_Q, drawn from default_rng(seed) in that order and rounded
    to bf16 in bf16 mode (float32 arrays holding the exact values)."""
    rng = np.random.default_rng(seed)
    std = 1.0 / np.sqrt(wl.d)
    wgo = _normal(rng, (wl.q, wl.d, wl.d), std=std)
    wo = _normal(rng, (wl.d, wl.d), std=std)
    if wl.dtype == "bf16":
        wgo, wo = round_bf16(wgo), round_bf16(wo)
    return wgo, wo


def attention_like(wl: Workload, seed: int = 0, std: float = 0.5) -> np.ndarray:
    """A stand-in attention output [total_cand][q][d] for testing the output
    stage alone: N(0, std^2) draws from default_rng(seed), bf16-rounded in bf16
    mode."""
    rng = np.random.default_rng(seed)
    O = _normal(rng, (wl.total_cand, wl.q, wl.d), std=std)
    return round_bf16(O) if wl.dtype == "bf16" else O


def anisotropic_memory(wl: Workload, seed: int = 0, decay: float = 0.85, shift: float = 0.3):
    """Memory rows whose per-head directions have a decaying spectrum (most
    energy in a few directions, as the TransX report s.3 observes for its
    memory), for the coded-memory tests: per head h a random orthogonal basis
    B_h (QR of a Gaussian matrix), rows (g * decay^i + shift) B_h^T with g
    N(0, 1), times a norm from U[0.5, 2].  Returns (K, V) [total_kv, d]
    (V is None in projection-free mode), bf16-rounded in bf16 mode; draws
    from default_rng(seed): bases, then K, then V."""
    rng = np.random.default_rng(seed)
    dh = wl.d // wl.heads
    bases = [np.linalg.qr(rng.normal(size=(dh, dh)))[0] for _ in range(wl.heads)]
    scales = decay ** np.arange(dh)

    def draw():
        X = np.zeros((wl.total_kv, wl.d))
        for h in range(wl.heads):
            g = rng.normal(size=(wl.total_kv, dh))
            X[:, h * dh:(h + 1) * dh] = (g * scales + shift) @ bases[h].T
        X *= rng.uniform(0.5, 2.0, size=(wl.total_kv, 1))
        X = X.astype(np.float32)
        return round_bf16(X) if wl.dtype == "bf16" else X

    K = draw()
    V = draw() if wl.kv_mode == "separate" else None
    return K, V


def output_grad(wl: Workload, seed: int = 0) -> np.ndarray:
    """A loss gradient dO [total_cand][q][d] for the backward pass: N(0, 1)
    draws from default_rng(seed), bf16-rounded in bf16 mode."""
    rng = np.random.default_rng(seed)
    g = _normal(rng, (wl.total_cand, wl.q, wl.d))
    return round_bf16(g) if wl.dtype == "bf16" else g


def prefix_lengths(wl: Workload, seed: int = 0, out_of_range: bool = True) -> np.ndarray:
    """Per-candidate memory prefix lengths [total_cand] int32 for the prefix
    cutoff (ReST reading note s.3.5, ULT: the samples of one user are ordered
    in time and each sees the part of the history before it).  Request r's
    candidates get sorted draws from U{0..L_r}; with out_of_range, about one
    in eight is replaced by a value below 0 or above L_r, which the method
    clamps.  Drawn from default_rng(seed), request by request."""
    rng = np.random.default_rng(seed)
    out = np.zeros(wl.total_cand, dtype=np.int32)
    for r in range(wl.R):
        a, b = int(wl.cu_cand[r]), int(wl.cu_cand[r + 1])
        L = int(wl.lengths[r])
        v = np.sort(rng.integers(0, L + 1, size=b - a))
        if out_of_range and b > a:
            hit = rng.random(b - a) < 0.125
            wild = np.where(rng.random(b - a) < 0.5, -rng.integers(1, 5, size=b - a),
                            L + rng.integers(1, 100, size=b - a))
            v = np.where(hit, wild, v)
        out[a:b] = v
    return out


CONFIGS = {
    "tiny": _tiny,       # 1 request, L=64, d=64, fp32
    "rest": _rest,       # ReST-like serving batch, bf16
    "long": _long,       # long history L=16384, d=512, bf16
    "transx": _transx,   # TransX-like 96-slot memory, separate K/V, bf16
    "ragged": _ragged,   # ragged shared-prefix training batch, bf16
}


def make(config: str, seed: int = 0) -> Workload:
    """Generate one of the named workloads (see CONFIGS) with the given seed."""
    try:
        return CONFIGS[config](seed)
    except KeyError:
        raise ValueError("unknown config %r (choose from %s)" % (config, sorted(CONFIGS)))
