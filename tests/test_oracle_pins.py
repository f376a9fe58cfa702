"""Pins for the fp64 CPU oracle (oracle/xattn_oracle.c).

The oracle is the reference every GPU result is compared with, so it is first
pinned to things other than itself:
  * hand-derived closed-form cases stored under tests/golden/ (each cites the
    passage and shows its derivation);
  * library routines that compute the same definition by another route:
    numpy matmul for the TSP projection, torch's CPU float64
    scaled_dot_product_attention for the per-head attention;
  * mathematical identities: softmax-of-one-row, identical keys, zero query,
    two keys (logistic weight), the log-sum-exp gradient identity for K = V,
    translation equivariance, key-permutation invariance, shared-prefix
    equivalence (the pages' reason for sharing the memory), request
    independence, softmax rows summing to 1, and the Gaussian large-L limit;
  * integer plan: cu_q, row_req against numpy, tile coverage and ordering.
A mutation test at the end plants plausible mistakes in copies of the oracle
source and checks that these pins catch every one of them.
"""
import glob
import importlib.util
import json
import os
import shutil
import tempfile

import numpy as np
import pytest
import torch
from scipy.special import expit, logsumexp

import oracle
from shared_history_candidate_amd import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
_ALL_GOLDEN = sorted(glob.glob(os.path.join(HERE, "golden", "*.json")))
GOLDEN = [p for p in _ALL_GOLDEN if json.load(open(p)).get("kind", "forward") == "forward"]
GOLDEN_OUTPUT = [p for p in _ALL_GOLDEN if json.load(open(p)).get("kind") == "output"]


def _rand_case(rng, R=3, q=2, d=8, heads=2, kv_mode="separate", Lmax=9, Nmax=4):
    lengths = rng.integers(1, Lmax + 1, size=R)
    cands = rng.integers(1, Nmax + 1, size=R)
    return W.custom("rand", lengths, cands, q=q, d=d, heads=heads, dtype="fp32",
                    kv_mode=kv_mode, rng=rng)


def _oracle_out(orc, wl, **kw):
    return orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, **kw)


# ----------------------------------------------------------------------------
# Golden closed forms (hand-derived)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
def test_golden_closed_forms(oracle_mod, path):
    g = json.load(open(path))
    assert g["source"] and g["derivation"]
    V = np.array(g["V"]) if g["V"] is not None else None
    O = oracle_mod.forward(g["cu_kv"], g["cu_cand"], g["q"], g["heads"], np.array(g["Z"]),
                           np.array(g["wt"]), np.array(g["K"]), V)
    np.testing.assert_allclose(O, np.array(g["O"]), rtol=g["rtol"], atol=1e-15)


# ----------------------------------------------------------------------------
# Library cross-checks
# ----------------------------------------------------------------------------
def _check_projection(orc, seed):
    rng = np.random.default_rng(seed)
    q, d, n = 3, 16, 7
    Z = rng.standard_normal((n, q, d))
    wt = rng.standard_normal((q, d, d))
    Q = orc.project(Z, wt, q)
    ref = np.stack([Z[:, s, :] @ wt[s].T for s in range(q)], axis=1)
    return np.max(np.abs(Q - ref))


def test_projection_matches_numpy_matmul(oracle_mod):
    """Eq. (8): slot s of every candidate uses its own W_Q[s]."""
    assert _check_projection(oracle_mod, 0) < 1e-12


def _sdpa_reference(wl):
    """Per request and head: torch CPU float64 scaled_dot_product_attention on
    Q = Z W_Q[slot] (numpy matmul) and the head's column slices of K, V."""
    d, dh, q = wl.d, wl.d_h, wl.q
    Z = wl.Z.astype(np.float64).reshape(-1, q, d)
    Q = np.stack([Z[:, s, :] @ wl.wt[s].astype(np.float64).T for s in range(q)], axis=1)
    Q = Q.reshape(-1, d)
    K = wl.K.astype(np.float64)
    V = wl.V.astype(np.float64) if wl.V is not None else K
    out = np.zeros_like(Q)
    for r in range(wl.R):
        rows = slice(int(wl.cu_cand[r]) * q, int(wl.cu_cand[r + 1]) * q)
        kv = slice(int(wl.cu_kv[r]), int(wl.cu_kv[r + 1]))
        if rows.stop == rows.start or kv.stop == kv.start:
            continue
        qt = torch.from_numpy(Q[rows]).reshape(-1, wl.heads, dh).transpose(0, 1).unsqueeze(0)
        kt = torch.from_numpy(K[kv]).reshape(-1, wl.heads, dh).transpose(0, 1).unsqueeze(0)
        vt = torch.from_numpy(V[kv]).reshape(-1, wl.heads, dh).transpose(0, 1).unsqueeze(0)
        o = torch.nn.functional.scaled_dot_product_attention(qt.contiguous(), kt.contiguous(),
                                                             vt.contiguous())
        out[rows] = o.squeeze(0).transpose(0, 1).reshape(-1, d).numpy()
    return out


def _check_sdpa(orc, seed, kv_mode):
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=3, q=int(rng.integers(1, 4)), d=8,
                    heads=int(rng.choice([1, 2, 4])), kv_mode=kv_mode)
    return np.max(np.abs(_oracle_out(orc, wl) - _sdpa_reference(wl)))


@pytest.mark.parametrize("kv_mode", ["shared", "separate"])
@pytest.mark.parametrize("seed", range(6))
def test_matches_torch_sdpa_float64(oracle_mod, seed, kv_mode):
    assert _check_sdpa(oracle_mod, seed, kv_mode) < 1e-12


def test_config_tiny_matches_torch_sdpa(oracle_mod):
    wl = W.make("tiny", 0)
    assert np.max(np.abs(_oracle_out(oracle_mod, wl) - _sdpa_reference(wl))) < 1e-12


# ----------------------------------------------------------------------------
# Closed forms and identities
# ----------------------------------------------------------------------------
def _check_single_row(orc, seed):
    """L = 1: one weight equal to 1, so each head outputs the memory row's slice."""
    rng = np.random.default_rng(seed)
    wl = W.custom("l1", [1, 1], [3, 2], q=2, d=8, heads=4, dtype="fp32",
                  kv_mode="separate", rng=rng)
    O = _oracle_out(orc, wl)
    ref = np.concatenate([np.repeat(wl.V[r:r + 1], wl.cands[r] * wl.q, 0) for r in range(2)])
    return np.max(np.abs(O - ref))


def test_single_memory_row(oracle_mod):
    assert _check_single_row(oracle_mod, 1) == 0.0


def _check_identical_keys(orc, seed):
    """All keys equal: uniform weights, output = column mean of V."""
    rng = np.random.default_rng(seed)
    wl = W.custom("ik", [5], [3], q=2, d=8, heads=2, dtype="fp32", kv_mode="separate", rng=rng)
    wl.K[:] = wl.K[0:1]
    O = _oracle_out(orc, wl)
    return np.max(np.abs(O - wl.V.astype(np.float64).mean(0, keepdims=True)))


def test_identical_keys_give_mean_value(oracle_mod):
    assert _check_identical_keys(oracle_mod, 2) < 1e-14


def test_identical_memory_rows_pfkv(oracle_mod):
    """K = V = H with all rows equal: the output is that row."""
    rng = np.random.default_rng(3)
    wl = W.custom("ir", [7], [2], q=3, d=8, heads=2, dtype="fp32", kv_mode="shared", rng=rng)
    wl.K[:] = wl.K[0:1]
    O = _oracle_out(oracle_mod, wl)
    assert np.max(np.abs(O - wl.K[0:1].astype(np.float64))) < 1e-14


def _check_zero_query(orc, seed):
    """Z = 0 gives Q = 0 and uniform weights: output = mean of V rows per request."""
    rng = np.random.default_rng(seed)
    wl = W.custom("zq", [4, 6], [2, 3], q=2, d=8, heads=2, dtype="fp32",
                  kv_mode="separate", rng=rng)
    wl.Z[:] = 0
    O = _oracle_out(orc, wl)
    ref = np.concatenate([np.repeat(wl.V[wl.cu_kv[r]:wl.cu_kv[r + 1]].astype(np.float64)
                                    .mean(0, keepdims=True), wl.cands[r] * wl.q, 0)
                          for r in range(2)])
    return np.max(np.abs(O - ref))


def test_zero_query_gives_mean_value(oracle_mod):
    assert _check_zero_query(oracle_mod, 4) < 1e-14


def _check_two_keys(orc, seed):
    """Two keys: weight of key 1 is the logistic function of s1 - s2."""
    rng = np.random.default_rng(seed)
    wl = W.custom("tk", [2], [3], q=1, d=4, heads=1, dtype="fp32", kv_mode="separate", rng=rng)
    O = _oracle_out(orc, wl)
    Q = wl.Z.astype(np.float64).reshape(-1, 4) @ wl.wt[0].astype(np.float64).T
    K = wl.K.astype(np.float64)
    V = wl.V.astype(np.float64)
    s = Q @ K.T / 2.0  # sqrt(d_h) = 2
    p1 = expit(s[:, 0] - s[:, 1])[:, None]
    return np.max(np.abs(O - (p1 * V[0] + (1 - p1) * V[1])))


def test_two_keys_logistic_weight(oracle_mod):
    assert _check_two_keys(oracle_mod, 5) < 1e-15


def _check_lse_gradient(orc, seed):
    """With K = V = H the head output is sqrt(d_h) times the gradient of
    q -> logsumexp(H_h q / sqrt(d_h)); compared by central differences of
    scipy's logsumexp (an independent route to the same number)."""
    rng = np.random.default_rng(seed)
    d, heads = 8, 2
    dh = d // heads
    wl = W.custom("lse", [11], [2], q=1, d=d, heads=heads, dtype="fp32", kv_mode="shared", rng=rng)
    O = _oracle_out(orc, wl)
    Q = wl.Z.astype(np.float64).reshape(-1, d) @ wl.wt[0].astype(np.float64).T
    H = wl.K.astype(np.float64)
    err = 0.0
    eps = 1e-6
    for row in range(Q.shape[0]):
        for h in range(heads):
            Hh = H[:, h * dh:(h + 1) * dh]
            qv = Q[row, h * dh:(h + 1) * dh]
            f = lambda x: logsumexp(Hh @ x / np.sqrt(dh))
            g = np.array([(f(qv + eps * np.eye(dh)[e]) - f(qv - eps * np.eye(dh)[e])) / (2 * eps)
                          for e in range(dh)])
            err = max(err, np.max(np.abs(O[row, h * dh:(h + 1) * dh] - np.sqrt(dh) * g)))
    return err


def test_logsumexp_gradient_identity(oracle_mod):
    assert _check_lse_gradient(oracle_mod, 6) < 1e-8


def _check_translation(orc, seed):
    """PF-KV: adding u to every memory row shifts each score row by a constant
    (weights unchanged) and shifts the values by u, so O -> O + u."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode="shared")
    O = _oracle_out(orc, wl)
    u = rng.standard_normal(8)
    O2 = orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K + u)
    return np.max(np.abs(O2 - (O + u)))


def test_translation_equivariance_pfkv(oracle_mod):
    assert _check_translation(oracle_mod, 7) < 1e-12


def test_separate_kv_shift_rules(oracle_mod):
    """Separate K/V: shifting all keys leaves O unchanged; shifting all values by u adds u."""
    rng = np.random.default_rng(8)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode="separate")
    O = _oracle_out(oracle_mod, wl)
    u = rng.standard_normal(8)
    Ok = oracle_mod.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K + u, wl.V)
    Ov = oracle_mod.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V + u)
    assert np.max(np.abs(Ok - O)) < 1e-12
    assert np.max(np.abs(Ov - (O + u))) < 1e-12


def _check_permutation(orc, seed):
    """Permuting memory rows within each request (K and V jointly) leaves O unchanged."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=3, q=2, d=8, heads=2, kv_mode="separate")
    O = _oracle_out(orc, wl)
    perm = np.concatenate([wl.cu_kv[r] + rng.permutation(wl.lengths[r]) for r in range(wl.R)])
    O2 = orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K[perm], wl.V[perm])
    return np.max(np.abs(O2 - O))


def test_key_permutation_invariance(oracle_mod):
    assert _check_permutation(oracle_mod, 9) < 1e-13


def _check_shared_prefix(orc, seed):
    """ReST s.3.5 shared-prefix serving: scoring a request's N candidates against
    one H equals N single-candidate requests that each carry a copy of H."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=2, q=3, d=8, heads=2, kv_mode="shared", Nmax=5)
    O = _oracle_out(orc, wl)
    Ks, lens, cands = [], [], []
    for r in range(wl.R):
        for _ in range(wl.cands[r]):
            Ks.append(wl.K[wl.cu_kv[r]:wl.cu_kv[r + 1]])
            lens.append(wl.lengths[r])
            cands.append(1)
    cu_kv = np.concatenate([[0], np.cumsum(lens)])
    cu_c = np.concatenate([[0], np.cumsum(cands)])
    O2 = orc.forward(cu_kv, cu_c, wl.q, wl.heads, wl.Z, wl.wt, np.concatenate(Ks))
    return np.max(np.abs(O2 - O))


def test_shared_prefix_equivalence(oracle_mod):
    assert _check_shared_prefix(oracle_mod, 10) == 0.0


def test_request_independence_and_order(oracle_mod):
    """Requests do not interact: reversing the request order reverses the row blocks."""
    rng = np.random.default_rng(11)
    wl = _rand_case(rng, R=4, q=2, d=8, heads=2, kv_mode="separate")
    O = _oracle_out(oracle_mod, wl)
    order = list(range(wl.R))[::-1]
    kv_idx = np.concatenate([np.arange(wl.cu_kv[r], wl.cu_kv[r + 1]) for r in order])
    c_idx = np.concatenate([np.arange(wl.cu_cand[r], wl.cu_cand[r + 1]) for r in order])
    cu_kv = np.concatenate([[0], np.cumsum(wl.lengths[order])])
    cu_c = np.concatenate([[0], np.cumsum(wl.cands[order])])
    O2 = oracle_mod.forward(cu_kv, cu_c, wl.q, wl.heads, wl.Z[c_idx], wl.wt, wl.K[kv_idx],
                            wl.V[kv_idx])
    rows = (c_idx[:, None] * wl.q + np.arange(wl.q)[None]).reshape(-1)
    assert np.array_equal(O2, O[rows])


def _check_probs(orc, seed, kv_mode):
    """oracle.probs, which projects the query itself, against (i) torch's
    float64 softmax of the row's scores computed here from the definition
    (Q = Z . W_Q[slot] with output-major weights, scores over the head's
    slice scaled by 1/sqrt(d_h)), and (ii) the forward: probs . V must give
    the oracle's output row for that head.  Largest deviation over every row
    and head."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=3, q=3, d=8, heads=2, kv_mode=kv_mode)
    O = _oracle_out(orc, wl)
    f64 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    Z = f64(wl.Z.reshape(-1, wl.d))
    wt = f64(wl.wt)
    K = f64(wl.K)
    V = K if wl.V is None else f64(wl.V)
    dh = wl.d // wl.heads
    err = 0.0
    for row in range(wl.rows):
        r = int(np.searchsorted(wl.cu_cand * wl.q, row, side="right") - 1)
        a, b = int(wl.cu_kv[r]), int(wl.cu_kv[r + 1])
        qv = wt[row % wl.q] @ Z[row]
        for h in range(wl.heads):
            sl = slice(h * dh, (h + 1) * dh)
            ref = torch.softmax(K[a:b, sl] @ qv[sl] / np.sqrt(dh), dim=0).numpy()
            p = orc.probs(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, row, h)
            err = max(err, float(np.max(np.abs(p - ref))))
            err = max(err, float(np.max(np.abs(p @ V[a:b, sl].numpy() - O[row, sl]))))
    return err


@pytest.mark.parametrize("kv_mode", ["shared", "separate"])
def test_probs_match_torch_softmax_and_forward(oracle_mod, kv_mode):
    assert _check_probs(oracle_mod, 13, kv_mode) < 1e-12


def test_softmax_rows_sum_to_one(oracle_mod):
    rng = np.random.default_rng(12)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode="shared")
    for row in range(wl.rows):
        for h in range(wl.heads):
            p = oracle_mod.probs(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, row, h)
            assert np.all(p >= 0)
            assert abs(p.sum() - 1.0) < 1e-12


def test_gaussian_large_memory_limit(oracle_mod):
    """K = V = H ~ N(0, I): as L grows the softmax-weighted mean tends to the
    exponentially tilted Gaussian mean q_h / sqrt(d_h) (loose statistical check;
    it catches a wrong score scale such as 1/sqrt(d) instead of 1/sqrt(d_h))."""
    rng = np.random.default_rng(13)
    wl = W.custom("big", [8192], [8], q=1, d=256, heads=4, dtype="fp32", kv_mode="shared", rng=rng)
    O = _oracle_out(oracle_mod, wl)
    Q = wl.Z.astype(np.float64).reshape(-1, 256) @ wl.wt[0].astype(np.float64).T
    slope = float(np.sum(O * Q) / np.sum(Q * Q))
    # 1/sqrt(d_h) = 0.125; the 1/sqrt(d) reading would give 0.0625.
    assert abs(slope - 0.125) < 0.0125
    assert np.mean(np.abs(O - Q / np.sqrt(64))) < 0.05


def test_thread_count_independence(oracle_mod):
    rng = np.random.default_rng(14)
    wl = _rand_case(rng, R=5, q=3, d=16, heads=4, kv_mode="shared", Lmax=40, Nmax=9)
    oracle_mod.set_threads(1)
    O1 = _oracle_out(oracle_mod, wl)
    oracle_mod.set_threads(4)
    O4 = _oracle_out(oracle_mod, wl)
    oracle_mod.set_threads(os.cpu_count() or 1)
    assert np.array_equal(O1, O4)


def test_row_subset_matches_full(oracle_mod):
    rng = np.random.default_rng(15)
    wl = _rand_case(rng, R=3, q=2, d=8, heads=2, kv_mode="separate")
    O = _oracle_out(oracle_mod, wl)
    rows = [0, wl.rows - 1, wl.rows // 2]
    assert np.array_equal(_oracle_out(oracle_mod, wl, rows=rows), O[rows])


# ----------------------------------------------------------------------------
# Integer plan
# ----------------------------------------------------------------------------
def check_plan(cu_kv, cu_cand, q, tile_m, cu_q, row_req, tiles):
    """Properties that define the plan: cu_q = q*cu_cand, row_req is the
    range map, tiles cover every query row exactly once with nc <= tile_m,
    ordered by request length descending (ties by index), then block, then slot."""
    cu_kv = np.asarray(cu_kv)
    cu_cand = np.asarray(cu_cand)
    R = len(cu_kv) - 1
    L = np.diff(cu_kv)
    N = np.diff(cu_cand)
    assert np.array_equal(cu_q, q * cu_cand)
    if row_req is not None:
        assert np.array_equal(row_req, np.repeat(np.arange(R), N * q))
    cover = np.zeros(int(cu_cand[-1]) * q, dtype=np.int64)
    for (r, s, c0, nc) in tiles:
        assert 0 <= r < R and 0 <= s < q and 0 < nc <= tile_m
        assert cu_cand[r] <= c0 and c0 + nc <= cu_cand[r + 1]
        assert (c0 - cu_cand[r]) % tile_m == 0
        cover[(np.arange(c0, c0 + nc)) * q + s] += 1
    assert np.all(cover == 1)
    keys = [(-L[r], r, c0, s) for (r, s, c0, nc) in tiles]
    assert keys == sorted(keys)


@pytest.mark.parametrize("seed", range(4))
def test_plan_properties(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 20))
    L = rng.integers(0, 50, size=R)
    L[rng.integers(0, R)] = L[0]  # force a tie
    N = rng.integers(0, 200, size=R)
    cu_kv = np.concatenate([[0], np.cumsum(L)])
    cu_c = np.concatenate([[0], np.cumsum(N)])
    for q in (1, 3):
        for tm in (16, 64):
            cu_q, row_req, tiles = oracle_mod.plan(cu_kv, cu_c, q, tm)
            check_plan(cu_kv, cu_c, q, tm, cu_q, row_req, tiles)
            assert len(tiles) == sum(q * ((n + tm - 1) // tm) for n in N)


def test_plan_configs(oracle_mod):
    for name in ("rest", "ragged"):
        wl = W.make(name, 0)
        cu_q, row_req, tiles = oracle_mod.plan(wl.cu_kv, wl.cu_cand, wl.q, 64)
        check_plan(wl.cu_kv, wl.cu_cand, wl.q, 64, cu_q, row_req, tiles)


# ----------------------------------------------------------------------------
# Per-candidate prefix cutoff (ReST reading note s.3.5, ULT)
# ----------------------------------------------------------------------------
def _check_prefix_sdpa(orc, seed):
    """Against torch float64 SDPA with a boolean mask that hides every key at
    or past the candidate's cutoff; cutoffs include 0 (zeros), 1, L and more
    than L, and negative values (read as 0)."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=3, q=2, d=8, heads=2, kv_mode="separate", Lmax=9, Nmax=4)
    kv_len = rng.integers(-2, 12, size=wl.total_cand)
    kv_len[: min(3, wl.total_cand)] = [0, 1, 100][: min(3, wl.total_cand)]
    O = orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V,
                    kv_len=kv_len)
    Zt = torch.tensor(wl.Z.astype(np.float64)).reshape(-1, wl.d)
    Kt = torch.tensor(wl.K.astype(np.float64))
    Vt = torch.tensor(wl.V.astype(np.float64))
    dh = wl.d // wl.heads
    err = 0.0
    for r in range(wl.R):
        k, v = Kt[wl.cu_kv[r]:wl.cu_kv[r + 1]], Vt[wl.cu_kv[r]:wl.cu_kv[r + 1]]
        L = k.shape[0]
        for c in range(wl.cu_cand[r], wl.cu_cand[r + 1]):
            cut = int(min(max(kv_len[c], 0), L))
            for s_ in range(wl.q):
                row = c * wl.q + s_
                qv = Zt[row] @ torch.tensor(wl.wt[s_].astype(np.float64)).T
                if cut == 0:
                    err = max(err, float(np.max(np.abs(O[row]))))
                    continue
                mask = (torch.arange(L) < cut).view(1, 1, L)
                o = torch.cat([torch.nn.functional.scaled_dot_product_attention(
                    qv[h * dh:(h + 1) * dh].view(1, 1, dh), k[:, h * dh:(h + 1) * dh].view(1, L, dh),
                    v[:, h * dh:(h + 1) * dh].view(1, L, dh), attn_mask=mask).view(dh)
                    for h in range(wl.heads)])
                err = max(err, float(np.max(np.abs(O[row] - o.numpy()))))
    return err


def _check_prefix_full_is_plain(orc, seed):
    """Cutoffs at or past every request's length change nothing (bitwise)."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=3, q=2, d=8, heads=2, kv_mode="shared", Lmax=9, Nmax=4)
    O1 = orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V)
    O2 = orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V,
                     kv_len=np.full(wl.total_cand, 1 << 20))
    return float(np.max(np.abs(O1 - O2)))


def _check_prefix_truncation(orc, seed):
    """A candidate with cutoff L' equals the same candidate alone in a request
    whose memory is the first L' rows (bitwise: rows are independent)."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode="shared", Lmax=9, Nmax=4)
    kv_len = rng.integers(1, 10, size=wl.total_cand)
    O = orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V,
                    kv_len=kv_len)
    err = 0.0
    for r in range(wl.R):
        L = int(wl.cu_kv[r + 1] - wl.cu_kv[r])
        for c in range(wl.cu_cand[r], wl.cu_cand[r + 1]):
            cut = min(int(kv_len[c]), L)
            Kc = wl.K[wl.cu_kv[r]:wl.cu_kv[r] + cut]
            Oc = orc.forward([0, cut], [0, 1], wl.q, wl.heads, wl.Z[c:c + 1], wl.wt, Kc)
            err = max(err, float(np.max(np.abs(Oc - O[c * wl.q:(c + 1) * wl.q]))))
    return err


@pytest.mark.parametrize("seed", range(4))
def test_prefix_cutoff_matches_masked_sdpa(oracle_mod, seed):
    assert _check_prefix_sdpa(oracle_mod, seed) < 1e-12


def test_prefix_cutoff_past_length_is_plain(oracle_mod):
    assert _check_prefix_full_is_plain(oracle_mod, 3) == 0.0


def test_prefix_cutoff_equals_truncated_memory(oracle_mod):
    assert _check_prefix_truncation(oracle_mod, 4) == 0.0


# ----------------------------------------------------------------------------
# Output gate and output projection (Eq. (7) after the attention)
# ----------------------------------------------------------------------------
def _perm_wo(d, rng):
    """W_o as a permutation (output-major: wo[p][o] = 1 for o = pi(p))."""
    pi = rng.permutation(d)
    while d > 1 and np.all(pi == pi[pi]):   # avoid involutions: a transpose must differ
        pi = rng.permutation(d)
    wo = np.zeros((d, d))
    wo[np.arange(d), pi] = 1.0
    return wo, pi


def _check_gate_half_and_saturated(orc, seed):
    """Slot 0 has W_go = 0, so its gate is exactly 1/2; slot 1 has W_go =
    50 I on positive tokens, so its gate rounds to exactly 1.  With W_o a
    permutation, Y is the permuted O (halved for slot 0), exactly."""
    rng = np.random.default_rng(seed)
    d, q, n = 6, 2, 5
    Z = np.abs(rng.standard_normal((n, q, d))) + 1.0
    O = rng.standard_normal((n, q, d))
    wgo = np.stack([np.zeros((d, d)), 50.0 * np.eye(d)])
    wo, pi = _perm_wo(d, rng)
    Y = orc.output(Z, wgo, O, wo, q).reshape(n, q, d)
    want = np.stack([O[:, 0, pi] / 2.0, O[:, 1, pi]], axis=1)
    return float(np.max(np.abs(Y - want)))


def _check_gate_symmetry(orc, seed):
    """sigmoid(-x) = 1 - sigmoid(x): the outputs for W_go and -W_go add up to
    O W_o (the ungated projection)."""
    rng = np.random.default_rng(seed)
    d, q, n = 8, 3, 4
    Z = rng.standard_normal((n, q, d))
    O = rng.standard_normal((n, q, d))
    wgo = rng.standard_normal((q, d, d)) / np.sqrt(d)
    wo = rng.standard_normal((d, d))
    Y = orc.output(Z, wgo, O, wo, q) + orc.output(Z, -wgo, O, wo, q)
    return float(np.max(np.abs(Y - O.reshape(-1, d) @ wo.T)))


def _check_gate_golden(orc, path):
    g = json.load(open(path))
    Y = orc.output(np.array(g["Z"]), np.array(g["wgo"]), np.array(g["O"]), np.array(g["wo"]),
                   g["q"])
    return np.allclose(Y, np.array(g["Y"]), rtol=max(g["rtol"], 1e-15), atol=1e-15)


def test_output_gate_half_and_saturated(oracle_mod):
    assert _check_gate_half_and_saturated(oracle_mod, 0) == 0.0


def test_output_gate_symmetry(oracle_mod):
    assert _check_gate_symmetry(oracle_mod, 1) < 1e-12


@pytest.mark.parametrize("path", GOLDEN_OUTPUT, ids=[os.path.basename(p) for p in GOLDEN_OUTPUT])
def test_output_golden(oracle_mod, path):
    assert _check_gate_golden(oracle_mod, path)


def test_full_eq7_composes(oracle_mod):
    """The full cross-attention of Eq. (7) is the attention output followed by
    the gate and the output projection: checked against torch float64 SDPA on
    a tiny batch (an independent library routine for the attention part)."""
    rng = np.random.default_rng(12)
    wl = W.custom("eq7", [5, 3], [2, 1], q=2, d=8, heads=2, dtype="fp32", seed=12)
    O = oracle_mod.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V)
    wgo = rng.standard_normal((2, 8, 8)) / np.sqrt(8)
    wo = rng.standard_normal((8, 8)) / np.sqrt(8)
    Y = oracle_mod.output(wl.Z, wgo, O, wo, wl.q)
    Zt = torch.tensor(wl.Z.astype(np.float64)).reshape(-1, 8)
    Kt = torch.tensor(wl.K.astype(np.float64))
    want = []
    for r in range(wl.R):
        rows = range(wl.cu_cand[r] * wl.q, wl.cu_cand[r + 1] * wl.q)
        k = Kt[wl.cu_kv[r]:wl.cu_kv[r + 1]]
        for row in rows:
            s = row % wl.q
            qv = Zt[row] @ torch.tensor(wl.wt[s].astype(np.float64)).T
            o = torch.cat([torch.nn.functional.scaled_dot_product_attention(
                qv[h * 4:(h + 1) * 4].view(1, 1, 4), k[:, h * 4:(h + 1) * 4].view(1, -1, 4),
                k[:, h * 4:(h + 1) * 4].view(1, -1, 4)).view(4) for h in range(2)])
            gate = torch.sigmoid(Zt[row] @ torch.tensor(wgo[s]).T)
            want.append(((o * gate) @ torch.tensor(wo).T).numpy())
    assert np.max(np.abs(Y - np.array(want))) < 1e-12


# ----------------------------------------------------------------------------
# Backward pass (gradients of <dO, O>)
# ----------------------------------------------------------------------------
def _torch_grads(wl, dO, kv_len=None):
    """Gradients of <dO, O> by torch CPU float64 autograd through an
    independent statement of the forward: Q = Z W_Q[slot]; per request, head
    and query row, softmax over the visible memory rows, then the weighted sum
    of values.  In projection-free mode H is one leaf used as both key and
    value, so autograd adds both roles itself."""
    d, dh, q = wl.d, wl.d_h, wl.q
    Z = torch.tensor(wl.Z.astype(np.float64).reshape(-1, d), requires_grad=True)
    wt = torch.tensor(wl.wt.astype(np.float64), requires_grad=True)
    K = torch.tensor(wl.K.astype(np.float64), requires_grad=True)
    V = torch.tensor(wl.V.astype(np.float64), requires_grad=True) if wl.V is not None else None
    Vm = V if V is not None else K
    rows = Z.shape[0]
    Q = torch.stack([Z[r] @ wt[r % q].T for r in range(rows)]) if rows else Z
    outs = []
    for r in range(wl.R):
        kv0, L = int(wl.cu_kv[r]), int(wl.cu_kv[r + 1] - wl.cu_kv[r])
        for row in range(int(wl.cu_cand[r]) * q, int(wl.cu_cand[r + 1]) * q):
            cut = L if kv_len is None else min(max(int(kv_len[row // q]), 0), L)
            heads_out = []
            for h in range(wl.heads):
                cols = slice(h * dh, (h + 1) * dh)
                if cut == 0:
                    heads_out.append(torch.zeros(dh, dtype=torch.float64))
                    continue
                sc = K[kv0:kv0 + cut, cols] @ Q[row, cols] / np.sqrt(dh)
                heads_out.append(torch.softmax(sc, dim=0) @ Vm[kv0:kv0 + cut, cols])
            outs.append(torch.cat(heads_out))
    O = torch.stack(outs)
    (O * torch.from_numpy(np.asarray(dO, dtype=np.float64).reshape(-1, d))).sum().backward()
    return {"dZ": Z.grad.numpy(), "dwt": wt.grad.numpy(), "dK": K.grad.numpy(),
            "dV": V.grad.numpy() if V is not None else None}


def _dO_for(wl, rng):
    return rng.normal(size=(wl.rows, wl.d))


def _check_bwd_autograd(orc, seed, kv_mode, prefix=False):
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=3, q=int(rng.integers(1, 4)), d=8,
                    heads=int(rng.choice([1, 2, 4])), kv_mode=kv_mode)
    dO = _dO_for(wl, rng)
    kv_len = rng.integers(-1, 11, size=wl.total_cand) if prefix else None
    g = orc.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, dO,
                     kv_len=kv_len)
    t = _torch_grads(wl, dO, kv_len)
    err = 0.0
    for k in ("dZ", "dwt", "dK", "dV"):
        if t[k] is None:
            assert g[k] is None
            continue
        err = max(err, float(np.max(np.abs(g[k].reshape(t[k].shape) - t[k]))))
    return err


@pytest.mark.parametrize("kv_mode", ["shared", "separate"])
@pytest.mark.parametrize("seed", range(4))
def test_backward_matches_torch_autograd(oracle_mod, seed, kv_mode):
    assert _check_bwd_autograd(oracle_mod, seed, kv_mode) < 1e-12


@pytest.mark.parametrize("kv_mode", ["shared", "separate"])
def test_backward_prefix_matches_torch_autograd(oracle_mod, kv_mode):
    assert _check_bwd_autograd(oracle_mod, 21, kv_mode, prefix=True) < 1e-12


def _check_bwd_finite_diff(orc, seed, kv_mode):
    """Central differences of f = <dO, forward(x)> (the separately pinned
    forward) along random directions in Z, W_Q, K and V, against <grad, dir>.
    Returns the largest relative mismatch."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode=kv_mode, Lmax=6, Nmax=3)
    dO = _dO_for(wl, rng)
    g = orc.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, dO)
    base = {"Z": wl.Z.astype(np.float64), "wt": wl.wt.astype(np.float64),
            "K": wl.K.astype(np.float64),
            "V": wl.V.astype(np.float64) if wl.V is not None else None}

    def f(x):
        O = orc.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, x["Z"], x["wt"], x["K"], x["V"])
        return float(np.sum(O * dO))

    worst = 0.0
    eps = 1e-6
    for name, gname in (("Z", "dZ"), ("wt", "dwt"), ("K", "dK"), ("V", "dV")):
        if base[name] is None:
            continue
        v = rng.normal(size=base[name].shape)
        xp = dict(base)
        xm = dict(base)
        xp[name] = base[name] + eps * v
        xm[name] = base[name] - eps * v
        fd = (f(xp) - f(xm)) / (2 * eps)
        an = float(np.sum(g[gname].reshape(v.shape) * v))
        worst = max(worst, abs(fd - an) / max(1.0, abs(an)))
    return worst


@pytest.mark.parametrize("kv_mode", ["shared", "separate"])
def test_backward_finite_differences(oracle_mod, kv_mode):
    assert _check_bwd_finite_diff(oracle_mod, 30, kv_mode) < 1e-7


def _check_bwd_single_row(orc, seed):
    """L = 1: the one weight is exactly 1 whatever the query, so no gradient
    reaches Z, W_Q or the key role, and the memory row's value gradient is the
    sum of the request's dO rows (head by head).  Returns the largest error."""
    rng = np.random.default_rng(seed)
    wl = W.custom("l1", [1, 1], [3, 2], q=2, d=8, heads=4, dtype="fp32",
                  kv_mode="separate", rng=rng)
    dO = _dO_for(wl, rng)
    g = orc.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, dO)
    err = max(np.max(np.abs(g["dZ"])), np.max(np.abs(g["dwt"])), np.max(np.abs(g["dK"])))
    for r in range(wl.R):
        a, b = int(wl.cu_cand[r]) * wl.q, int(wl.cu_cand[r + 1]) * wl.q
        err = max(err, float(np.max(np.abs(g["dV"][r] - dO[a:b].sum(axis=0)))))
    return err


def test_backward_single_memory_row(oracle_mod):
    assert _check_bwd_single_row(oracle_mod, 31) < 1e-14


def _check_bwd_identical_keys(orc, seed):
    """All keys of a request equal: the weights are uniform for every query,
    so nothing flows back into the queries (dZ = dW_Q = 0)."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode="separate")
    K = wl.K.copy()
    for r in range(wl.R):
        K[wl.cu_kv[r]:wl.cu_kv[r + 1]] = K[wl.cu_kv[r]]
    dO = _dO_for(wl, rng)
    g = orc.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, K, wl.V, dO)
    return max(np.max(np.abs(g["dZ"])), np.max(np.abs(g["dwt"])))


def test_backward_identical_keys(oracle_mod):
    assert _check_bwd_identical_keys(oracle_mod, 32) < 1e-13


def _check_bwd_shared_prefix_sum(orc, seed):
    """TransX report s.2 (trajectory packing): the memory gradient of a
    request's N candidates scored against one H equals the sum, over N
    single-candidate requests that each carry a copy of H, of their memory
    gradients; the query-side gradients are unchanged."""
    rng = np.random.default_rng(seed)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode="shared", Nmax=5)
    dO = _dO_for(wl, rng)
    g = orc.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, None, dO)
    Ks, lens, owner = [], [], []
    for r in range(wl.R):
        for _ in range(wl.cands[r]):
            Ks.append(wl.K[wl.cu_kv[r]:wl.cu_kv[r + 1]])
            lens.append(wl.lengths[r])
            owner.append(r)
    cu_kv = np.concatenate([[0], np.cumsum(lens)])
    cu_c = np.arange(len(lens) + 1)
    g2 = orc.backward(cu_kv, cu_c, wl.q, wl.heads, wl.Z, wl.wt, np.concatenate(Ks), None, dO)
    err = max(np.max(np.abs(g2["dZ"] - g["dZ"])), np.max(np.abs(g2["dwt"] - g["dwt"])))
    summed = np.zeros_like(g["dK"])
    for n, r in enumerate(owner):
        summed[wl.cu_kv[r]:wl.cu_kv[r + 1]] += g2["dK"][cu_kv[n]:cu_kv[n + 1]]
    return max(err, float(np.max(np.abs(summed - g["dK"]))))


def test_backward_candidate_gradients_sum_into_one_memory(oracle_mod):
    assert _check_bwd_shared_prefix_sum(oracle_mod, 33) < 1e-13


def _check_bwd_prefix_truncation(orc, seed):
    """With every candidate of a request cut at L', the gradients equal those
    of the request with its memory truncated to L' rows; rows past L' get
    zero memory gradient."""
    rng = np.random.default_rng(seed)
    wl = W.custom("trunc", [9], [4], q=2, d=8, heads=2, dtype="fp32", kv_mode="separate",
                  rng=rng)
    cut = 5
    dO = _dO_for(wl, rng)
    g = orc.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, dO,
                     kv_len=np.full(wl.total_cand, cut))
    t = orc.backward([0, cut], wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K[:cut], wl.V[:cut],
                     dO)
    err = max(np.max(np.abs(g["dZ"] - t["dZ"])), np.max(np.abs(g["dwt"] - t["dwt"])),
              np.max(np.abs(g["dK"][:cut] - t["dK"])), np.max(np.abs(g["dV"][:cut] - t["dV"])),
              np.max(np.abs(g["dK"][cut:])), np.max(np.abs(g["dV"][cut:])))
    return err


def test_backward_prefix_truncation(oracle_mod):
    assert _check_bwd_prefix_truncation(oracle_mod, 34) == 0.0


def test_backward_is_linear_in_dO(oracle_mod):
    rng = np.random.default_rng(35)
    wl = _rand_case(rng, R=2, q=2, d=8, heads=2, kv_mode="shared")
    a, b = _dO_for(wl, rng), _dO_for(wl, rng)
    ga = oracle_mod.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, None, a)
    gb = oracle_mod.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, None, b)
    gc = oracle_mod.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, None,
                             2.0 * a - 3.0 * b)
    for k in ("dZ", "dwt", "dK"):
        assert np.max(np.abs(gc[k] - (2.0 * ga[k] - 3.0 * gb[k]))) < 1e-12


def test_backward_thread_count_independent(oracle_mod):
    rng = np.random.default_rng(36)
    wl = _rand_case(rng, R=5, q=3, d=16, heads=4, kv_mode="shared", Lmax=40, Nmax=6)
    dO = _dO_for(wl, rng)
    oracle_mod.set_threads(1)
    g1 = oracle_mod.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, None, dO)
    oracle_mod.set_threads(4)
    g4 = oracle_mod.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, None, dO)
    for k in ("dQ", "dZ", "dwt", "dK"):
        assert np.array_equal(g1[k], g4[k])


# ----------------------------------------------------------------------------
# Mutation test: plausible mistakes planted in copies of the oracle are caught
# ----------------------------------------------------------------------------
MUTANTS = {
    "scale_uses_d": ("1.0 / sqrt((double)d_h)", "1.0 / sqrt((double)d)"),
    "slot_ignored": ("wt + (size_t)(row % q) * d * d", "wt + (size_t)0 * d * d"),
    "weight_transposed": ("Z[(size_t)row * d + i] * w[(size_t)o * d + i]",
                          "Z[(size_t)row * d + i] * w[(size_t)i * d + o]"),
    "key_head_offset_dropped": ("K[(size_t)(kv0 + j) * d + head * d_h + e]",
                                "K[(size_t)(kv0 + j) * d + e]"),
    "value_head_offset_dropped": ("Vm[(size_t)(kv0 + j) * d + h * d_h + e]",
                                  "Vm[(size_t)(kv0 + j) * d + e]"),
    "separate_value_ignored": ("const double *Vm = V ? V : K;", "const double *Vm = K;"),
    "last_key_dropped": ("for (int j = 0; j < L; ++j) {\n        double s = 0.0;",
                         "for (int j = 0; j < L - 1; ++j) {\n        double s = 0.0;"),
    "no_normalisation": ("p[j] /= z;", "p[j] /= 1.0;"),
    "sign_of_max": ("p[j] = exp(p[j] - m);", "p[j] = exp(m - p[j]);"),
    "wrong_request_base": ("const int kv0 = cu_kv[r], L = cu_kv[r + 1] - cu_kv[r];\n                /* visible",
                           "const int kv0 = 0, L = cu_kv[r + 1] - cu_kv[r];\n                /* visible"),
    "gate_sign": ("/ (1.0 + exp(-acc));", "/ (1.0 + exp(acc));"),
    "cutoff_ignored": ("Lc = want < 0 ? 0 : (want < L ? want : L);", "Lc = L;"),
    "cutoff_off_by_one": ("Lc = want < 0 ? 0 : (want < L ? want : L);",
                          "Lc = want < 0 ? 0 : (want + 1 < L ? want + 1 : L);"),
    "gate_missing": ("x[o] = O[(size_t)row * d + o] / (1.0 + exp(-acc));",
                     "x[o] = O[(size_t)row * d + o];"),
    "gate_slot_ignored": ("const double *w = wgo + (size_t)(row % q) * d * d;",
                          "const double *w = wgo;"),
    "output_weight_transposed": ("acc += x[o] * wo[(size_t)p * d + o];",
                                 "acc += x[o] * wo[(size_t)o * d + p];"),
    "bwd_softmax_mean_dropped": ("const double ds = p[j] * (dp[j] - pdp);",
                                 "const double ds = p[j] * dp[j];"),
    "bwd_key_scale_dropped": ("gkj[e] += c * ds * qi[e];", "gkj[e] += ds * qi[e];"),
    "bwd_value_role_dropped": ("dK[k] = gK[k] + gV[k];", "dK[k] = gK[k];"),
    "bwd_dz_weight_transposed": ("acc += gQ[(size_t)row * d + o] * w[(size_t)o * d + i];",
                                 "acc += gQ[(size_t)row * d + o] * w[(size_t)i * d + o];"),
    "bwd_dw_all_slots": ("for (long row = s; row < total_rows; row += q) {",
                         "for (long row = 0; row < total_rows; row += 1) {"),
    "bwd_dq_reads_values": ("dqi[e] += c * ds * kj[e];",
                            "dqi[e] += c * ds * Vm[(size_t)(kv0 + j) * d + h * d_h + e];"),
    # oracle_probs projects the query with a copy of the loop of the forward:
    # mistakes planted in that copy alone
    "probs_slot_ignored": ("return ORACLE_EINVAL;\n    const double *w = wt + (size_t)(row % q) * d * d;",
                           "return ORACLE_EINVAL;\n    const double *w = wt + (size_t)0 * d * d;"),
    "probs_weight_transposed": ("acc += Z[(size_t)row * d + i] * w[(size_t)o * d + i];\n        qrow[o] = acc;\n    }\n    if (L > 0)",
                                "acc += Z[(size_t)row * d + i] * w[(size_t)i * d + o];\n        qrow[o] = acc;\n    }\n    if (L > 0)"),
    "probs_head_offset": ("softmax_weights(qrow, K, d, d_h, head, kv0, L, p);",
                          "softmax_weights(qrow, K, d, d_h, 0, kv0, L, p);"),
    "bwd_cutoff_ignored": ("Lc = want < 0 ? 0 : (want < L ? want : L);\n                    }\n                    if (Lc == 0)\n                        continue;",
                           "Lc = L;\n                    }\n                    if (Lc == 0)\n                        continue;"),
}


def _all_pins(orc):
    """Run every pin above against an oracle module; return the failing ones."""
    fails = []
    checks = {
        "projection": lambda: _check_projection(orc, 0) < 1e-12,
        "sdpa_shared": lambda: all(_check_sdpa(orc, s, "shared") < 1e-12 for s in range(3)),
        "sdpa_separate": lambda: all(_check_sdpa(orc, s, "separate") < 1e-12 for s in range(3)),
        "single_row": lambda: _check_single_row(orc, 1) == 0.0,
        "identical_keys": lambda: _check_identical_keys(orc, 2) < 1e-14,
        "zero_query": lambda: _check_zero_query(orc, 4) < 1e-14,
        "two_keys": lambda: _check_two_keys(orc, 5) < 1e-15,
        "lse_gradient": lambda: _check_lse_gradient(orc, 6) < 1e-8,
        "translation": lambda: _check_translation(orc, 7) < 1e-12,
        "permutation": lambda: _check_permutation(orc, 9) < 1e-13,
        "shared_prefix": lambda: _check_shared_prefix(orc, 10) == 0.0,
        "probs_shared": lambda: _check_probs(orc, 13, "shared") < 1e-12,
        "probs_separate": lambda: _check_probs(orc, 13, "separate") < 1e-12,
        "gate_half_saturated": lambda: _check_gate_half_and_saturated(orc, 0) == 0.0,
        "gate_symmetry": lambda: _check_gate_symmetry(orc, 1) < 1e-12,
        "prefix_sdpa": lambda: all(_check_prefix_sdpa(orc, s_) < 1e-12 for s_ in range(2)),
        "prefix_truncation": lambda: _check_prefix_truncation(orc, 4) == 0.0,
        "bwd_autograd_shared": lambda: _check_bwd_autograd(orc, 0, "shared") < 1e-12,
        "bwd_autograd_separate": lambda: _check_bwd_autograd(orc, 1, "separate") < 1e-12,
        "bwd_autograd_prefix": lambda: _check_bwd_autograd(orc, 21, "shared", True) < 1e-12,
        "bwd_finite_diff": lambda: all(_check_bwd_finite_diff(orc, 30, m) < 1e-7
                                       for m in ("shared", "separate")),
        "bwd_single_row": lambda: _check_bwd_single_row(orc, 31) < 1e-14,
        "bwd_identical_keys": lambda: _check_bwd_identical_keys(orc, 32) < 1e-13,
        "bwd_shared_prefix_sum": lambda: _check_bwd_shared_prefix_sum(orc, 33) < 1e-13,
        "bwd_prefix_truncation": lambda: _check_bwd_prefix_truncation(orc, 34) == 0.0,
    }
    for path in GOLDEN_OUTPUT:
        checks["golden:" + os.path.basename(path)] = lambda path=path: _check_gate_golden(orc, path)
    for path in GOLDEN:
        g = json.load(open(path))
        V = np.array(g["V"]) if g["V"] is not None else None

        def gold(g=g, V=V):
            O = orc.forward(g["cu_kv"], g["cu_cand"], g["q"], g["heads"], np.array(g["Z"]),
                            np.array(g["wt"]), np.array(g["K"]), V)
            return np.allclose(O, np.array(g["O"]), rtol=max(g["rtol"], 1e-15), atol=1e-15)
        checks["golden:" + os.path.basename(path)] = gold
    for name, fn in checks.items():
        try:
            ok = bool(fn())
        except Exception:
            ok = False
        if not ok:
            fails.append(name)
    return fails


def _load_mutant(tmpdir, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "xattn_oracle.c")).read()
    assert src.count(old) >= 1, "mutation anchor for %s not found" % name
    msrc = os.path.join(tmpdir, "mut_%s.c" % name)
    open(msrc, "w").write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("oracle_mut_" + name,
                                                  os.path.join(os.path.dirname(oracle.__file__),
                                                               "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._SRC = msrc
    mod._LIB = os.path.join(tmpdir, "libmut_%s.so" % name)
    mod.build(force=True)
    return mod


def test_unmutated_oracle_passes_all_pins(oracle_mod):
    assert _all_pins(oracle_mod) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    tmpdir = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        mod = _load_mutant(tmpdir, name, *MUTANTS[name])
        assert _all_pins(mod), "mutant %s passed every pin" % name
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
