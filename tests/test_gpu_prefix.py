"""GPU parity of the per-candidate prefix cutoff (xattn_forward_prefix; ReST
reading note s.3.5, ULT: each training sample of a user sees only the part of
the user's sequence before it).  The HIP path, through the C ABI, against the
fp64 oracle's forward with kv_len on the same seeded inputs and cutoffs:
bf16 element-wise max-abs <= 2e-2, fp32 normwise relative <= 1e-4.  Cutoffs
include values below 0 and above L_r (clamped), 0 (all-zero rows) and L_r."""
import numpy as np
import pytest
import torch

import oracle
from shared_history_candidate_amd import workloads as W
from shared_history_candidate_amd import xattn as X

from gpu_util import assert_close, ctx_for, require_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _run(wl, kv_len, ctx=None):
    require_gpu()
    ctx = ctx or ctx_for(wl)
    t = X.to_device(wl)
    cl = torch.from_numpy(np.ascontiguousarray(kv_len, dtype=np.int32)).to("cuda")
    O = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    cand_kv_len=cl)
    torch.cuda.synchronize()
    return O


def _check(wl, kv_len, rows=None, what=""):
    got = _run(wl, kv_len).float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V,
                         rows=rows, kv_len=kv_len)
    if rows is not None:
        got = got[rows]
    err, rel = assert_close(got, ref, wl.dtype, what or wl.name)
    print("prefix %s: rows=%d max-abs %.3e normwise %.3e" % (what or wl.name, len(ref), err, rel))
    return got


def _zero_rows(wl, kv_len):
    """Query rows of candidates that see no memory row."""
    rows = []
    for r in range(wl.R):
        for c in range(int(wl.cu_cand[r]), int(wl.cu_cand[r + 1])):
            if min(max(int(kv_len[c]), 0), int(wl.lengths[r])) == 0:
                rows.extend(range(c * wl.q, (c + 1) * wl.q))
    return np.array(rows, dtype=np.int64)


EDGE_LENGTHS = [1, 2, 31, 33, 63, 65, 97, 1023, 300]
EDGE_CANDS = [1, 33, 65, 0, 129, 3, 64, 5, 40]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("q", [1, 3])
@pytest.mark.parametrize("dh,heads", [(32, 4), (64, 2), (128, 2)])
def test_prefix_edge_shapes_bf16(mode, q, dh, heads):
    wl = W.custom("edge", EDGE_LENGTHS, EDGE_CANDS, q=q, d=dh * heads, heads=heads,
                  dtype="bf16", kv_mode=mode, seed=dh + q)
    kv_len = W.prefix_lengths(wl, seed=dh * 7 + q)
    got = _check(wl, kv_len, what="edge dh=%d q=%d %s" % (dh, q, mode))
    zr = _zero_rows(wl, kv_len)
    assert zr.size > 0 and np.all(got[zr] == 0.0)


@pytest.mark.parametrize("variant", ["1,4", "2,2", "4,1", "2,1"])
@pytest.mark.parametrize("dh,heads,mode", [(64, 4, "shared"), (32, 8, "separate"),
                                           (128, 2, "shared")])
def test_prefix_every_variant(monkeypatch, variant, dh, heads, mode):
    """Every work-group shape (query blocks x memory splits) the library
    builds, forced through XATTN_VARIANT (shapes not built for a head width
    fall back to the default choice)."""
    monkeypatch.setenv("XATTN_VARIANT", variant)
    wl = W.custom("var", [700, 129, 64, 1500], [70, 9, 33, 40], q=3, d=dh * heads,
                  heads=heads, dtype="bf16", kv_mode=mode, seed=11)
    _check(wl, W.prefix_lengths(wl, seed=5), what="variant %s dh=%d %s" % (variant, dh, mode))


@pytest.mark.parametrize("name", ["rest", "ragged"])
def test_prefix_full_length_matches_forward(name):
    """Cutoffs at or past L_r give xattn_forward's bits (rest runs xattn_forward
    as one launch, ragged as projection + attention)."""
    require_gpu()
    wl = W.make(name, 0)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ref = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"],
                      wl.heads).clone()
    kv_len = np.repeat(wl.lengths, wl.cands).astype(np.int32)
    kv_len[::3] += 1000
    got = _run(wl, kv_len, ctx)
    assert torch.equal(got, ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefix_nothing_visible(dtype):
    wl = W.custom("none", [40, 200], [5, 70], q=3, d=128, heads=2, dtype=dtype,
                  kv_mode="shared", seed=2)
    kv_len = np.where(np.arange(wl.total_cand) % 2 == 0, 0, -7).astype(np.int32)
    got = _run(wl, kv_len)
    assert torch.count_nonzero(got).item() == 0


def test_prefix_one_row_each():
    """Every candidate sees exactly its request's first memory row: the
    softmax is a single weight, O = V[first row] per head."""
    wl = W.custom("one", [1, 64, 65, 500], [3, 40, 70, 9], q=2, d=256, heads=4, dtype="bf16",
                  kv_mode="separate", seed=4)
    _check(wl, np.ones(wl.total_cand, dtype=np.int32), what="one row")


def test_prefix_rest_workload():
    wl = W.make("rest", 0)
    _check(wl, W.prefix_lengths(wl, seed=1))


def test_prefix_ragged_workload():
    wl = W.make("ragged", 0)
    _check(wl, W.prefix_lengths(wl, seed=2), rows=sample_rows(wl, 2000))


def test_prefix_long_workload():
    wl = W.make("long", 0)
    _check(wl, W.prefix_lengths(wl, seed=3), rows=sample_rows(wl, 48))


@pytest.mark.parametrize("dh", [4, 32, 64, 128])
@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_prefix_fp32(dh, mode):
    wl = W.custom("f32", [5, 70, 33, 130], [3, 70, 1, 20], q=2, d=dh * 2, heads=2,
                  dtype="fp32", kv_mode=mode, seed=dh)
    _check(wl, W.prefix_lengths(wl, seed=dh), what="fp32 dh=%d %s" % (dh, mode))


@pytest.mark.parametrize("name", ["rest", "ragged"])
def test_attend_q_prefix_matches_forward_prefix(name):
    """xattn_attend_q_prefix over xattn_project's queries and the plan that
    xattn_forward_prefix left in the workspace gives the same bits."""
    require_gpu()
    wl = W.make(name, 0)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    cl = torch.from_numpy(W.prefix_lengths(wl, seed=9)).to("cuda")
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    a = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    workspace=ws, cand_kv_len=cl).clone()
    Q = ctx.project(t["Z"], t["W_Q"])
    b = ctx.attend_q(Q, t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws, cand_kv_len=cl)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_prefix_later_tiles_far_above_the_first(monkeypatch, mode):
    """Cutoffs on a memory whose later tiles score about 2^170 above the first
    (the moving-maximum pass, with lanes that see only the first tile, part
    of it or nothing)."""
    from test_gpu_parity import _rising_memory
    monkeypatch.setenv("XATTN_SHORT", "0")
    wl = _rising_memory(mode, 37)
    rng = np.random.default_rng(5)
    kv_len = np.concatenate([rng.integers(-3, int(wl.lengths[r]) + 4, int(wl.cu_cand[r + 1] - wl.cu_cand[r]))
                             for r in range(wl.R)]).astype(np.int32)
    kv_len[:4] = [0, 17, 64, 65]
    _check(wl, kv_len, what="prefix rising memory %s" % mode)
