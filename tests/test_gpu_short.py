"""GPU parity of the short-memory kernel (projection and attention in one
launch, csrc/short_bf16.hip) against the fp64 oracle: bf16 element-wise
max-abs <= 2e-2.

The kernel keeps a request's whole memory in LDS up to 96 rows (separate K
and V) or 192 rows (K = V) and streams longer memories in chunks of that
size; query rows go in chunks of 64 candidates.  The edge shapes cross every
one of those boundaries (memory lengths 0, 1, 31..33, 95..97, 191..193 and
multi-chunk ones; candidate counts 0, 1, 63..65, 127..129), every head width,
both memory modes and one or three query slots.  XATTN_SHORT=1 routes these
small batches to the kernel (by default only batches of more than 16 requests
whose mean memory fits take it)."""
import numpy as np
import pytest
import torch

import oracle
from shared_history_candidate_amd import workloads as W
from shared_history_candidate_amd import xattn as X

from gpu_util import assert_close, ctx_for, gpu_forward, require_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _oracle(wl, rows=None):
    return oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, rows=rows)


def _path(wl):
    return ctx_for(wl).forward_path(wl.R, wl.total_cand, wl.total_kv, wl.heads)


def _check_short(wl, what, rows=None):
    assert _path(wl) == X.PATH_SHORT, what
    got = gpu_forward(wl)
    ref = _oracle(wl, rows)
    if rows is not None:
        got = got[rows]
    err, rel = assert_close(got, ref, "bf16", what)
    print("%s: rows=%d max-abs %.3e normwise %.3e" % (what, len(ref), err, rel))
    return got


SEP_LENGTHS = [1, 31, 32, 33, 95, 96, 97, 0, 250]
SEP_CANDS = [3, 64, 65, 1, 129, 63, 2, 7, 128]
SHARED_LENGTHS = [1, 33, 191, 192, 193, 0, 450, 96]
SHARED_CANDS = [65, 2, 63, 128, 5, 4, 127, 64]


@pytest.mark.parametrize("q", [1, 3])
@pytest.mark.parametrize("dh,heads", [(32, 8), (64, 4), (128, 2)])
@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_short_edge_shapes(monkeypatch, mode, dh, heads, q):
    monkeypatch.setenv("XATTN_SHORT", "1")
    require_gpu()
    lengths, cands = (SEP_LENGTHS, SEP_CANDS) if mode == "separate" else (SHARED_LENGTHS,
                                                                           SHARED_CANDS)
    wl = W.custom("short_edge", lengths, cands, q=q, d=256, heads=heads, dtype="bf16",
                  kv_mode=mode, seed=dh + 7 * q)
    got = _check_short(wl, "short %s dh=%d q=%d" % (mode, dh, q))
    for r in range(wl.R):
        if wl.lengths[r] == 0:   # no memory rows: zero output rows
            a, b = wl.cu_cand[r] * wl.q, wl.cu_cand[r + 1] * wl.q
            assert np.all(got[a:b] == 0.0)


@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_short_many_requests_split_over_work_groups(monkeypatch, mode):
    """More work items than work-groups, not a multiple of them: work-groups
    start and end inside requests, meet empty ones, and restage memories."""
    monkeypatch.delenv("XATTN_SHORT", raising=False)
    require_gpu()
    rng = np.random.default_rng(5)
    R = 700
    lengths = rng.integers(0, 97, R)
    cands = rng.integers(0, 150, R)
    wl = W.custom("short_many", lengths, cands, q=1, d=256, heads=4, dtype="bf16",
                  kv_mode=mode, seed=9)
    _check_short(wl, "short many %s" % mode, rows=sample_rows(wl, 4000))


def test_short_transx_config_takes_the_short_path():
    """The TransX-like batch (256 requests x 96 memory rows, 1024 candidates
    with one query token) runs the short kernel by default."""
    require_gpu()
    wl = W.make("transx", 0)
    _check_short(wl, "transx", rows=sample_rows(wl, 3000))


@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_short_and_split_paths_agree(monkeypatch, mode):
    """Both paths within the bf16 bound of the oracle on the same inputs."""
    require_gpu()
    rng = np.random.default_rng(3)
    wl = W.custom("short_vs", rng.integers(1, 120, 40), rng.integers(0, 200, 40), q=3, d=256,
                  heads=4, dtype="bf16", kv_mode=mode, seed=4)
    ref = _oracle(wl)
    outs = {}
    for flag in ("1", "0"):
        monkeypatch.setenv("XATTN_SHORT", flag)
        assert _path(wl) == (X.PATH_SHORT if flag == "1" else X.PATH_GEMM)
        outs[flag] = gpu_forward(wl)
        assert_close(outs[flag], ref, "bf16", "XATTN_SHORT=%s %s" % (flag, mode))
    print("short vs split: max |diff| %.3e" % np.max(np.abs(outs["1"] - outs["0"])))


def test_short_attend_reuses_plan_and_is_deterministic(monkeypatch):
    """attend runs the same kernel over the plan forward stored: same bits,
    and the same bits again on a non-default stream."""
    monkeypatch.setenv("XATTN_SHORT", "1")
    require_gpu()
    wl = W.custom("short_attend", [96, 5, 200, 64], [300, 1, 70, 64], q=2, d=256, heads=4,
                  dtype="bf16", kv_mode="separate", seed=12)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    a = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    workspace=ws).clone()
    b = ctx.attend(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                        workspace=ws, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, c)
    got = a.float().cpu().numpy().astype(np.float64).reshape(wl.rows, wl.d)
    assert_close(got, _oracle(wl), "bf16", "short attend")


def test_short_device_validation_flags_bad_offsets(monkeypatch):
    """Offsets that fail the planner's check leave O untouched and raise the
    workspace flag, as on the other paths."""
    monkeypatch.setenv("XATTN_SHORT", "1")
    require_gpu()
    wl = W.custom("short_bad", [10, 20], [4, 4], q=1, d=256, heads=4, dtype="bf16",
                  kv_mode="separate", seed=1)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    O = torch.full((wl.total_cand, wl.q, wl.d), 7.0, dtype=torch.bfloat16, device="cuda")
    bad_kv = torch.tensor([0, 25, 20], dtype=torch.int32, device="cuda")   # decreasing
    ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], bad_kv, t["cu_cand"], wl.heads, O=O,
                workspace=ws)
    assert ctx.device_error(ws) == 1
    assert torch.all(O == 7.0)
    ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, O=O,
                workspace=ws)
    assert ctx.device_error(ws) == 0
    got = O.float().cpu().numpy().astype(np.float64).reshape(wl.rows, wl.d)
    assert_close(got, _oracle(wl), "bf16", "short after bad offsets")
