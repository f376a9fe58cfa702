"""GPU parity of the backward pass (xattn_backward) against the fp64 oracle's
gradients of <dO, O> on the same seeded inputs.  Tolerance per gradient
tensor, normwise (max|delta| / max|ref|): bf16 <= 2e-2 (the operands, P, dS
and dQ are rounded to bf16; a simulation of that arithmetic in numpy stays
below 6e-3 on these shapes), fp32 <= 1e-4.  Covers every head width, both
memory modes, one and three query slots, ragged and empty requests, the
serving and training workloads, and bitwise determinism."""
import numpy as np
import pytest
import torch

import oracle
from shared_history_candidate_amd import workloads as W
from shared_history_candidate_amd import xattn as X

from gpu_util import ctx_for, require_gpu

pytestmark = pytest.mark.gpu

BWD_BF16_NORM = 2e-2
BWD_FP32_NORM = 1e-4


def _up(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()


def _gpu_grads(wl, dO, ctx=None):
    require_gpu()
    ctx = ctx or ctx_for(wl)
    t = X.to_device(wl)
    g = ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], _up(dO, ctx.torch_dtype), t["cu_kv"],
                     t["cu_cand"], wl.heads)
    torch.cuda.synchronize()
    return g


def _np(t, shape=None):
    a = t.float().cpu().numpy().astype(np.float64)
    return a.reshape(shape) if shape is not None else a


def _check(wl, seed=0, what=""):
    dO = W.output_grad(wl, seed)
    g = _gpu_grads(wl, dO)
    ref = oracle.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, dO)
    tol = BWD_BF16_NORM if wl.dtype == "bf16" else BWD_FP32_NORM
    pairs = [("dZ", g["dZ"], ref["dZ"]), ("dW_Q", g["dW_Q"], ref["dwt"]),
             ("dK", g["dK"], ref["dK"])]
    if wl.V is not None:
        pairs.append(("dV", g["dV"], ref["dV"]))
    out = {}
    for name, got, r in pairs:
        got = _np(got, r.shape)
        assert np.all(np.isfinite(got)), "%s: non-finite %s" % (what, name)
        err = float(np.max(np.abs(got - r))) if r.size else 0.0
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        rel = err / scale if scale > 0 else err
        print("%s %s: max|ref| %.3g max-abs %.3e normwise %.3e" % (what, name, scale, err, rel))
        assert rel <= tol, "%s %s normwise %.3e > %.1e" % (what, name, rel, tol)
        out[name] = got
    return out, ref


EDGE_LENGTHS = [1, 2, 31, 33, 63, 65, 97, 1023, 300]
EDGE_CANDS = [1, 33, 65, 0, 129, 3, 64, 5, 40]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("q", [1, 3])
@pytest.mark.parametrize("dh,heads", [(32, 4), (64, 2), (128, 2)])
def test_backward_edge_shapes_bf16(mode, q, dh, heads):
    wl = W.custom("edge", EDGE_LENGTHS, EDGE_CANDS, q=q, d=dh * heads, heads=heads,
                  dtype="bf16", kv_mode=mode, seed=dh + q)
    _check(wl, seed=q, what="edge dh=%d q=%d %s" % (dh, q, mode))


@pytest.mark.parametrize("lengths,cands", [
    ([0, 40], [5, 7]),                 # request without memory rows: zero dZ for it
    ([10, 0, 0, 33], [0, 0, 4, 2]),    # memory nobody reads: zero dK
    ([1], [1]),
    ([700], [300]),                    # several query tiles and memory tiles
])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_edge_requests(lengths, cands, dtype):
    wl = W.custom("edge_req", lengths, cands, q=3, d=128, heads=2, dtype=dtype,
                  kv_mode="shared", seed=len(lengths))
    got, _ = _check(wl, seed=1, what="edge_req %s %s" % (lengths, dtype))
    for r in range(wl.R):
        if wl.lengths[r] == 0:
            a, b = wl.cu_cand[r] * wl.q, wl.cu_cand[r + 1] * wl.q
            assert np.all(got["dZ"].reshape(-1, wl.d)[a:b] == 0.0)
        if wl.cands[r] == 0:
            assert np.all(got["dK"][wl.cu_kv[r]:wl.cu_kv[r + 1]] == 0.0)


@pytest.mark.parametrize("dh", [4, 16, 32, 64, 128])
@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_backward_fp32(dh, mode):
    wl = W.custom("f32", [5, 70, 33, 130], [3, 70, 1, 20], q=2, d=dh * 2, heads=2,
                  dtype="fp32", kv_mode=mode, seed=dh)
    _check(wl, seed=dh, what="fp32 dh=%d %s" % (dh, mode))


@pytest.mark.parametrize("name", ["rest", "ragged"])
def test_backward_workload(name):
    _check(W.make(name, 0), seed=5, what=name)


def test_backward_transx_part():
    full = W.make("transx", 0)
    wl = W.custom("transx_part", full.lengths[:16], full.cands[:16], q=1, d=full.d,
                  heads=full.heads, dtype="bf16", kv_mode="separate", seed=3)
    _check(wl, seed=6, what="transx part")


def test_backward_long_memory():
    """One request with the long workload's memory (16384 rows, d = 512):
    the dK/dV kernel's query loop and the dQ kernel's memory loop at length."""
    wl = W.custom("long_one", [16384], [64], q=3, d=512, heads=8, dtype="bf16",
                  kv_mode="shared", seed=9)
    _check(wl, seed=7, what="long one request")


def test_backward_deterministic_bitwise():
    require_gpu()
    wl = W.make("ragged", 1)
    dO = W.output_grad(wl, 2)
    ctx = ctx_for(wl)
    a = _gpu_grads(wl, dO, ctx)
    b = _gpu_grads(wl, dO, ctx)
    for k in ("dZ", "dW_Q", "dK"):
        assert torch.equal(a[k], b[k]), k


def test_backward_no_candidates():
    """No query rows: every memory gradient and dW_Q are zero."""
    require_gpu()
    wl = W.custom("nocand", [40, 9], [0, 0], q=3, d=128, heads=2, dtype="bf16",
                  kv_mode="separate", seed=1)
    g = _gpu_grads(wl, np.zeros((0, 3, 128), dtype=np.float32))
    assert torch.count_nonzero(g["dK"]).item() == 0
    assert torch.count_nonzero(g["dV"]).item() == 0
    assert torch.count_nonzero(g["dW_Q"]).item() == 0


# ---------------------------------------------------------------------------
# Backward of the per-candidate prefix cutoff (ULT training batches)
# ---------------------------------------------------------------------------
def _check_prefix(wl, kv_len, seed=0, what=""):
    dO = W.output_grad(wl, seed)
    require_gpu()
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    cl = torch.from_numpy(np.ascontiguousarray(kv_len, dtype=np.int32)).to("cuda")
    g = ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], _up(dO, ctx.torch_dtype), t["cu_kv"],
                     t["cu_cand"], wl.heads, cand_kv_len=cl)
    torch.cuda.synchronize()
    ref = oracle.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, dO,
                          kv_len=kv_len)
    tol = BWD_BF16_NORM if wl.dtype == "bf16" else BWD_FP32_NORM
    names = [("dZ", "dZ"), ("dW_Q", "dwt"), ("dK", "dK")] + ([("dV", "dV")] if wl.V is not None
                                                             else [])
    for gn, rn in names:
        got = _np(g[gn], ref[rn].shape)
        r = ref[rn]
        err = float(np.max(np.abs(got - r)))
        scale = float(np.max(np.abs(r)))
        rel = err / scale if scale > 0 else err
        print("prefix %s %s: max-abs %.3e normwise %.3e" % (what, gn, err, rel))
        assert np.all(np.isfinite(got)) and rel <= tol, "%s %s normwise %.3e" % (what, gn, rel)


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("dh,heads", [(32, 4), (64, 2), (128, 2)])
def test_backward_prefix_edge_bf16(mode, dh, heads):
    wl = W.custom("edge", EDGE_LENGTHS, EDGE_CANDS, q=3, d=dh * heads, heads=heads,
                  dtype="bf16", kv_mode=mode, seed=dh)
    _check_prefix(wl, W.prefix_lengths(wl, seed=dh + 1), seed=2,
                  what="edge dh=%d %s" % (dh, mode))


@pytest.mark.parametrize("dh", [16, 64])
@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_backward_prefix_fp32(dh, mode):
    wl = W.custom("f32", [5, 70, 33, 130], [3, 70, 1, 20], q=2, d=dh * 2, heads=2,
                  dtype="fp32", kv_mode=mode, seed=dh)
    _check_prefix(wl, W.prefix_lengths(wl, seed=dh), seed=3, what="fp32 dh=%d %s" % (dh, mode))


def test_backward_prefix_ragged_training_batch():
    wl = W.make("ragged", 0)
    _check_prefix(wl, W.prefix_lengths(wl, seed=4, out_of_range=False), seed=8, what="ragged")


@pytest.mark.parametrize("name", ["rest", "ragged"])
def test_backward_prefix_full_length_matches_plain(name):
    """Cutoffs at or past L_r give the bits of the backward without cutoffs."""
    require_gpu()
    wl = W.make(name, 0)
    dO = _up(W.output_grad(wl, 3), torch.bfloat16)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    kv_len = np.repeat(wl.lengths, wl.cands).astype(np.int32)
    kv_len[::2] += 77
    a = ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], dO, t["cu_kv"], t["cu_cand"], wl.heads)
    b = ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], dO, t["cu_kv"], t["cu_cand"], wl.heads,
                     cand_kv_len=torch.from_numpy(kv_len).to("cuda"))
    torch.cuda.synchronize()
    for k in ("dZ", "dW_Q", "dK"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("ks", ["1", "2"])
@pytest.mark.parametrize("dh,heads,mode,cut", [(32, 4, "separate", False), (64, 2, "shared", True),
                                               (128, 2, "shared", False)])
def test_backward_dq_memory_splits(monkeypatch, ks, dh, heads, mode, cut):
    """The dQ kernel with 1 and 2 memory splits (forced through XATTN_DQ_KS;
    two splits are not built where their LDS would not fit twice per CU)."""
    monkeypatch.setenv("XATTN_DQ_KS", ks)
    wl = W.custom("ks", [700, 65, 1, 300], [40, 90, 2, 11], q=3, d=dh * heads, heads=heads,
                  dtype="bf16", kv_mode=mode, seed=int(ks) + dh)
    if cut:
        _check_prefix(wl, W.prefix_lengths(wl, seed=3), seed=4, what="ks=%s dh=%d" % (ks, dh))
    else:
        _check(wl, seed=4, what="ks=%s dh=%d %s" % (ks, dh, mode))
