"""GPU parity of the training pair: xattn_forward_train (the forward that also
stores each row's softmax normaliser per head) and xattn_backward_saved (the
backward that reuses those statistics instead of repeating the forward).

- O of the training forward: element-wise max-abs <= 2e-2 against the fp64
  oracle, as for xattn_forward.
- lse: against ln sum_j exp(s_j) = s_j* - ln p_j* at the row's largest oracle
  weight p_j* (oracle.probs, with s_j* from the oracle's projected query).  The
  kernel's scores come from the query rounded to bf16 twice (projection, then
  the folded softmax scale), so each score can be off by at most
  2^-8 * sum_e |q_e k_je| / sqrt(d_h) plus fp32 rounding, and a log-sum-exp
  moves by no more than its largest argument does; the test allows twice that.
- Gradients: normwise (max|delta| / max|ref|) <= 2e-2 against the oracle's,
  the bound of the recomputing backward; the bf16 O behind D adds one more
  bf16 rounding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from shared_history_candidate_amd import workloads as W
from shared_history_candidate_amd import xattn as X

from gpu_util import BF16_MAX_ABS, ctx_for, require_gpu, sample_rows

pytestmark = pytest.mark.gpu

BWD_BF16_NORM = 2e-2


def _up(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()


def _np(t, shape=None):
    a = t.float().cpu().numpy().astype(np.float64)
    return a.reshape(shape) if shape is not None else a


def _train(wl, kv_len=None):
    require_gpu()
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    cl = (torch.from_numpy(np.ascontiguousarray(kv_len, dtype=np.int32)).to("cuda")
          if kv_len is not None else None)
    O, lse = ctx.forward_train(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"],
                               wl.heads, cand_kv_len=cl)
    torch.cuda.synchronize()
    return ctx, t, cl, O, lse


def _check_lse(wl, lse, rows):
    """lse (log2 units) of the sampled rows against the oracle's normaliser."""
    dh = wl.d // wl.heads
    Q = oracle.project(wl.Z, wl.wt, wl.q).reshape(-1, wl.d)
    K = np.asarray(wl.K, dtype=np.float64).reshape(-1, wl.d)
    got = _np(lse).reshape(-1, wl.heads) * math.log(2.0)
    worst = 0.0
    for row in rows:
        r = int(np.searchsorted(np.asarray(wl.cu_cand) * wl.q, row, side="right") - 1)
        kv0, L = int(wl.cu_kv[r]), int(wl.cu_kv[r + 1] - wl.cu_kv[r])
        for h in range(wl.heads):
            g = got[row, h]
            if L == 0:
                assert g == -np.inf, (row, h, g)
                continue
            p = oracle.probs(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, int(row), h)
            j = int(np.argmax(p))
            qh = Q[row, h * dh:(h + 1) * dh]
            kh = K[kv0:kv0 + L, h * dh:(h + 1) * dh]
            s_j = float(qh @ kh[j]) / math.sqrt(dh)
            ref = s_j - math.log(p[j])
            bound = 2.0 * (2.0 ** -8 * float(np.max(np.abs(kh) @ np.abs(qh))) / math.sqrt(dh)
                           + 1e-5 * (1.0 + abs(ref)))
            err = abs(g - ref)
            worst = max(worst, err / bound)
            assert np.isfinite(g) and err <= bound, (row, h, g, ref, bound)
    return worst


@pytest.mark.parametrize("name", ["rest", "ragged"])
def test_forward_train_output_and_lse(name):
    wl = W.make(name, 0)
    _, _, _, O, lse = _train(wl)
    rows = sample_rows(wl, 48, seed=3)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V,
                         rows=rows)
    got = _np(O).reshape(-1, wl.d)[rows]
    err = float(np.max(np.abs(got - ref)))
    assert np.all(np.isfinite(got)) and err <= BF16_MAX_ABS, err
    worst = _check_lse(wl, lse, rows)
    print("%s: O max-abs %.3e, lse worst error / bound %.3f" % (name, err, worst))


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("dh,heads", [(32, 4), (64, 2), (128, 2)])
def test_forward_train_edge_shapes(mode, dh, heads):
    """Ragged tails and a request without memory rows (lse = -inf, O = 0)."""
    wl = W.custom("edge", [1, 0, 31, 65, 1023, 300], [1, 4, 65, 3, 129, 40], q=3,
                  d=dh * heads, heads=heads, dtype="bf16", kv_mode=mode, seed=dh)
    _, _, _, O, lse = _train(wl)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V)
    got = _np(O).reshape(-1, wl.d)
    assert float(np.max(np.abs(got - ref))) <= BF16_MAX_ABS
    _check_lse(wl, lse, np.arange(wl.rows))


def test_forward_train_short_memory_shape():
    """The short-memory kernel's lse (its scale is applied in fp32 to the
    unscaled scores, so it meets the backward's pre-scaled scores only to
    within the same bound)."""
    full = W.make("transx", 0)
    wl = W.custom("transx_part", full.lengths[:32], full.cands[:32], q=1, d=full.d,
                  heads=full.heads, dtype="bf16", kv_mode="separate", seed=4)
    ctx = ctx_for(wl)
    assert ctx.forward_path(wl.R, int(wl.cu_cand[-1]), int(wl.cu_kv[-1]), wl.heads) == \
        X.PATH_SHORT
    _, _, _, O, lse = _train(wl)
    rows = sample_rows(wl, 64, seed=5)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V,
                         rows=rows)
    assert float(np.max(np.abs(_np(O).reshape(-1, wl.d)[rows] - ref))) <= BF16_MAX_ABS
    _check_lse(wl, lse, rows)


def _saved_grads(wl, dO, kv_len=None):
    ctx, t, cl, O, lse = _train(wl, kv_len)
    g = ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], _up(dO, ctx.torch_dtype), t["cu_kv"],
                     t["cu_cand"], wl.heads, cand_kv_len=cl, O=O, lse=lse)
    torch.cuda.synchronize()
    return g


def _check_saved(wl, seed=0, kv_len=None, what=""):
    dO = W.output_grad(wl, seed)
    g = _saved_grads(wl, dO, kv_len)
    ref = oracle.backward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, dO,
                          kv_len=kv_len)
    names = [("dZ", "dZ"), ("dW_Q", "dwt"), ("dK", "dK")] + ([("dV", "dV")]
                                                             if wl.V is not None else [])
    for gn, rn in names:
        r = ref[rn]
        got = _np(g[gn], r.shape)
        err = float(np.max(np.abs(got - r))) if r.size else 0.0
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        rel = err / scale if scale > 0 else err
        print("saved %s %s: max-abs %.3e normwise %.3e" % (what, gn, err, rel))
        assert np.all(np.isfinite(got)) and rel <= BWD_BF16_NORM, (what, gn, rel)
    return g


@pytest.mark.parametrize("name", ["rest", "ragged"])
def test_backward_saved_workload(name):
    _check_saved(W.make(name, 0), seed=5, what=name)


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("q", [1, 3])
@pytest.mark.parametrize("dh,heads", [(32, 4), (64, 2), (128, 2)])
def test_backward_saved_edge_shapes(mode, q, dh, heads):
    wl = W.custom("edge", [1, 2, 31, 33, 0, 65, 97, 1023, 300], [1, 33, 65, 4, 129, 3, 64, 5, 40],
                  q=q, d=dh * heads, heads=heads, dtype="bf16", kv_mode=mode, seed=dh + q)
    _check_saved(wl, seed=q, what="edge dh=%d q=%d %s" % (dh, q, mode))


def test_backward_saved_prefix_ragged():
    wl = W.make("ragged", 0)
    _check_saved(wl, seed=8, kv_len=W.prefix_lengths(wl, seed=4, out_of_range=False),
                 what="ragged prefix")


def test_backward_saved_transx_part():
    """32 TransX requests: the short-memory kernel stores the statistics."""
    full = W.make("transx", 0)
    wl = W.custom("transx_part", full.lengths[:32], full.cands[:32], q=1, d=full.d,
                  heads=full.heads, dtype="bf16", kv_mode="separate", seed=3)
    _check_saved(wl, seed=6, what="transx part")


def test_backward_saved_deterministic_and_close_to_recomputed():
    """Two runs give the same bits; the recomputing backward differs only by
    the rounding of O behind D."""
    require_gpu()
    wl = W.make("ragged", 1)
    dO = W.output_grad(wl, 2)
    a = _saved_grads(wl, dO)
    b = _saved_grads(wl, dO)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    c = ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], _up(dO, ctx.torch_dtype), t["cu_kv"],
                     t["cu_cand"], wl.heads)
    torch.cuda.synchronize()
    for k in ("dZ", "dW_Q", "dK"):
        assert torch.equal(a[k], b[k]), k
        x, y = _np(a[k]), _np(c[k])
        assert float(np.max(np.abs(x - y))) <= 1e-2 * float(np.max(np.abs(y))), k


def test_training_pair_rejects_fp32_and_missing_statistics():
    require_gpu()
    wl = W.custom("f32", [5, 7], [2, 3], q=2, d=64, heads=2, dtype="fp32", kv_mode="shared",
                  seed=1)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    with pytest.raises(X.XAttnError) as e:
        ctx.forward_train(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads)
    assert e.value.status == X.XATTN_EUNSUPPORTED
    wb = W.custom("b", [5, 7], [2, 3], q=2, d=64, heads=2, dtype="bf16", kv_mode="shared",
                  seed=1)
    cb = ctx_for(wb)
    tb = X.to_device(wb)
    O, _ = cb.forward_train(tb["Z"], tb["W_Q"], tb["K"], tb["V"], tb["cu_kv"], tb["cu_cand"],
                            wb.heads)
    with pytest.raises(ValueError):
        cb.backward(tb["Z"], tb["W_Q"], tb["K"], tb["V"], O, tb["cu_kv"], tb["cu_cand"],
                    wb.heads, O=O)
