"""GPU parity of the single-launch output stage (csrc/output_bf16.hip: gate
GEMM, sigmoid, product with O and the W_o GEMM in one kernel, bf16, d = 256)
against the fp64 oracle's Eq. (7) gate and projection, element-wise max-abs
<= 2e-2; and bit-equality with the two GEMM launches (XATTN_FUSED_OUTPUT=0),
which compute the same arithmetic in the same order.

Shapes cross the kernel's boundaries: candidate counts that leave a partial
unit of 64 (1, 63, 65, 130, 1000), one or three slots (work-groups whose
share of units spans a slot change reload W_go), more units than
work-groups."""
import numpy as np
import pytest
import torch

import oracle
from shared_history_candidate_amd import workloads as W
from shared_history_candidate_amd import xattn as X

from gpu_util import assert_close, ctx_for, require_gpu

pytestmark = pytest.mark.gpu


def _up(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()


def _run(wl, wgo, wo, O, fused, monkeypatch):
    monkeypatch.setenv("XATTN_FUSED_OUTPUT", "1" if fused else "0")
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    dt = ctx.torch_dtype
    Y = ctx.output(t["Z"], _up(wgo, dt), _up(O, dt), _up(wo, dt), ws)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("total,q", [(1, 1), (63, 3), (65, 1), (130, 3), (1000, 1),
                                      (5000, 3)])
def test_output_single_launch(monkeypatch, total, q):
    require_gpu()
    wl = W.custom("out", [16], [total], q=q, d=256, heads=4, dtype="bf16", seed=total + q)
    wgo, wo = W.output_weights(wl, 5)
    O = W.attention_like(wl, 6)
    fused = _run(wl, wgo, wo, O, True, monkeypatch)
    split = _run(wl, wgo, wo, O, False, monkeypatch)
    assert torch.equal(fused, split)
    got = fused.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    ref = oracle.output(wl.Z, wgo, O, wo, wl.q)
    err, rel = assert_close(got, ref, "bf16", "output total=%d q=%d" % (total, q))
    print("output total=%d q=%d: max-abs %.3e normwise %.3e" % (total, q, err, rel))


def test_output_single_launch_transx_batch(monkeypatch):
    """The whole TransX-like batch (262144 candidates, one slot): bit-equal
    to the two launches, and the oracle on sampled rows."""
    require_gpu()
    wl = W.make("transx", 0)
    wgo, wo = W.output_weights(wl, 5)
    O = W.attention_like(wl, 6)
    fused = _run(wl, wgo, wo, O, True, monkeypatch)
    split = _run(wl, wgo, wo, O, False, monkeypatch)
    assert torch.equal(fused, split)
    rows = np.random.default_rng(1).choice(wl.total_cand, 2000, replace=False)
    got = fused.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)[rows]
    ref = oracle.output(wl.Z[rows], wgo, O[rows], wo, wl.q)
    assert_close(got, ref, "bf16", "output transx")
