"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare it with the fp64 oracle on the same seeded inputs."""
import numpy as np
import torch

from shared_history_candidate_amd import xattn as X

BF16_MAX_ABS = 2e-2      # bf16 operands, fp32 accumulation (element-wise max-abs)
FP32_NORM_REL = 1e-4     # fp32 mode: max|delta| / max|ref|


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (run them with -m gpu on an MI355X)")


def ctx_for(wl):
    return X.XAttn(wl.d, wl.q, wl.dtype, wl.kv_mode)


def gpu_forward(wl, ctx=None, stream=None, O=None, workspace=None):
    """Run xattn_forward on the workload; returns O as float64 numpy [rows, d]."""
    require_gpu()
    ctx = ctx or ctx_for(wl)
    t = X.to_device(wl)
    out = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                      O=O, workspace=workspace, stream=stream)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)


def sample_rows(wl, n, seed=0):
    """n random query rows plus the first and last row of every request."""
    rng = np.random.default_rng(seed)
    rows = set(rng.integers(0, wl.rows, size=min(n, wl.rows)).tolist()) if wl.rows else set()
    for r in range(wl.R):
        a, b = int(wl.cu_cand[r]) * wl.q, int(wl.cu_cand[r + 1]) * wl.q
        if b > a:
            rows.update([a, b - 1])
    return np.array(sorted(rows), dtype=np.int64)


def assert_close(got, ref, dtype, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output " + what
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    rel = err / scale if scale > 0 else err
    if dtype == "bf16":
        assert err <= BF16_MAX_ABS, "%s max-abs %.3e > %.1e (normwise %.3e)" % (what, err, BF16_MAX_ABS, rel)
    else:
        assert rel <= FP32_NORM_REL, "%s normwise rel %.3e > %.1e" % (what, rel, FP32_NORM_REL)
    return err, rel
