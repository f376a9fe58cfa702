"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  bf16: element-wise max-abs <= 2e-2; fp32: normwise
relative <= 1e-4; integer plan outputs bit-exact.  The benchmark workloads
run at full size with seeds 0-4: every row where the host oracle is fast
enough (tiny, rest, ragged, transx), and on the long history the rows of
every (request, slot, 32-candidate block) work item."""
import ctypes

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


def _check(wl, rows=None, what=""):
    got = gpu_forward(wl)
    ref = _oracle(wl, rows)
    if rows is not None:
        got = got[rows]
    err, rel = assert_close(got, ref, wl.dtype, what or wl.name)
    print("%s: rows=%d max-abs %.3e normwise %.3e" % (what or wl.name, len(ref), err, rel))
    return err


# ---------------------------------------------------------------------------
# The five benchmark workloads, seeds 0-4
# ---------------------------------------------------------------------------
SEEDS = range(5)


def block_rows(wl, block=32, seed=0):
    """Rows of every (request, slot, block of `block` candidates) work item of
    the attention kernels: the block's first and last candidate and one drawn
    inside it, for every slot (every head is compared on each row)."""
    rng = np.random.default_rng(seed)
    rows = set()
    for r in range(wl.R):
        c0, c1 = int(wl.cu_cand[r]), int(wl.cu_cand[r + 1])
        for b0 in range(c0, c1, block):
            b1 = min(b0 + block, c1)
            for c in {b0, b1 - 1, int(rng.integers(b0, b1))}:
                rows.update(c * wl.q + s for s in range(wl.q))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("seed", SEEDS)
def test_config_tiny_fp32(seed):
    _check(W.make("tiny", seed), what="tiny seed %d" % seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_config_rest_bf16(seed):
    _check(W.make("rest", seed), what="rest seed %d" % seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_config_ragged_bf16(seed):
    """Every row."""
    _check(W.make("ragged", seed), what="ragged seed %d" % seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_config_transx_bf16(seed):
    """Every row (262144 query rows)."""
    _check(W.make("transx", seed), what="transx seed %d" % seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_config_long_bf16(seed):
    """Rows of every (request, slot, 32-candidate block) work item: 4 x 3 x
    16 blocks, each checked at its first, last and one inner candidate."""
    wl = W.make("long", seed)
    rows = block_rows(wl, 32, seed)
    assert len(rows) >= wl.R * wl.q * (512 // 32) * 2
    _check(wl, rows=rows, what="long seed %d" % seed)


# ---------------------------------------------------------------------------
# Edge shapes: ragged tails of both tiles, empty requests, every d_h, q, mode
# ---------------------------------------------------------------------------
EDGE_LENGTHS = [1, 2, 31, 33, 63, 65, 97, 1023]
EDGE_CANDS = [1, 33, 65, 0, 129, 3, 64, 5]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("q", [1, 3])
@pytest.mark.parametrize("dh,heads", [(32, 4), (64, 2), (128, 2)])
def test_edge_shapes_bf16(mode, q, dh, heads):
    wl = W.custom("edge", EDGE_LENGTHS, EDGE_CANDS, q=q, d=dh * heads, heads=heads,
                  dtype="bf16", kv_mode=mode, seed=dh + q)
    _check(wl, what="edge dh=%d q=%d %s" % (dh, q, mode))


@pytest.mark.parametrize("lengths,cands", [
    ([0, 40], [5, 7]),                 # request without memory rows -> zeros
    ([10, 0, 0, 33], [0, 0, 4, 2]),    # empty requests of both kinds
    ([1], [1]),                        # one row, one candidate
    ([4096], [300]),                   # long memory, several tiles of queries
])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_requests(lengths, cands, dtype):
    wl = W.custom("edge_req", lengths, cands, q=3, d=128, heads=2, dtype=dtype,
                  kv_mode="shared", seed=len(lengths))
    _check(wl)
    got = gpu_forward(wl)
    for r in range(wl.R):
        if wl.lengths[r] == 0:
            a, b = wl.cu_cand[r] * wl.q, wl.cu_cand[r + 1] * wl.q
            assert np.all(got[a:b] == 0.0)


def test_many_small_requests():
    rng = np.random.default_rng(7)
    R = 256
    wl = W.custom("many", rng.integers(1, 41, R), rng.integers(0, 6, R), q=3, d=256, heads=4,
                  dtype="bf16", kv_mode="separate", seed=7)
    _check(wl)


@pytest.mark.parametrize("dh", [4, 16, 32, 64, 128])
@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_fp32_mode(dh, mode):
    wl = W.custom("f32", [5, 70, 33], [3, 70, 1], q=2, d=dh * 2, heads=2, dtype="fp32",
                  kv_mode=mode, seed=dh)
    _check(wl)


# ---------------------------------------------------------------------------
# Integer plan: bit-exact against the oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["rest", "ragged", "transx", "tiny"])
def test_plan_bit_exact(name):
    require_gpu()
    wl = W.make(name, 0)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    cu_q, row_req, tiles, tm = ctx.plan(t["cu_kv"], t["cu_cand"], wl.heads, wl.total_cand,
                                        wl.total_kv)
    o_cu_q, o_row_req, o_tiles = oracle.plan(wl.cu_kv, wl.cu_cand, wl.q, tm)
    assert np.array_equal(cu_q.cpu().numpy(), o_cu_q)
    assert np.array_equal(row_req.cpu().numpy(), o_row_req)
    assert np.array_equal(tiles.cpu().numpy(), o_tiles)


def test_plan_bit_exact_ragged_edges():
    require_gpu()
    rng = np.random.default_rng(3)
    for trial in range(4):
        R = int(rng.integers(1, 300))
        L = rng.integers(0, 50, R)
        N = rng.integers(0, 140, R)
        wl = W.custom("p", L, N, q=int(rng.integers(1, 4)), d=64, heads=2, dtype="bf16",
                      seed=trial)
        ctx = ctx_for(wl)
        t = X.to_device(wl)
        cu_q, row_req, tiles, tm = ctx.plan(t["cu_kv"], t["cu_cand"], wl.heads, wl.total_cand,
                                            wl.total_kv)
        o = oracle.plan(wl.cu_kv, wl.cu_cand, wl.q, tm)
        assert np.array_equal(cu_q.cpu().numpy(), o[0])
        assert np.array_equal(row_req.cpu().numpy(), o[1])
        assert np.array_equal(tiles.cpu().numpy(), o[2])


@pytest.mark.parametrize("R,spread", [(512, 10**6), (513, 40), (1025, 3), (2049, 10**6),
                                      (4096, 40), (4096, 10**6)])
def test_plan_bit_exact_many_requests(R, spread):
    """More requests than the planner has threads: the ranking sorts in LDS
    (few distinct lengths: long runs of ties broken by request index); 512
    and 513 requests sit on either side of the batches whose offsets the
    planner holds in LDS."""
    require_gpu()
    rng = np.random.default_rng(R + spread)
    wl = W.custom("p_many", rng.integers(0, spread, R) % 200, rng.integers(0, 5, R), q=2, d=64,
                  heads=2, dtype="bf16", seed=1)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    cu_q, row_req, tiles, tm = ctx.plan(t["cu_kv"], t["cu_cand"], wl.heads, wl.total_cand,
                                        wl.total_kv)
    o = oracle.plan(wl.cu_kv, wl.cu_cand, wl.q, tm)
    assert np.array_equal(cu_q.cpu().numpy(), o[0])
    assert np.array_equal(row_req.cpu().numpy(), o[1])
    assert np.array_equal(tiles.cpu().numpy(), o[2])


@pytest.mark.parametrize("R", [256, 300, 4096])
def test_forward_many_requests_projection_path(monkeypatch, R):
    """The planner inside the projection launch (256 threads) with more
    requests than threads; every row against the oracle."""
    monkeypatch.setenv("XATTN_SHORT", "0")
    require_gpu()
    rng = np.random.default_rng(R)
    wl = W.custom("many_gemm", rng.integers(0, 30, R), rng.integers(0, 4, R), q=3, d=256,
                  heads=4, dtype="bf16", kv_mode="separate", seed=R)
    assert ctx_for(wl).forward_path(wl.R, wl.total_cand, wl.total_kv, wl.heads) == X.PATH_GEMM
    _check(wl, what="many requests R=%d" % R)


# ---------------------------------------------------------------------------
# TSP projection entry point
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["rest", "tiny"])
def test_projection(name):
    require_gpu()
    wl = W.make(name, 0)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    Q = ctx.project(t["Z"], t["W_Q"])
    torch.cuda.synchronize()
    got = Q.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    ref = oracle.project(wl.Z, wl.wt, wl.q).reshape(-1, wl.d)
    if wl.dtype == "bf16":
        # fp32 accumulation, one rounding to bf16 (relative 2^-9) per element
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)
    else:
        assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))


# ---------------------------------------------------------------------------
# Behaviour: determinism, streams, workspace reuse, device-side validation
# ---------------------------------------------------------------------------
def test_deterministic_bitwise():
    wl = W.make("rest", 0)
    a = gpu_forward(wl)
    b = gpu_forward(wl)
    assert np.array_equal(a, b)


def test_shared_prefix_equivalence_on_gpu():
    """Scoring 12 candidates against one memory equals 12 single-candidate
    requests that each carry a copy of it (bitwise: rows are independent)."""
    base = W.custom("sp", [300], [12], q=3, d=256, heads=4, dtype="bf16", seed=11)
    rep = W.custom("sp_rep", [300] * 12, [1] * 12, q=3, d=256, heads=4, dtype="bf16", seed=11)
    rep.K = np.tile(base.K, (12, 1))
    rep.Z = base.Z.copy()
    rep.wt = base.wt.copy()
    assert np.array_equal(gpu_forward(base), gpu_forward(rep))


def test_non_default_stream_and_workspace_reuse():
    require_gpu()
    big = W.make("rest", 3)
    small = W.custom("small", [77, 5], [9, 40], q=3, d=256, heads=4, dtype="bf16", seed=5)
    ctx = ctx_for(big)
    ws = ctx.alloc_workspace(big.R, big.total_cand, big.heads)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = gpu_forward(big, ctx=ctx, stream=s, workspace=ws)
        b = gpu_forward(small, ctx=ctx, stream=s, workspace=ws)
    assert_close(a, _oracle(big), "bf16")
    assert_close(b, _oracle(small), "bf16")


def test_device_validation_flags_bad_offsets():
    require_gpu()
    wl = W.custom("bad", [10, 20], [4, 4], q=3, d=128, heads=2, dtype="bf16", seed=1)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    O = torch.full((wl.total_cand, wl.q, wl.d), 7.0, dtype=torch.bfloat16, device="cuda")
    bad_kv = torch.tensor([0, 25, 20], dtype=torch.int32, device="cuda")  # decreasing
    ctx.forward(t["Z"], t["W_Q"], t["K"], None, bad_kv, t["cu_cand"], wl.heads, O=O, workspace=ws)
    flag = ctypes.c_int32(0)
    st = X.lib().xattn_device_error(ctx._h, ctypes.c_void_p(ws.data_ptr()), ctypes.byref(flag),
                                    None)
    assert st == X.XATTN_EDEVICE_VALIDATION and flag.value == 1
    assert ctx.device_error(ws) == 1
    assert torch.all(O == 7.0)
    bad_c = torch.tensor([0, 4, 9], dtype=torch.int32, device="cuda")  # cu[R] != total_cand
    ctx.forward(t["Z"], t["W_Q"], t["K"], None, t["cu_kv"], bad_c, wl.heads, O=O, workspace=ws)
    assert ctx.device_error(ws) == 2
    assert torch.all(O == 7.0)
    ctx.forward(t["Z"], t["W_Q"], t["K"], None, t["cu_kv"], t["cu_cand"], wl.heads, O=O,
                workspace=ws)
    assert ctx.device_error(ws) == 0


@pytest.mark.parametrize("name", ["rest", "tiny"])
def test_attend_and_attend_q_match_forward(name):
    """attend (projection + attention over the stored plan) and attend_q
    (attention over caller-projected queries) run the same kernels as forward."""
    require_gpu()
    wl = W.make(name, 0)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    a = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    workspace=ws).clone()
    b = ctx.attend(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws)
    Q = ctx.project(t["Z"], t["W_Q"])
    c = ctx.attend_q(Q, t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, c)


@pytest.mark.parametrize("R,dh,heads,q,mode", [
    (1, 64, 4, 3, "shared"), (5, 32, 8, 2, "separate"), (16, 64, 2, 1, "shared"),
    (16, 128, 2, 3, "separate"), (17, 64, 4, 3, "shared"), (3, 64, 8, 2, "shared"),
    # 32-wide heads over one memory: head pairs (an even count) and single heads
    (7, 32, 8, 2, "shared"), (4, 32, 3, 1, "shared"), (9, 32, 2, 3, "shared"),
])
def test_single_launch_and_split_paths_agree(R, dh, heads, q, mode):
    """Small batches on models up to 256 wide run as one launch (the attention
    kernel plans the batch and projects its own queries); attend_q runs the
    attention kernel over queries from the projection GEMM, and attend reads
    the plan the single launch published.  All three give the same bits, and
    match the oracle."""
    require_gpu()
    rng = np.random.default_rng(R * 100 + dh)
    wl = W.custom("paths", rng.integers(1, 300, R), rng.integers(0, 90, R), q=q, d=dh * heads,
                  heads=heads, dtype="bf16", kv_mode=mode, seed=R + dh)
    if wl.total_cand == 0:
        pytest.skip("no candidates drawn")
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    a = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    workspace=ws).clone()
    b = ctx.attend(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws)
    Q = ctx.project(t["Z"], t["W_Q"])
    c = ctx.attend_q(Q, t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = _oracle(wl)
    if ctx.forward_path(wl.R, wl.total_cand, wl.total_kv, wl.heads) == X.PATH_SHORT:
        # the short-memory kernel blocks the softmax differently from the
        # attention kernel attend_q runs: each is held to the oracle
        assert_close(c.float().cpu().numpy().astype(np.float64).reshape(wl.rows, wl.d), ref,
                     "bf16", "attend_q R=%d dh=%d" % (R, dh))
    else:
        assert torch.equal(a, c)
    got = a.float().cpu().numpy().astype(np.float64).reshape(wl.rows, wl.d)
    assert_close(got, ref, "bf16", "paths R=%d dh=%d" % (R, dh))


# ---------------------------------------------------------------------------
# Output gate and output projection of Eq. (7)
# ---------------------------------------------------------------------------
def _up(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt).contiguous()


@pytest.mark.parametrize("name,dtype", [("rest", "bf16"), ("transx", "bf16"), ("tiny", "fp32")])
def test_output_stage_alone(name, dtype):
    """xattn_output on a stand-in attention output against the oracle's gate
    and projection of the same inputs."""
    require_gpu()
    wl = W.make(name, 0)
    if name == "transx":   # a slice of the batch keeps the oracle fast
        wl = W.custom("transx_part", wl.lengths[:8], wl.cands[:8], q=wl.q, d=wl.d,
                      heads=wl.heads, dtype="bf16", kv_mode="separate", seed=3)
    wgo, wo = W.output_weights(wl, 5)
    O = W.attention_like(wl, 6)
    ctx = ctx_for(wl)
    dt = ctx.torch_dtype
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    Y = ctx.output(t["Z"], _up(wgo, dt), _up(O, dt), _up(wo, dt), ws)
    torch.cuda.synchronize()
    got = Y.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    ref = oracle.output(wl.Z, wgo, O, wo, wl.q)
    err, rel = assert_close(got, ref, wl.dtype, "output " + name)
    print("output %s: max-abs %.3e normwise %.3e" % (name, err, rel))


@pytest.mark.parametrize("name", ["rest", "ragged"])
def test_full_eq7(name):
    """Attention (xattn_forward) then the gate and output projection
    (xattn_output) against the oracle's full Eq. (7) on every row; the stored
    plan survives xattn_output (xattn_attend afterwards gives the same bits)."""
    require_gpu()
    wl = W.make(name, 0)
    wgo, wo = W.output_weights(wl, 7)
    ctx = ctx_for(wl)
    dt = ctx.torch_dtype
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    O = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    workspace=ws).clone()
    Y = ctx.output(t["Z"], _up(wgo, dt), O, _up(wo, dt), ws)
    O2 = ctx.attend(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    got = Y.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    ref = oracle.output(wl.Z, wgo, _oracle(wl), wo, wl.q)
    err, rel = assert_close(got, ref, wl.dtype, "eq7 " + name)
    print("full Eq. (7) %s: max-abs %.3e normwise %.3e" % (name, err, rel))


# ---------------------------------------------------------------------------
# Softmax reference: later memory tiles far above a split's first tile
# ---------------------------------------------------------------------------
def _rising_memory(mode, seed, heads=4):
    """Every query's scores against the memory rows past a request's first tile
    exceed its scores against the first tile by about 170 in log2 units, so
    their weights relative to the first tile's maximum overflow fp32: the
    kernel has to take its moving-maximum pass.  All later rows are the same
    key (the reference is the mean of their values, well conditioned); every
    query has a large component along that key's direction."""
    rng = np.random.default_rng(seed)
    lengths, cands = [64 * 3 + 17, 64 * 6, 200, 40, 130], [70, 5, 33, 9, 64]
    wl = W.custom("rising_" + mode, lengths, cands, q=1, d=256, heads=heads, dtype="bf16",
                  kv_mode=mode, seed=seed)
    dh = wl.d // wl.heads
    z0 = 3.0 * rng.standard_normal(wl.d)
    wl.Z = W.round_bf16(z0[None, None, :] + 0.3 * rng.standard_normal(wl.Z.shape))
    w = z0 @ wl.wt[0].T                       # the common query direction
    K = np.empty_like(wl.K)
    for h in range(wl.heads):
        u = w[h * dh:(h + 1) * dh]
        K[:, h * dh:(h + 1) * dh] = 20.0 * u / np.linalg.norm(u)
    for r in range(wl.R):
        a = int(wl.cu_kv[r])
        K[a:a + 64] *= -1.0                   # the first tile points the other way
    wl.K = W.round_bf16(K)
    return wl


@pytest.mark.parametrize("variant", ["default", "2,2", "4,1", "2,1", "1,4"])
@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_later_tiles_far_above_the_first(monkeypatch, mode, variant):
    monkeypatch.setenv("XATTN_SHORT", "0")
    if variant != "default":
        monkeypatch.setenv("XATTN_VARIANT", variant)
    require_gpu()
    wl = _rising_memory(mode, 31)
    _check(wl, what="rising memory %s variant %s" % (mode, variant))


@pytest.mark.parametrize("variant", ["default", "2,1", "4,1"])
def test_later_tiles_far_above_the_first_head_pairs(monkeypatch, variant):
    """The same memory at 32-wide heads over one K = V memory, attended over
    projected queries (attend_q), where a work-group takes two heads over
    shared tiles: the moving-maximum pass runs for the pair."""
    monkeypatch.setenv("XATTN_SHORT", "0")
    if variant != "default":
        monkeypatch.setenv("XATTN_VARIANT", variant)
    require_gpu()
    wl = _rising_memory("shared", 37, heads=8)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    # the forward leaves the batch's plan in the workspace for attend_q
    a = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    workspace=ws).clone()
    Q = ctx.project(t["Z"], t["W_Q"])
    O = ctx.attend_q(Q, t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, O)
    got = O.float().cpu().numpy().astype(np.float64).reshape(wl.rows, wl.d)
    err, rel = assert_close(got, _oracle(wl), "bf16", "rising memory head pairs %s" % variant)
    print("rising memory head pairs %s: max-abs %.3e normwise %.3e" % (variant, err, rel))


@pytest.mark.parametrize("cut", [False, True])
@pytest.mark.parametrize("heads", [2, 6, 16, 32])
def test_head_pairs_every_pair_count(heads, cut):
    """32-wide heads over one K = V memory run as head pairs; the work-group
    order is XCD-chunked when the pair count divides 8 (1, 8 pairs here) and
    plain otherwise (3, 16 pairs).  Every row of a 24-request batch (more
    than the single launch takes, so the projection GEMM and the attention
    kernel run) against the oracle, with and without per-candidate prefix
    cutoffs."""
    require_gpu()
    rng = np.random.default_rng(heads * 10 + cut)
    R = 24
    lengths = rng.integers(1, 700, R)
    cands = rng.integers(0, 80, R)
    wl = W.custom("pairs%d" % heads, lengths, cands, q=2, d=32 * heads, heads=heads,
                  dtype="bf16", kv_mode="shared", seed=heads + 100 * cut)
    if wl.total_cand == 0:
        pytest.skip("no candidates drawn")
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    kv_len = W.prefix_lengths(wl, seed=heads) if cut else None
    cl = torch.from_numpy(kv_len).to("cuda") if cut else None
    O = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                    cand_kv_len=cl)
    torch.cuda.synchronize()
    got = O.float().cpu().numpy().astype(np.float64).reshape(wl.rows, wl.d)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V, kv_len=kv_len)
    err, rel = assert_close(got, ref, "bf16", "head pairs heads=%d cut=%d" % (heads, cut))
    print("head pairs heads=%d cut=%d: rows=%d max-abs %.3e normwise %.3e" % (heads, cut, wl.rows, err, rel))
