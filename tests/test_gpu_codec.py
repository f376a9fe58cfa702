"""GPU parity of the coded memory (TransX report s.3) against the fp64 codec
oracle (oracle/codec.py) and the fp64 attention oracle.

  * encode: norms within fp32 rounding; every code inside the set of codes
    the fp32 arithmetic can reach: the GPU decides the code from an fp32
    rotation (a d_h-term dot product), the oracle from fp64, so the GPU's
    quantiser input t may differ from the exact one by the a-priori bound
    dt = (d_h + 4) 2^-24 sum_o |u_o E_oi| 2^b / (2 a) + 4 2^-24 (|t| + 1);
    its code must lie in [floor(t - dt), floor(t + dt)] (clamped), and must
    equal the oracle's wherever that set is a single code;
  * fold: the rotated query weights against E^T W_Q in fp64 (bf16 rounding);
  * attention over the coded memory: the oracle encodes and packs the memory
    (codes, and norms rounded to the fp32 the library takes), the library
    attends over exactly those codes, and the oracle decodes the same codes
    and norms (fp64) and runs its forward; element-wise max-abs <= 2e-2
    (bf16).  No input of these checks comes from the GPU.
The codebooks are fitted by the oracle on a sample of the memory rows with a
decaying spectrum, so bit tables are uneven and contain 0-bit coordinates."""
import numpy as np
import pytest
import torch

import oracle
from oracle import codec as OC
from shared_history_candidate_amd import workloads as W
from shared_history_candidate_amd import xattn as X

from gpu_util import assert_close, ctx_for, require_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _book(cb):
    return X.Codebook(cb["bits"], cb["center"], cb["half"], cb["rot"], cb["budget"])


def _setup(lengths, cands, dh, heads, mode, budget_per_coord, q=3, seed=0):
    wl = W.custom("codec", lengths, cands, q=q, d=dh * heads, heads=heads, dtype="bf16",
                  kv_mode=mode, seed=seed)
    K, V = W.anisotropic_memory(wl, seed + 1)
    budget = int(budget_per_coord * dh)
    cbk = OC.fit(K, heads, budget)
    cbv = OC.fit(V, heads, budget) if V is not None else None
    return wl, K, V, cbk, cbv


def _gpu_codes(ctx, cb, Xrows):
    t = torch.from_numpy(np.ascontiguousarray(Xrows, dtype=np.float32)).to("cuda").to(
        torch.bfloat16)
    codes, norms = ctx.codec_encode(_book(cb), t)
    torch.cuda.synchronize()
    return codes, norms


def _oracle_codes(cb, Xrows):
    """The oracle's codes of the rows Xrows as the library takes them (packed
    words [heads, n, words] int32 and fp32 norms [heads, n], on the device),
    and the oracle's fp64 decode of exactly those codes and norms."""
    n64, c = OC.encode(Xrows, cb)
    n32 = n64.astype(np.float32)
    words = OC.pack(c, cb["bits"])                           # [n, heads, words]
    codes_t = torch.from_numpy(
        np.ascontiguousarray(np.transpose(words, (1, 0, 2))).view(np.int32)).to("cuda")
    norms_t = torch.from_numpy(np.ascontiguousarray(n32.T)).to("cuda")
    return codes_t, norms_t, OC.decode(n32.astype(np.float64), c, cb)


def _unpacked(codes_t, cb):
    words = codes_t.cpu().numpy().view(np.uint32)            # [heads, n, words]
    return OC.unpack(np.transpose(words, (1, 0, 2)), cb["bits"])   # [n, heads, d_h]


@pytest.mark.parametrize("dh,heads,bpc", [(32, 4, 4), (64, 2, 3), (128, 2, 2), (64, 4, 8)])
def test_encode_matches_oracle(dh, heads, bpc):
    require_gpu()
    wl, K, _, cbk, _ = _setup([300, 97, 1], [4, 2, 1], dh, heads, "shared", bpc)
    ctx = ctx_for(wl)
    codes, norms = _gpu_codes(ctx, cbk, K)
    got = _unpacked(codes, cbk)
    ref_n, ref_c = OC.encode(K, cbk)
    assert np.allclose(norms.cpu().numpy().T, ref_n, rtol=2e-6, atol=0)
    # exact quantiser input and the fp32 error bound of the GPU's
    xr = OC.rotated_values(K, cbk)
    bits = cbk["bits"][None]
    lev = 2.0 ** bits
    half = cbk["half"][None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xr - cbk["center"][None] + half) / (2 * half) * lev
        u = np.stack([K[:, h * dh:(h + 1) * dh] / np.linalg.norm(K[:, h * dh:(h + 1) * dh],
                                                                 axis=1, keepdims=True)
                      for h in range(heads)], axis=1)
        sabs = np.einsum("nho,hoi->nhi", np.abs(u), np.abs(cbk["rot"]))
        dt = (dh + 4) * 2.0 ** -24 * sabs * lev / (2 * half) + 4 * 2.0 ** -24 * (np.abs(t) + 1)
    coded = np.broadcast_to(bits > 0, got.shape)
    lo = np.clip(np.floor(t - dt), 0, lev - 1)
    hi = np.clip(np.floor(t + dt), 0, lev - 1)
    ok = (got >= lo) & (got <= hi)
    assert np.all(ok[coded]), int(np.sum(~ok[coded]))
    assert np.all(got[~coded] == 0)
    single = coded & (lo == hi)
    assert np.array_equal(got[single], ref_c[single])
    print("dh=%d bpc=%d: codes %d, ambiguous under the fp32 bound %d, differing %d" %
          (dh, bpc, int(coded.sum()), int(np.sum(coded & (lo != hi))),
           int(np.sum(got != ref_c))))


def test_fold_query_weights():
    require_gpu()
    wl, K, _, cbk, _ = _setup([64], [2], 64, 4, "shared", 4)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    Wr = ctx.codec_fold(_book(cbk), t["W_Q"]).float().cpu().numpy()
    ref = np.zeros_like(wl.wt, dtype=np.float64)
    for h in range(4):
        rows = slice(h * 64, (h + 1) * 64)
        for s in range(wl.q):
            ref[s, rows] = cbk["rot"][h].T @ wl.wt[s, rows].astype(np.float64)
    err = np.max(np.abs(Wr - ref))
    assert err <= 2 ** -8 * np.max(np.abs(ref)) + 1e-6, err


EDGE_LENGTHS = [1, 31, 65, 97, 300, 0, 130]
EDGE_CANDS = [3, 65, 1, 40, 7, 2, 0]


@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("dh,heads,bpc", [(32, 4, 4), (64, 2, 4), (128, 2, 3), (64, 2, 8)])
def test_codec_attention_matches_oracle(mode, dh, heads, bpc, decode):
    """Both paths over a coded memory: each tile reconstructed in LDS (plain
    workspace) and the memory decoded once into bf16 planes (codec
    workspace)."""
    require_gpu()
    wl, K, V, cbk, cbv = _setup(EDGE_LENGTHS, EDGE_CANDS, dh, heads, mode, bpc, seed=dh)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    kc, kn, Kd = _oracle_codes(cbk, K)
    vc, vn, Vd = _oracle_codes(cbv, V) if V is not None else (None, None, None)
    Wr = ctx.codec_fold(_book(cbk), t["W_Q"])
    O = ctx.forward_codec(_book(cbk), _book(cbv) if cbv else None, t["Z"], Wr, kc, kn, vc, vn,
                          t["cu_kv"], t["cu_cand"], wl.heads, decode=decode)
    torch.cuda.synchronize()
    got = O.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, Kd, Vd)
    err, rel = assert_close(got, ref, "bf16", "codec %s dh=%d bpc=%d" % (mode, dh, bpc))
    print("codec %s dh=%d bpc=%d: max-abs %.3e normwise %.3e" % (mode, dh, bpc, err, rel))
    # requests without memory rows give zero rows
    for r in range(wl.R):
        if wl.lengths[r] == 0:
            a, b = wl.cu_cand[r] * wl.q, wl.cu_cand[r + 1] * wl.q
            assert np.all(got[a:b] == 0.0)


def test_codec_attention_transx_slice():
    """The TransX memory shape (96 rows: 64 recent + 32 summaries, separate
    K and V, one query per candidate) at 4.5 bits per coordinate."""
    require_gpu()
    full = W.make("transx", 0)
    wl = W.custom("transx_part", full.lengths[:8], full.cands[:8], q=1, d=full.d,
                  heads=full.heads, dtype="bf16", kv_mode="separate", seed=5)
    K, V = W.anisotropic_memory(wl, 6)
    budget = 288
    cbk, cbv = OC.fit(K, wl.heads, budget), OC.fit(V, wl.heads, budget)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    kc, kn, Kd = _oracle_codes(cbk, K)
    vc, vn, Vd = _oracle_codes(cbv, V)
    O = ctx.forward_codec(_book(cbk), _book(cbv), t["Z"], ctx.codec_fold(_book(cbk), t["W_Q"]),
                          kc, kn, vc, vn, t["cu_kv"], t["cu_cand"], wl.heads)
    torch.cuda.synchronize()
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, Kd, Vd)
    got = O.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    err, rel = assert_close(got, ref, "bf16", "codec transx")
    print("codec transx: max-abs %.3e normwise %.3e" % (err, rel))


@pytest.mark.parametrize("qw", ["2", "4", "8"])
@pytest.mark.parametrize("dh,heads,mode", [(32, 4, "separate"), (64, 2, "shared"),
                                           (128, 2, "separate")])
def test_codec_every_query_wave_count(monkeypatch, qw, dh, heads, mode):
    """Work-groups of 2, 4 and 8 query waves sharing each reconstructed tile
    (forced through XATTN_CODEC_QW) give the oracle's result."""
    require_gpu()
    monkeypatch.setenv("XATTN_CODEC_QW", qw)
    wl, K, V, cbk, cbv = _setup([700, 65, 1, 300], [90, 300, 2, 11], dh, heads, mode, 4, seed=3)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    kc, kn, Kd = _oracle_codes(cbk, K)
    vc, vn, Vd = _oracle_codes(cbv, V) if V is not None else (None, None, None)
    O = ctx.forward_codec(_book(cbk), _book(cbv) if cbv else None, t["Z"],
                          ctx.codec_fold(_book(cbk), t["W_Q"]), kc, kn, vc, vn, t["cu_kv"],
                          t["cu_cand"], wl.heads, decode=False)
    torch.cuda.synchronize()
    got = O.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, Kd, Vd)
    err, rel = assert_close(got, ref, "bf16", "codec qw=%s dh=%d %s" % (qw, dh, mode))
    print("codec qw=%s dh=%d %s: max-abs %.3e" % (qw, dh, mode, err))


SHORT_LENGTHS = [1, 31, 32, 33, 95, 96, 97, 0, 250]
SHORT_CANDS = [3, 64, 65, 1, 129, 63, 2, 7, 128]


def _codec_forward(ctx, wl, t, K, V, cbk, cbv):
    """The library's coded forward over the oracle's codes of K (and V), and
    the oracle's decode of those codes."""
    kc, kn, Kd = _oracle_codes(cbk, K)
    vc, vn, Vd = _oracle_codes(cbv, V) if V is not None else (None, None, None)
    O = ctx.forward_codec(_book(cbk), _book(cbv) if cbv else None, t["Z"],
                          ctx.codec_fold(_book(cbk), t["W_Q"]), kc, kn, vc, vn, t["cu_kv"],
                          t["cu_cand"], wl.heads)
    torch.cuda.synchronize()
    return O.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d), Kd, Vd


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("dh,heads,bpc", [(32, 8, 4), (64, 4, 4.5), (128, 2, 3), (64, 4, 8)])
def test_codec_short_memory_kernel(monkeypatch, mode, dh, heads, bpc):
    """The short-memory kernel over a coded memory (d = 256): each request's
    memory decoded once per work-group, keys in the rotated basis, values
    rotated back on the matrix cores; memories longer than 96 rows streamed
    in chunks.  Against the oracle's decode of its own codes (the ones the
    library attends over) and its forward."""
    monkeypatch.setenv("XATTN_SHORT", "1")
    require_gpu()
    wl, K, V, cbk, cbv = _setup(SHORT_LENGTHS, SHORT_CANDS, dh, heads, mode, bpc, seed=dh + 1)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    got, Kd, Vd = _codec_forward(ctx, wl, t, K, V, cbk, cbv)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, Kd, Vd)
    err, rel = assert_close(got, ref, "bf16", "codec short %s dh=%d bpc=%g" % (mode, dh, bpc))
    print("codec short %s dh=%d bpc=%g: max-abs %.3e normwise %.3e" % (mode, dh, bpc, err, rel))
    for r in range(wl.R):
        if wl.lengths[r] == 0:
            a, b = wl.cu_cand[r] * wl.q, wl.cu_cand[r + 1] * wl.q
            assert np.all(got[a:b] == 0.0)


def test_codec_short_memory_transx_batch():
    """The whole TransX-like batch at 4.5 bits per coordinate takes the
    short-memory kernel by default; sampled rows against the oracle."""
    require_gpu()
    full = W.make("transx", 0)
    wl = W.custom("transx_codec", full.lengths, full.cands, q=1, d=full.d, heads=full.heads,
                  dtype="bf16", kv_mode="separate", seed=5)
    K, V = W.anisotropic_memory(wl, 6)
    cbk, cbv = OC.fit(K, wl.heads, 288), OC.fit(V, wl.heads, 288)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    got, Kd, Vd = _codec_forward(ctx, wl, t, K, V, cbk, cbv)
    rows = np.sort(np.random.default_rng(2).choice(wl.rows, 1500, replace=False))
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, Kd, Vd, rows=rows)
    err, rel = assert_close(got[rows], ref, "bf16", "codec transx batch")
    print("codec transx batch: max-abs %.3e normwise %.3e" % (err, rel))


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("dh,heads", [(64, 4), (128, 2)])
def test_codec_decoded_planes_long_memory(mode, dh, heads):
    """The decode path on memories of more decode blocks than the decode grid
    (9001 rows: work-groups loop over 64-row blocks, the last one partial),
    against the oracle on sampled rows; the same inputs through the per-tile
    reconstruction agree with it within the same bound."""
    require_gpu()
    wl, K, V, cbk, cbv = _setup([5000, 4001], [40, 3], dh, heads, mode, 4.5, seed=11)
    ctx = ctx_for(wl)
    t = X.to_device(wl)
    kc, kn, Kd = _oracle_codes(cbk, K)
    vc, vn, Vd = _oracle_codes(cbv, V) if V is not None else (None, None, None)
    Wr = ctx.codec_fold(_book(cbk), t["W_Q"])
    outs = {}
    for decode in (True, False):
        O = ctx.forward_codec(_book(cbk), _book(cbv) if cbv else None, t["Z"], Wr, kc, kn, vc,
                              vn, t["cu_kv"], t["cu_cand"], wl.heads, decode=decode)
        torch.cuda.synchronize()
        outs[decode] = O.float().cpu().numpy().astype(np.float64).reshape(-1, wl.d)
    rows = sample_rows(wl, 60)
    ref = oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, Kd, Vd, rows=rows)
    for decode in (True, False):
        err, rel = assert_close(outs[decode][rows], ref, "bf16",
                                "codec long %s dh=%d decode=%s" % (mode, dh, decode))
        print("codec long %s dh=%d decode=%s: max-abs %.3e" % (mode, dh, decode, err))
