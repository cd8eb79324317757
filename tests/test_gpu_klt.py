"""GPU parity of the static per-head KLT key basis (NVKV_K_KLT).

* calibration (nvkv_calibrate_key_basis): the GPU's fp64 Jacobi basis against the oracle's
  LAPACK basis -- eigenvalue order and sign convention identical, columns of well-separated
  eigenvalues equal to 1e-5, orthonormal to 1e-5, an eigen-residual against the oracle's
  covariance; g_K within 1e-5 (the two bases agree to rounding, not bit for bit);
* encoding: with the oracle's basis and scales installed, codes and scales bit-exact (the
  fixed fp32 rotation order), with and without smoothing and the MSE scale search;
* decode, the fused decode step (its new-token rotation bit-exact) and causal prefill
  attention over KLT caches, to the decode bar;
* end to end with the GPU's own calibration against the oracle's own.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P
from tests.test_gpu_fused import check_cache_rows, gpu_decode_append, new_rows, spoil_slots
from tests.test_gpu_parity import assert_close, gpu_calibrate, gpu_decode, gpu_fill_cache, oracle_decode
from tests.test_gpu_prefill import assert_rows_close, gpu_prefill

pytestmark = pytest.mark.gpu

KLT = O.FLAG_KLT
KLT_FLAGS = [KLT, KLT | O.FLAG_SMOOTH]
_LAYERS = {}


def gpu_calibrate_basis(nk, kw, hkv, flags, r, exclude_pos0=True):
    W, Tw = kw.shape[0], kw.shape[1]
    basis = torch.empty((hkv, 128, 128), dtype=torch.float32, device="cuda")
    g = torch.full((2,), -1.0, dtype=torch.float32, device="cuda")
    wsb = nk.calibrate_key_basis_workspace_bytes(hkv)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    nk.calibrate_key_basis(P.to_dev_u16(kw), W, Tw, hkv, exclude_pos0, flags, r, basis, g, ws, wsb)
    torch.cuda.synchronize()
    return basis.cpu().numpy(), g.cpu().numpy()


def oracle_klt_layer(name, flags, T=None, sink=True):
    """Oracle calibration (s, r, basis, g) and encoding of a workload layer (memoised)."""
    key = (name, flags, T, sink)
    if key not in _LAYERS:
        c, k, v, kw, vw, q = P.workload(name, T=T, sink=sink)
        kwf, vwf = S.bf16_to_f32(kw), S.bf16_to_f32(vw)
        s, r, g = O.calibrate(kwf, vwf, True, flags)
        basis, lam = O.klt_basis(kwf, r if flags & O.FLAG_SMOOTH else None, flags)
        y = O.key_transform(S.bf16_to_f32(k), r[None, None], flags, basis)
        kc, ks = O.quantize_keys(y, g[0], flags)
        vc, vs = O.quantize_rows(S.bf16_to_f32(v), g[1])
        _LAYERS[key] = (c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs)
    return _LAYERS[key]


def oracle_klt_decode(q, s, flags, basis, kc, ks, vc, vs, g, seq, hkv):
    B, Hq = q.shape[:2]
    grp = Hq // hkv
    qp = O.query_transform(S.bf16_to_f32(q).astype(np.float64), np.repeat(s, grp, axis=0)[None], flags,
                           np.repeat(basis, grp, axis=0)[None])
    khat = [O.dequantize(kc[b], ks[b], g[0]) for b in range(B)]
    vhat = [O.dequantize(vc[b], vs[b], g[1]) for b in range(B)]
    return O.attention(qp, khat, vhat, seq, P.sm_scale()), max(float(np.abs(x).max()) for x in vhat)


def install(lib, c, k, v, flags, pages, s, r, g, basis):
    """GPU cache filled through quantize_append_kv with the oracle's calibration installed."""
    return gpu_fill_cache(lib, k, v, c["hkv"], flags, pages, torch.from_numpy(s).cuda(),
                          torch.from_numpy(r).cuda(), g, basis=basis,
                          chunk=1000 if c["T"] * c["B"] > 4000 else None)


@pytest.mark.parametrize("name", ["tiny", "layer"])
@pytest.mark.parametrize("flags", KLT_FLAGS)
def test_calibrate_key_basis_matches_oracle(lib, name, flags):
    c, k, v, kw, vw, q, s, r, g, basis, lam, *_ = oracle_klt_layer(name, flags)
    hkv = c["hkv"]
    sg, rg, gg = gpu_calibrate(lib, kw, vw, hkv, flags)
    assert np.array_equal(rg.cpu().numpy(), r)
    assert float(gg[1]) == g[1]                          # g_V as before; g_K comes with the basis
    Bg, g2 = gpu_calibrate_basis(lib, kw, hkv, flags, rg)
    assert abs(float(g2[0]) - float(g[0])) <= 1e-5 * float(g[0]) and float(g2[1]) == -1.0
    kwf = O.key_transform(S.bf16_to_f32(kw), r[None, None] if flags & O.FLAG_SMOOTH else None, flags & O.FLAG_SMOOTH)
    X = kwf[:, 1:].astype(np.float64).reshape(-1, hkv, 128)
    for h in range(hkv):
        Bo, Bh = basis[h].astype(np.float64), Bg[h].astype(np.float64)
        assert np.max(np.abs(Bh.T @ Bh - np.eye(128))) <= 1e-5
        D = X[:, h] - X[:, h].mean(0)
        C = D.T @ D / D.shape[0]
        resid = C @ Bh - Bh * lam[h][None, :]
        assert np.max(np.abs(resid)) <= 1e-5 * np.max(np.abs(lam[h]))
        l = lam[h]
        gap = np.minimum(np.abs(np.diff(l, prepend=np.inf)), np.abs(np.diff(l, append=-np.inf)))
        sep = gap > 1e-6 * np.abs(l).max()
        assert sep.sum() >= 100, (h, int(sep.sum()))          # most columns are determined
        assert np.max(np.abs(Bh[:, sep] - Bo[:, sep])) <= 1e-5, h


@pytest.mark.parametrize("name,flags", [("tiny", KLT), ("tiny", KLT | 1), ("tiny", KLT | 1 | O.FLAG_MSE_SCALE),
                                        ("layer", KLT | 1)])
@pytest.mark.parametrize("paged", [False, True])
def test_quantize_klt_bit_exact(lib, name, flags, paged):
    c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs = oracle_klt_layer(name, flags)
    pages = P.Pages(c["B"], c["T"], paged)
    cache = install(lib, c, k, v, flags, pages, s, r, g, basis)
    kd, ksd = cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy()
    vd, vsd = cache.v_data.cpu().numpy(), cache.v_scales.cpu().numpy()
    for b in range(c["B"]):
        gc, gs = P.rows_from_cache_vec(kd, ksd, pages, c["hkv"], b, c["T"])
        assert np.array_equal(gs, ks[b]), f"K scales differ, seq {b}"
        assert np.array_equal(gc, kc[b]), f"K codes differ, seq {b}"
        gc, gs = P.rows_from_cache_vec(vd, vsd, pages, c["hkv"], b, c["T"], values=True)
        assert np.array_equal(gs, vs[b]) and np.array_equal(gc, vc[b])


@pytest.mark.parametrize("name,flags", [("tiny", KLT), ("tiny", KLT | 1), ("layer", KLT | 1)])
def test_decode_klt_parity(lib, name, flags):
    c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs = oracle_klt_layer(name, flags)
    pages = P.Pages(c["B"], c["T"], True)
    cache = install(lib, c, k, v, flags, pages, s, r, g, basis)
    seq = [c["T"]] * c["B"]
    ref, vmax = oracle_klt_decode(q, s, flags, basis, kc, ks, vc, vs, g, seq, c["hkv"])
    for split in (0, 64):
        assert_close(gpu_decode(lib, cache, q, pages, seq, c["T"], split), ref, vmax, seq)


@pytest.mark.parametrize("name,flags", [("tiny", KLT | 1), ("tiny", KLT | 1 | O.FLAG_MSE_SCALE), ("layer", KLT | 1)])
def test_fused_step_klt(lib, name, flags):
    c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs = oracle_klt_layer(name, flags)
    T, B, hkv = c["T"], c["B"], c["hkv"]
    pages = P.Pages(B, T, True)
    cache = install(lib, c, k, v, flags, pages, s, r, g, basis)
    seq = [T] * B
    kn, vn = new_rows(k, v, seq)
    ref, vmax = oracle_klt_decode(q, s, flags, basis, kc, ks, vc, vs, g, seq, hkv)
    for split in (0, 96):
        spoil_slots(lib, cache, pages, seq, hkv, seed=split)
        got = gpu_decode_append(lib, cache, q, kn, vn, pages, seq, T, split)
        assert_close(got, ref, vmax, seq)
        check_cache_rows(cache, pages, hkv, kc, ks, vc, vs, seq)


@pytest.mark.parametrize("name,Tq", [("tiny", 256), ("layer", 40)])
def test_prefill_klt_parity(lib, name, Tq):
    flags = KLT | 1
    c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs = oracle_klt_layer(name, flags)
    B, T, hkv, hq = c["B"], c["T"], c["hkv"], c["hq"]
    pages = P.Pages(B, T, True)
    cache = install(lib, c, k, v, flags, pages, s, r, g, basis)
    qb = S.make_query_block(c["cfg"], 0, B, Tq, hq)
    grp = hq // hkv
    qp = O.query_transform(S.bf16_to_f32(qb).astype(np.float64), np.repeat(s, grp, axis=0)[None, None], flags,
                           np.repeat(basis, grp, axis=0)[None, None])
    khat = [O.dequantize(kc[b], ks[b], g[0]) for b in range(B)]
    vhat = [O.dequantize(vc[b], vs[b], g[1]) for b in range(B)]
    vmax = max(float(np.abs(x).max()) for x in vhat)
    seq = [T] * B
    ref = O.causal_attention(qp, khat, vhat, seq, P.sm_scale())
    got = gpu_prefill(lib, cache, qb, pages, seq, T)
    assert_rows_close(got, ref, vmax, seq)


def test_klt_end_to_end_with_gpu_calibration(lib):
    """Product calibration (GPU s, r, basis, g) -> append -> decode, against the oracle's own
    calibration and encoding: the two bases agree to rounding, so a handful of codes may
    differ; the outputs agree to well within the quantisation error."""
    flags = KLT | 1
    c, k, v, kw, vw, q, s, r, g, basis, lam, kc, ks, vc, vs = oracle_klt_layer("tiny", flags)
    hkv = c["hkv"]
    sg, rg, gg = gpu_calibrate(lib, kw, vw, hkv, flags)
    Bg, g2 = gpu_calibrate_basis(lib, kw, hkv, flags, rg)
    gg[0] = float(g2[0])
    pages = P.Pages(c["B"], c["T"], True)
    cache = gpu_fill_cache(lib, k, v, hkv, flags, pages, sg, rg, gg, basis=Bg)
    codes = P.rows_from_cache_vec(cache.k_data.cpu().numpy(), cache.k_scales.cpu().numpy(), pages, hkv, 0, c["T"])
    assert np.mean(codes[0] != kc[0]) < 0.01
    seq = [c["T"]] * c["B"]
    ref, vmax = oracle_klt_decode(q, s, flags, basis, kc, ks, vc, vs, g, seq, hkv)
    got = gpu_decode(lib, cache, q, pages, seq, c["T"])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 1e-2, rel


def test_calibrate_key_basis_zero_windows(lib):
    """All-zero calibration keys: a zero covariance, whose eigenbasis is the identity in both
    implementations (no rotation happens; ties keep index order), and g_K = 1 (A_K = 0)."""
    hkv = 2
    kw = np.zeros((2, 9, hkv, 128), np.uint16)
    r = torch.ones((hkv, 128), dtype=torch.float32, device="cuda")
    Bg, g = gpu_calibrate_basis(lib, kw, hkv, KLT, r)
    Bo, _ = O.klt_basis(S.bf16_to_f32(kw), None, KLT)
    assert np.array_equal(Bg, Bo) and np.array_equal(Bg[0], np.eye(128, dtype=np.float32))
    assert float(g[0]) == 1.0


def test_calibrate_key_basis_rank_deficient(lib):
    """Keys confined (up to bf16 rounding) to a 16-dimensional subspace: the 16 leading
    columns are determined and match the oracle's; the near-null space is only required to
    be orthonormal and orthogonal to them."""
    rng = np.random.default_rng(17)
    U = np.linalg.qr(rng.standard_normal((128, 16)))[0]
    kw = S.bf16_round((rng.standard_normal((3, 65, 1, 16)) * np.linspace(3, 1, 16)) @ U.T)
    r = torch.ones((1, 128), dtype=torch.float32, device="cuda")
    Bg, g = gpu_calibrate_basis(lib, kw, 1, KLT, r)
    kwf = S.bf16_to_f32(kw)
    Bo, lam = O.klt_basis(kwf, None, KLT)
    Bh, Bref = Bg[0].astype(np.float64), Bo[0].astype(np.float64)
    assert np.max(np.abs(Bh.T @ Bh - np.eye(128))) <= 1e-5
    assert np.max(np.abs(Bh[:, :16] - Bref[:, :16])) <= 1e-5
    assert lam[0][15] > 1e3 * lam[0][16]
    _, _, go = O.calibrate(kwf, None, True, KLT)
    assert abs(float(g[0]) - float(go[0])) <= 1e-5 * float(go[0])
