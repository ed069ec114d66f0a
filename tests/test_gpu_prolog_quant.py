"""GPU parity of the quantised MLA prolog (``mla_prolog_quant``, through the C ABI).

Expected values come from ``oracle.mla_prolog_quant`` (fp64; "MlaProlog" page,
mla_prolog_quant) on the exact inputs: bf16 activations and weights, int8
wq_b with float32 per-column scales.
  * q and kv, bf16: |gpu - oracle| <= 1e-2 + 2^-8 |oracle| per element and a
    mean of at most 3e-3, as for the plain prolog (outputs of unit rms, half
    a bf16 ulp 2^-9 relative). A code of c^Q that lands on the other side of
    a rounding boundary than the oracle's moves one of q_lora_rank terms of
    a product by one step, far inside that bound.
  * qr_scale_out, fp32: within 1e-4 relative of the oracle's max |c^Q| / 127
    (c^Q is an fp32 product of 4096 terms and an fp32 norm on the GPU).
  * qr_out, int8: the codes are a decision taken from fp32 values on the GPU
    and from fp64 values in the oracle. Where the oracle's c^Q / s lies
    farther than 5e-3 from a rounding boundary (k + 1/2), which is well above
    the fp32 error of c^Q / s (at most about 127 * 1e-5), the codes must be
    equal; elsewhere either neighbour is a correct rounding, so they may
    differ by 1. Every code lies in [-127, 127], and every row that is not
    zero reaches 127 in magnitude.
Covered: the page's sizes at t = 1, 37 and 130 (a ragged second 128-row
tile), 3 heads (plain tile order), q_lora_rank 512, 1536 and 2048 with small
h, a row of zeros (scale 0, codes 0, q row 0), row independence, and sampled
rows of the 16384-token workload.
"""
import numpy as np
import pytest
import torch

import mla_varlen_prefill_amd as mla
from mla_varlen_prefill_amd import synth
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
ABS, REL, MEAN = 1e-2, 2.0 ** -8, 3e-3
SCALE_REL = 1e-4
BOUNDARY = 5e-3


def _say(msg):
    print(msg, flush=True)


def run_gpu(d, eps=synth.PROLOG_EPS):
    out = mla.prolog_quant(d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"],
                           d["gamma_cq"], d["gamma_ckv"], d["wq_b_scale"], eps)
    torch.cuda.synchronize()
    return out


def run_oracle(d, rows=None, eps=synth.PROLOG_EPS):
    f = lambda x: x.double().cpu().numpy()
    x, cos, sin = f(d["token_x"]), f(d["rope_cos"]), f(d["rope_sin"])
    if rows is not None:
        x, cos, sin = x[rows], cos[rows], sin[rows]
    heads = d["wq_b"].shape[1] // d["wkv"].shape[1]
    cq = oracle.rms_norm(x @ f(d["wq_a"]), f(d["gamma_cq"]), eps)
    q, kv, qr, s = oracle.mla_prolog_quant(x, f(d["wq_a"]), d["wq_b"].cpu().numpy(), f(d["wkv"]), cos, sin,
                                           f(d["gamma_cq"]), f(d["gamma_ckv"]), f(d["wq_b_scale"]), heads, eps)
    return q, kv, qr, s, cq


def assert_close(gpu, ref, what):
    g = gpu.double().cpu().numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite"
    err = np.abs(g - ref)
    bad = err > ABS + REL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, worst {err.max():.3e}"
    assert err.mean() <= MEAN, f"{what}: mean abs err {err.mean():.3e}"


def assert_codes(gqr, gs, rqr, rs, rcq, what):
    gqr = gqr.cpu().numpy().astype(np.int64)
    gs = gs.cpu().numpy().reshape(-1).astype(np.float64)
    assert np.all(np.abs(gqr) <= 127), f"{what}: code out of range"
    nz = rs > 0
    assert np.all(np.abs(gqr[nz]).max(axis=1) == 127), f"{what}: a row's largest code is not 127"
    assert np.all(gqr[~nz] == 0) and np.all(gs[~nz] == 0), f"{what}: zero row"
    assert np.allclose(gs[nz], rs[nz], rtol=SCALE_REL, atol=0), f"{what}: scales"
    u = np.where(nz[:, None], rcq / np.where(nz, rs, 1.0)[:, None], 0.0)
    near = np.abs(np.abs(u - np.floor(u)) - 0.5) < BOUNDARY
    diff = gqr - rqr
    assert np.all(diff[~near] == 0), f"{what}: {int((diff[~near] != 0).sum())} codes differ away from a boundary"
    assert np.all(np.abs(diff[near]) <= 1), f"{what}: a boundary code differs by more than 1"


def check(d, what):
    q, kv, qr, qs = run_gpu(d)
    rq, rkv, rqr, rs, rcq = run_oracle(d)
    assert q.shape == rq.shape and kv.shape == rkv.shape and qr.shape == rqr.shape and qs.shape == (rq.shape[0], 1)
    assert qr.dtype == torch.int8 and qs.dtype == torch.float32
    assert_codes(qr, qs, rqr, rs, rcq, what + " c^Q codes")
    assert_close(q, rq, what + " q")
    assert_close(kv, rkv, what + " kv")


@pytest.mark.parametrize("t", [1, 37, 130])
def test_prolog_quant_page_sizes_match_oracle(t):
    _say(f"[gpu] quantised prolog page sizes t={t}")
    d = synth.prolog_quant_inputs(t, seed=t + 3, device=DEV, position0=5 * t)
    check(d, f"t={t}")


@pytest.mark.parametrize("cfg", [
    dict(t=200, h=4096, q_lora_rank=1024, num_heads=3),
    dict(t=129, h=256, q_lora_rank=512, num_heads=8),
    dict(t=70, h=128, q_lora_rank=1536, num_heads=16),
    dict(t=40, h=128, q_lora_rank=2048, num_heads=4),
], ids=["3-heads", "rank512-h256", "rank1536-h128", "rank2048-h128"])
def test_prolog_quant_other_sizes(cfg):
    _say(f"[gpu] quantised prolog {cfg}")
    d = synth.prolog_quant_inputs(seed=11, device=DEV, **cfg)
    check(d, str(cfg))


def test_prolog_quant_zero_row_and_row_independence():
    _say("[gpu] quantised prolog zero row, row independence")
    d = synth.prolog_quant_inputs(150, seed=21, device=DEV)
    d["token_x"][17] = 0
    q, kv, qr, qs = run_gpu(d)
    assert float(qs[17]) == 0.0 and int(qr[17].abs().max()) == 0 and float(q[17].abs().max()) == 0.0
    check(d, "zero row")
    # rows 0..63 alone give the same bits as inside the 150-row call
    d2 = {k: (v[:64].clone() if k in ("token_x", "rope_cos", "rope_sin") else v) for k, v in d.items()}
    q2, kv2, qr2, qs2 = run_gpu(d2)
    assert torch.equal(q2, q[:64]) and torch.equal(kv2, kv[:64]) and torch.equal(qr2, qr[:64])
    assert torch.equal(qs2, qs[:64])


def test_prolog_quant_workload_sampled_rows():
    """The 16384-token workload (the bench's call): every output row is
    computed; seeded rows, the first and the last, are checked against the
    oracle."""
    t = synth.PROLOG_TOKENS
    _say(f"[gpu] quantised prolog {t} tokens, sampled rows")
    d = synth.prolog_quant_inputs(t, seed=5, device=DEV)
    q, kv, qr, qs = run_gpu(d)
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[0, t - 1, 127, 128], rng.choice(t, 60, replace=False)]))
    rq, rkv, rqr, rs, rcq = run_oracle(d, rows)
    ri = torch.as_tensor(rows, device=DEV)
    assert_codes(qr[ri], qs[ri], rqr, rs, rcq, "workload codes")
    assert_close(q[ri], rq, "workload q")
    assert_close(kv[ri], rkv, "workload kv")


@pytest.mark.parametrize("t", [37, 300])
def test_prolog_quant_prepacked_equals_packing_call(t):
    # int8 wq_b packed once gives the packing operator's outputs bit for bit
    _say(f"[gpu] quantised prolog prepacked, {t} tokens")
    d = synth.prolog_quant_inputs(t, seed=33, device=DEV)
    packed = mla.pack_prolog_weights(d["wq_a"], d["wq_b"], d["wkv"])
    want = run_gpu(d)
    got = mla.prolog_quant(d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"],
                           d["gamma_cq"], d["gamma_ckv"], d["wq_b_scale"], synth.PROLOG_EPS, packed=packed)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "kv", "codes", "scales"), want, got):
        assert torch.equal(a, b), name
