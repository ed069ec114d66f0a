"""GPU parity of the non-quantised MLA prolog (``mla_prolog``, through the C ABI).

Expected values come from ``oracle.mla_prolog`` (fp64, "MlaProlog" page
formulas) on the exact bf16 inputs. Tolerance, element by element:
|gpu - oracle| <= 1e-2 + 2^-8 |oracle|, and mean |gpu - oracle| <= 3e-3 per
output. The outputs are bf16 (half an ulp is 2^-9 relative) of values with
unit root mean square; the fp32 products add little, and rounding c^Q to
bf16 before the second product adds about 2^-9 / sqrt(3) of the row's rms to
each q value (random-sign sum of 1024 terms).
Covered: the page's sizes at several t (one token, ragged tails of the
128-row tile, several tiles), other head counts (the column tiles not a
multiple of 8, which changes the launch's tile order), a smaller
q_lora_rank and h, row independence (a row's bits do not depend on the other
rows), the measured 16384-token workload on sampled rows, and the kv tile
run in the second product's launch (bit-exact against a call that runs it in
the first).
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


def _say(msg):
    print(msg, flush=True)


def run_gpu(d, eps=synth.PROLOG_EPS):
    q, kv, cq = mla.prolog(d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"],
                           d["gamma_cq"], d["gamma_ckv"], eps)
    torch.cuda.synchronize()
    return q, kv, cq


def run_oracle(d, rows=None, eps=synth.PROLOG_EPS):
    f = lambda x: x.double().cpu().numpy()
    x, cos, sin = f(d["token_x"]), f(d["rope_cos"]), f(d["rope_sin"])
    if rows is not None:
        x, cos, sin = x[rows], cos[rows], sin[rows]
    heads = d["wq_b"].shape[1] // d["wkv"].shape[1]
    return oracle.mla_prolog(x, f(d["wq_a"]), f(d["wq_b"]), f(d["wkv"]), cos, sin, f(d["gamma_cq"]),
                             f(d["gamma_ckv"]), heads, eps)


def assert_close(gpu, ref, what):
    g = gpu.double().cpu().numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite"
    err = np.abs(g - ref)
    bad = err > ABS + REL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, worst {err.max():.3e}"
    assert err.mean() <= MEAN, f"{what}: mean abs err {err.mean():.3e}"
    return float(err.max())


def check(d, what):
    q, kv, cq = run_gpu(d)
    rq, rkv, rcq = run_oracle(d)
    assert q.shape == rq.shape and kv.shape == rkv.shape and cq.shape == rcq.shape
    return (assert_close(q, rq, what + " q"), assert_close(kv, rkv, what + " kv"),
            assert_close(cq, rcq, what + " c^Q"))


@pytest.mark.parametrize("t", [1, 37, 128, 300])
def test_prolog_page_sizes_match_oracle(t):
    _say(f"[gpu] prolog page sizes t={t}")
    d = synth.prolog_inputs(t, seed=t, device=DEV, position0=7 * t)
    check(d, f"t={t}")


@pytest.mark.parametrize("cfg", [
    dict(t=200, h=4096, q_lora_rank=1024, num_heads=3),   # 3 column tiles: plain tile order
    dict(t=129, h=256, q_lora_rank=512, num_heads=8),      # one fp32 tile of c^Q, small K
    dict(t=70, h=128, q_lora_rank=1536, num_heads=16),     # three fp32 tiles, K = 128
], ids=["3-heads", "rank512-h256", "rank1536-h128"])
def test_prolog_other_sizes_match_oracle(cfg):
    _say(f"[gpu] prolog {cfg}")
    t = cfg.pop("t")
    d = synth.prolog_inputs(t, seed=5, device=DEV, **cfg)
    check(d, str(cfg))


def test_prolog_rows_are_independent():
    # every output row depends on its own token only. The first product is
    # split over K when the call has few 128-row tiles, into a number of runs
    # that depends on the tile count (h 4096: 16 at 257..384 rows, 32 up to
    # 128 rows), and the runs' sums are added in run order. A prefix run with
    # the same tile count gives the same bits as the full run; a shorter one
    # agrees to the prolog's tolerance.
    _say("[gpu] prolog row independence")
    d = synth.prolog_inputs(300, seed=9, device=DEV)
    full = run_gpu(d)
    for n, exact in ((260, True), (77, False)):
        part = {k: (v[:n].contiguous() if k in ("token_x", "rope_cos", "rope_sin") else v) for k, v in d.items()}
        pre = run_gpu(part)
        for name, a, b in zip(("q", "kv", "cq"), full, pre):
            if exact:
                assert torch.equal(a[:n], b), (n, name)
            else:
                assert_close(b, a[:n].double().cpu().numpy(), f"{n}-row prefix {name}")


def test_prolog_workload_sampled():
    t = synth.PROLOG_TOKENS
    _say(f"[gpu] prolog workload t={t}, sampled rows")
    d = synth.prolog_inputs(t, seed=1, device=DEV)
    q, kv, cq = run_gpu(d)
    assert torch.isfinite(q).all() and torch.isfinite(kv).all() and torch.isfinite(cq).all()
    rng = np.random.default_rng(17)
    rows = np.array(sorted(set(rng.integers(0, t, size=40).tolist()) | {0, 127, 128, t - 1}), np.int64)
    rq, rkv, rcq = run_oracle(d, rows)
    idx = torch.from_numpy(rows).to(DEV)
    assert_close(q[idx], rq, "workload q")
    assert_close(kv[idx], rkv, "workload kv")
    assert_close(cq[idx], rcq, "workload c^Q")


@pytest.mark.parametrize("t,heads", [(synth.PROLOG_TOKENS, 64), (11008, 3)], ids=["page-16384", "3-heads-11008"])
def test_prolog_kv_tile_in_second_launch_is_bit_exact(t, heads):
    # From 86 to 128 row tiles (about 10.9K to 16K tokens at these sizes) the
    # kv tile runs in the second product's launch, ahead of the head tiles
    # (3 heads: the head tiles not a multiple of 8, the other tile order).
    # Same arithmetic: the first 8192 rows equal an 8192-token call (kv tile
    # in the first launch; neither call splits the first product over K) bit
    # for bit, and so does the prepacked operator; sampled rows match the
    # oracle.
    n = 8192
    _say(f"[gpu] prolog kv tile placement, {t} vs {n} tokens, {heads} heads")
    d = synth.prolog_inputs(t, num_heads=heads, seed=41, device=DEV)
    full = run_gpu(d)
    part = {k: (v[:n].contiguous() if k in ("token_x", "rope_cos", "rope_sin") else v) for k, v in d.items()}
    sub = run_gpu(part)
    for name, a, b in zip(("q", "kv", "cq"), full, sub):
        assert torch.equal(a[:n], b), name
    packed = mla.pack_prolog_weights(d["wq_a"], d["wq_b"], d["wkv"])
    got = mla.prolog(d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"], d["gamma_cq"],
                     d["gamma_ckv"], synth.PROLOG_EPS, packed=packed)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "kv", "cq"), full, got):
        assert torch.equal(a, b), "prepacked " + name
    rows = np.array(sorted({0, n - 1, n, t - 1} | set(np.random.default_rng(43).integers(0, t, 12).tolist())),
                    np.int64)
    rq, rkv, rcq = run_oracle(d, rows)
    idx = torch.from_numpy(rows).to(DEV)
    for got_, ref, what in ((full[0][idx], rq, "q"), (full[1][idx], rkv, "kv"), (full[2][idx], rcq, "c^Q")):
        assert_close(got_, ref, what)


def test_prolog_rope_tables_with_unequal_pair_entries():
    """rope_cos / rope_sin hold one value per element ("MlaProlog" page,
    parameter list: [t, rope_dim]); with the two entries of every pair set
    apart (independent random tables) the kernel must read the odd element's
    own entries, as the oracle does."""
    t = 37
    _say(f"[gpu] prolog t={t}, pair-unequal rope tables")
    d = synth.prolog_inputs(t, seed=9, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(91)
    d["rope_cos"] = torch.rand((t, 64), generator=g, device=DEV).mul(2).sub(1).to(torch.bfloat16)
    d["rope_sin"] = torch.rand((t, 64), generator=g, device=DEV).mul(2).sub(1).to(torch.bfloat16)
    assert (d["rope_cos"][:, 0::2] != d["rope_cos"][:, 1::2]).float().mean() > 0.9
    q, kv, cq = run_gpu(d)
    rq, rkv, rcq = run_oracle(d)
    for got, ref, what in ((q, rq, "q"), (kv, rkv, "kv"), (cq, rcq, "c^Q")):
        assert_close(got, ref, what)


@pytest.mark.parametrize("t", [64, 300, 1024])
def test_prolog_prepacked_equals_packing_call(t):
    # weights packed once (mla_prolog_pack_weights) give the packing
    # operator's outputs bit for bit
    _say(f"[gpu] prolog prepacked, {t} tokens")
    d = synth.prolog_inputs(t, seed=31, device=DEV)
    packed = mla.pack_prolog_weights(d["wq_a"], d["wq_b"], d["wkv"])
    want = run_gpu(d)
    got = mla.prolog(d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"], d["gamma_cq"],
                     d["gamma_ckv"], synth.PROLOG_EPS, packed=packed)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "kv", "cq"), want, got):
        assert torch.equal(a, b), name


def test_prolog_prepacked_buffer_serves_many_calls():
    # one packed buffer, three calls with other tokens (same weights: the
    # generator seeds the weights independently of t)
    _say("[gpu] prolog prepacked, one buffer for several calls")
    d0 = synth.prolog_inputs(16, seed=32, device=DEV)
    packed = mla.pack_prolog_weights(d0["wq_a"], d0["wq_b"], d0["wkv"])
    for t in (1, 130, 16):
        d = synth.prolog_inputs(t, seed=32, device=DEV)
        assert all(torch.equal(d[k], d0[k]) for k in ("wq_a", "wq_b", "wkv"))
        got = mla.prolog(d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"], d["gamma_cq"],
                         d["gamma_ckv"], synth.PROLOG_EPS, packed=packed)
        torch.cuda.synchronize()
        for name, a, b in zip(("q", "kv", "cq"), run_gpu(d), got):
            assert torch.equal(a, b), (t, name)
