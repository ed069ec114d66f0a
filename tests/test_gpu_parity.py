"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Tolerance for attention outputs: max |gpu - oracle| <= 2e-2 and mean <= 2e-3
over every compared element; the gather and all index handling are compared
bit for bit. Small cases compare every output element; the full-size
workloads compare seeded samples of (sequence, head, row) triples plus the
boundary rows, and check whole-output properties (finite, deterministic).
"""
import math

import numpy as np
import pytest
import torch

import mla_varlen_prefill_amd as mla
from mla_varlen_prefill_amd import synth
import oracle

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def run_gpu(t, qs, ks, params, mask=None, mask_type=None):
    mt = params["mask_type"] if mask_type is None else mask_type
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, params["head_num"],
                      params["kv_head_num"], params["qk_scale"], mt, mask)
    torch.cuda.synchronize()
    return out


def oracle_full(t, qs, ks, params, mask=None, mask_type=None, kv_padded=False):
    mt = params["mask_type"] if mask_type is None else mask_type
    d = {n: x.double().cpu().numpy() for n, x in t.items()}
    if kv_padded:
        b, m = d["k"].shape[:2]
        hk = params["kv_head_num"]
        for n in ("k", "k_rope", "v"):
            d[n] = d[n].reshape(b, m, hk, -1)
    tile = mask.double().cpu().numpy() if mask is not None else None
    return oracle.attention(d["q"], d["q_rope"], d["k"], d["k_rope"], d["v"], qs, ks, params["head_num"],
                            params["kv_head_num"], params["qk_scale"], mt, tile, kv_padded=kv_padded)


def assert_close(gpu, ref, what):
    g = gpu.double().cpu().numpy() if isinstance(gpu, torch.Tensor) else gpu
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    assert err.max() <= MAX_ABS, f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean abs err {err.mean():.3e}"
    return float(err.max()), float(err.mean())


def make(qs, ks, heads, kv_heads, dtype=torch.bfloat16, sigma=1.0, seed=0, mask_type=synth.MASK_CAUSAL,
         scale=None, kv_padded_max_seq=0):
    t = synth.attention_inputs(qs, ks, heads, kv_heads, dtype, sigma, seed, DEV,
                               kv_padded_max_seq=kv_padded_max_seq)
    params = dict(head_num=heads, kv_head_num=kv_heads, qk_scale=synth.QK_SCALE if scale is None else scale,
                  mask_type=mask_type)
    return t, np.asarray(qs, np.int32), np.asarray(ks, np.int32), params


SMALL = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, dtype, mask_type
    ("tiny-workload", [17, 40], [17, 40], 4, 4, torch.bfloat16, synth.MASK_CAUSAL),
    ("ragged-causal", [1, 63, 64, 65, 129, 300], [1, 63, 64, 65, 129, 300], 2, 2, torch.bfloat16,
     synth.MASK_CAUSAL),
    ("ragged-undefined", [5, 130, 257], [77, 130, 190], 3, 3, torch.bfloat16, synth.MASK_UNDEFINED),
    ("spec-fp16", [64, 200], [64, 200], 2, 2, torch.float16, synth.MASK_SPEC),
    ("chunked-gqa", [100, 33], [700, 260], 8, 2, torch.bfloat16, synth.MASK_CAUSAL),
    ("mqa-fp16", [150], [150], 4, 1, torch.float16, synth.MASK_CAUSAL),
    ("q-longer-than-kv", [200, 70], [50, 0], 2, 2, torch.bfloat16, synth.MASK_CAUSAL),
    ("empty-sequences", [0, 45, 0], [10, 45, 0], 2, 2, torch.bfloat16, synth.MASK_CAUSAL),
    ("single-query-spec", [1, 1, 1], [1000, 3, 64], 4, 4, torch.bfloat16, synth.MASK_SPEC),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_match_oracle(case):
    name, qs, ks, h, hk, dt, mt = case
    _say(f"[gpu] {name}: q={qs} kv={ks} H={h} Hkv={hk} {dt} mask={mt}")
    t, qs, ks, params = make(qs, ks, h, hk, dt, seed=len(name), mask_type=mt)
    out = run_gpu(t, qs, ks, params)
    ref = oracle_full(t, qs, ks, params)
    assert_close(out, ref, name)


def test_padded_kv_layout_matches_oracle():
    qs, ks = [37, 90], [60, 90]
    _say(f"[gpu] padded layout q={qs} kv={ks}")
    t, qs, ks, params = make(qs, ks, 2, 2, seed=5, kv_padded_max_seq=128)
    out = run_gpu(t, qs, ks, params)
    ref = oracle_full(t, qs, ks, params, kv_padded=True)
    assert_close(out, ref, "padded")


def test_2d_query_and_output_forms():
    qs = [70, 20]
    t, qs, ks, params = make(qs, qs, 2, 2, seed=6)
    out3 = run_gpu(t, qs, ks, params)
    q2 = t["q"].reshape(t["q"].shape[0], -1)
    qr2 = t["q_rope"].reshape(t["q_rope"].shape[0], -1)
    out2 = torch.empty((q2.shape[0], 2 * 128), dtype=q2.dtype, device=DEV)
    mla.prefill(q2, qr2, t["k"], t["k_rope"], t["v"], qs, ks, 2, 2, params["qk_scale"], synth.MASK_CAUSAL,
                out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out2.reshape(out3.shape), out3)


def test_mask_free_with_causal_tile_equals_causal_bit_exact():
    # 40 heads: enough work that neither plan splits an item (a split plan
    # cuts a MASK_FREE item, which runs to the end of its 512-key block, at
    # other tiles than the causal one, so only the rounding would agree)
    qs, ks = [600, 1100], [1100, 1100]
    _say(f"[gpu] mask-free causal tile q={qs} kv={ks}")
    for mt in (synth.MASK_CAUSAL, synth.MASK_FREE):
        _, items, tasks = mla.mla_prefill_plan_host(qs, ks, 40, 40, mt)
        assert ((tasks[:, 2] == 0) & ((tasks[:, 0] < 0) | (tasks[:, 3] == items[tasks[:, 0], 2]))).all()
    t, qs, ks, params = make(qs, ks, 40, 40, seed=7)
    causal = run_gpu(t, qs, ks, params)
    for dt in (torch.float16, torch.bfloat16):
        tile = synth.causal_mask_tile(dt, DEV)
        free = run_gpu(t, qs, ks, params, mask=tile, mask_type=synth.MASK_FREE)
        assert torch.equal(free, causal)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_mask_free_random_tile_matches_oracle(dtype):
    qs, ks = [300, 530], [700, 530]
    _say(f"[gpu] mask-free random tile {dtype}")
    t, qs, ks, params = make(qs, ks, 2, 2, seed=8)
    tile = synth.random_mask_tile(9, dtype, DEV)
    out = run_gpu(t, qs, ks, params, mask=tile, mask_type=synth.MASK_FREE)
    ref = oracle_full(t, qs, ks, params, mask=tile, mask_type=synth.MASK_FREE)
    assert_close(out, ref, "mask-free random tile")


def test_rows_without_visible_keys_are_zero():
    t, qs, ks, params = make([200, 70], [50, 0], 2, 2, seed=10)
    out = run_gpu(t, qs, ks, params)
    assert (out[:150] == 0).all() and (out[200:] == 0).all()
    assert out[150:200].abs().sum() > 0


def test_causal_invariance_on_gpu():
    """Changing keys/values after position p leaves every row at positions <= p
    bit-identical."""
    n = 333
    t, qs, ks, params = make([n], [n], 2, 2, seed=11)
    base = run_gpu(t, qs, ks, params)
    cut = 190
    for name in ("k", "k_rope", "v"):
        t2 = dict(t)
        t2[name] = t[name].clone()
        t2[name][cut + 1:] += 3.0
        out = run_gpu(t2, qs, ks, params)
        assert torch.equal(out[:cut + 1], base[:cut + 1])
        assert not torch.equal(out[cut + 1:], base[cut + 1:])


def test_single_key_row_is_exact_value_row():
    t, qs, ks, params = make([64, 9], [64, 9], 4, 4, seed=12)
    out = run_gpu(t, qs, ks, params)
    assert torch.equal(out[0], t["v"][0])
    assert torch.equal(out[64], t["v"][64])


def test_zero_query_gives_mean_of_visible_values():
    n = 150
    t, qs, ks, params = make([n], [n], 1, 1, seed=13)
    t["q"].zero_()
    t["q_rope"].zero_()
    out = run_gpu(t, qs, ks, params).double().cpu().numpy()
    v = t["v"].double().cpu().numpy()
    ref = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None, None]
    assert np.abs(out - ref).max() <= MAX_ABS


def test_deterministic_rerun():
    t, qs, ks, params = make([300, 257], [300, 400], 4, 4, seed=14)
    a = run_gpu(t, qs, ks, params)
    b = run_gpu(t, qs, ks, params)
    assert torch.equal(a, b)


# ---------------------------------------------------------------- full sizes

def sampled_oracle_check(t, qs, ks, params, out, n_heads_sample, rows_per_head, seed, mask=None,
                         mask_type=None, extra_rows=()):
    """Compare sampled rows with the oracle. Picks (b, h) pairs, then rows in
    each: seeded random ones plus the first, second and last row and any
    ``extra_rows(b)`` given."""
    rng = np.random.default_rng(seed)
    mt = params["mask_type"] if mask_type is None else mask_type
    H, Hkv = params["head_num"], params["kv_head_num"]
    qoff = np.concatenate([[0], np.cumsum(qs)])
    koff = np.concatenate([[0], np.cumsum(ks)])
    tile = mask.double().cpu().numpy() if mask is not None else None
    errs = []
    bs = [b for b in range(len(qs)) if qs[b] > 0]
    for n in range(n_heads_sample):
        b = bs[n % len(bs)] if n < len(bs) else int(rng.choice(bs))
        h = int(rng.integers(0, H)) if n > 0 else H - 1
        hk = oracle.kv_head_of(h, H, Hkv)
        ql, kl = int(qs[b]), int(ks[b])
        rows = set(int(x) for x in rng.integers(0, ql, size=rows_per_head))
        rows |= {0, min(1, ql - 1), ql - 1}
        rows |= {r for r in extra_rows(b) if 0 <= r < ql} if callable(extra_rows) else set()
        rows = np.array(sorted(rows), dtype=np.int64)
        sl = slice(int(qoff[b]), int(qoff[b]) + ql)
        kv = slice(int(koff[b]), int(koff[b]) + kl)
        ref = oracle.attention_head(
            t["q"][sl, h].double().cpu().numpy(), t["q_rope"][sl, h].double().cpu().numpy(),
            t["k"][kv, hk].double().cpu().numpy(), t["k_rope"][kv, hk].double().cpu().numpy(),
            t["v"][kv, hk].double().cpu().numpy(), params["qk_scale"], mt, tile, rows=rows)
        got = out[int(qoff[b]) + torch.from_numpy(rows).to(DEV), h].double().cpu().numpy()
        errs.append(np.abs(got - ref))
    err = np.concatenate([e.ravel() for e in errs])
    assert err.max() <= MAX_ABS, f"max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean():.3e}"
    return float(err.max()), float(err.mean())


@pytest.mark.parametrize("name", ["single", "varlen", "chunked"])
def test_full_size_workload_sampled(name):
    _say(f"[gpu] full-size workload {name}")
    t, qs, ks, params = synth.workload_inputs(name, device=DEV)
    out = run_gpu(t, qs, ks, params)
    assert torch.isfinite(out).all()
    sampled_oracle_check(t, qs, ks, params, out, n_heads_sample=12, rows_per_head=24, seed=100)
    again = run_gpu(t, qs, ks, params)
    assert torch.equal(out, again)


def test_full_size_chunked_mask_free_sampled():
    _say("[gpu] full-size chunked, MASK_FREE with causal fp16 tile")
    t, qs, ks, params = synth.workload_inputs("chunked", device=DEV)
    tile = synth.causal_mask_tile(torch.float16, DEV)
    out = run_gpu(t, qs, ks, params, mask=tile, mask_type=synth.MASK_FREE)
    causal = run_gpu(t, qs, ks, params)
    assert torch.equal(out, causal)

    def boundary_rows(b):
        # rows whose key position is at 0, 1 or 511 modulo 512
        p0 = int(ks[b]) - int(qs[b])
        return [r for r in range(int(qs[b])) if (p0 + r) % 512 in (0, 1, 511)][:12]

    sampled_oracle_check(t, qs, ks, params, out, n_heads_sample=6, rows_per_head=8, seed=101, mask=tile,
                         mask_type=synth.MASK_FREE, extra_rows=boundary_rows)
