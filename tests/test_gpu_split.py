"""GPU parity of split items. When a launch holds little work for the GPU's
compute units (few heads, few sequences), mla_prefill cuts items longer than
an even share of the work into runs of key tiles, each run a workgroup of its
own that writes its rows over its own keys in fp32 with their log-sum-exp,
and a merge kernel combines the runs of each row. Every case here is checked
to be planned with splits (mla_prefill_plan_host) and compared with the fp64
oracle to the attention bar (max abs 2e-2, mean abs 2e-3); the
allocation-free entry point, which runs every item whole, gives the unsplit
result of the same inputs for a second comparison at that bar.
"""
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


def split_tasks(qs, ks, h, hk, mt):
    """Workgroups of the launch that hold part of an item's key tiles."""
    _, items, tasks = mla.mla_prefill_plan_host(qs, ks, h, hk, mt)
    real = tasks[tasks[:, 0] >= 0]
    return int(((real[:, 2] != 0) | (real[:, 3] != items[real[:, 0], 2])).sum())


def check(got, want, what):
    g = got.double().cpu().numpy() if isinstance(got, torch.Tensor) else got
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - want)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, f"{what}: max {err.max():.3e} mean {err.mean():.3e}"


def unsplit(t, qs, ks, h, hk, scale, mt, tile):
    """The same problem through the allocation-free entry point, which runs
    every item whole (packed K/V [sum kv, Hkv, D])."""
    out = torch.full((t["q"].shape[0], h, t["v"].shape[-1]), float("nan"), dtype=t["q"].dtype, device=DEV)
    mla.mla_prefill_no_alloc(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, tile, h, scale, hk, mt, 0,
                             out)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, dtype, mask_type, head dim, qkScale
    ("causal-2048", [2048], [2048], 2, 2, torch.bfloat16, synth.MASK_CAUSAL, 128, synth.QK_SCALE),
    ("causal-ragged", [1500, 37], [1700, 37], 2, 2, torch.bfloat16, synth.MASK_CAUSAL, 128, synth.QK_SCALE),
    ("q-longer-than-kv", [2000], [1500], 2, 2, torch.float16, synth.MASK_CAUSAL, 128, synth.QK_SCALE),
    ("undefined-fp16", [300, 100], [3000, 2000], 4, 4, torch.float16, synth.MASK_UNDEFINED, 128, synth.QK_SCALE),
    ("spec-8-over-1", [700], [3000], 8, 1, torch.bfloat16, synth.MASK_SPEC, 128, synth.QK_SCALE),
    ("head-dim-64", [1000], [2500], 2, 2, torch.bfloat16, synth.MASK_CAUSAL, 64, synth.QK_SCALE),
    ("scale-one", [1300], [1300], 2, 2, torch.bfloat16, synth.MASK_CAUSAL, 128, 1.0),
    ("negative-scale-fp16", [1300], [1300], 2, 2, torch.float16, synth.MASK_CAUSAL, 128, -0.1),
    ("group-8-over-2", [1200], [2000], 8, 2, torch.bfloat16, synth.MASK_CAUSAL, 128,
     synth.QK_SCALE),
    ("group-16-over-4-fp16", [900], [2400], 16, 4, torch.float16, synth.MASK_CAUSAL, 128, synth.QK_SCALE),
    ("group-2-undefined-d64", [700, 300], [2500, 1300], 6, 3, torch.bfloat16, synth.MASK_UNDEFINED, 64,
     synth.QK_SCALE),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle_and_unsplit(case):
    name, qs, ks, h, hk, dt, mt, d, scale = case
    n = split_tasks(qs, ks, h, hk, mt)
    _say(f"[gpu] split {name}: q={qs} kv={ks} H={h} Hkv={hk} {dt} mask={mt} D={d} scale={scale}: {n} split tasks")
    assert n > 0
    t = synth.attention_inputs(qs, ks, h, hk, dt, 1.0, len(name) + 100, DEV, d_nope=d)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, h, hk, scale, mt)
    torch.cuda.synchronize()
    f = {k: x.double().cpu().numpy() for k, x in t.items()}
    want = oracle.attention(f["q"], f["q_rope"], f["k"], f["k_rope"], f["v"], qs, ks, h, hk, scale, mt, None)
    check(out, want, name)
    check(unsplit(t, qs, ks, h, hk, scale, mt, None), want, name + " unsplit")
    if name == "q-longer-than-kv":
        assert (out[:500] == 0).all() and out[500:].abs().sum() > 0  # rows before the first key see nothing


MF_CASES = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, data dtype, tile dtype, head dim
    ("bf16-tile", [900, 400], [2600, 1500], 2, 2, torch.bfloat16, torch.bfloat16, 128),
    ("fp16-tile", [900, 400], [2600, 1500], 2, 2, torch.bfloat16, torch.float16, 128),
    ("fp16-data-d64-grouped", [1500, 200], [2600, 900], 4, 2, torch.float16, torch.float16, 64),
]


@pytest.mark.parametrize("case", MF_CASES, ids=[c[0] for c in MF_CASES])
def test_split_mask_free_random_tile(case):
    # runs are cut at multiples of 512 keys, so each run's 512-key blocks are
    # those of the tile
    name, qs, ks, h, hk, dt, tdt, d = case
    n = split_tasks(qs, ks, h, hk, synth.MASK_FREE)
    _say(f"[gpu] split MASK_FREE random tile {name}: {n} split tasks")
    assert n > 0
    _, items, tasks = mla.mla_prefill_plan_host(qs, ks, h, hk, synth.MASK_FREE)
    assert (tasks[:, 2] % 8 == 0).all()
    t = synth.attention_inputs(qs, ks, h, hk, dt, 1.0, 120, DEV, d_nope=d)
    tile = synth.random_mask_tile(121, tdt, DEV)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, h, hk, synth.QK_SCALE,
                      synth.MASK_FREE, tile)
    torch.cuda.synchronize()
    f = {k: x.double().cpu().numpy() for k, x in t.items()}
    want = oracle.attention(f["q"], f["q_rope"], f["k"], f["k_rope"], f["v"], qs, ks, h, hk, synth.QK_SCALE,
                            synth.MASK_FREE, tile.double().cpu().numpy())
    check(out, want, f"mask-free split {name}")
    check(unsplit(t, qs, ks, h, hk, synth.QK_SCALE, synth.MASK_FREE, tile), want, f"mask-free unsplit {name}")


def test_split_padded_kv_layout():
    # padded K/V [batch, max_seq, Hkv * D]: a run's first key row is its
    # sequence's row b * max_seq plus the run's first key
    qs, ks = [1200, 300], [2100, 1800]
    n = split_tasks(qs, ks, 2, 1, synth.MASK_CAUSAL)
    _say(f"[gpu] split padded K/V: {n} split tasks")
    assert n > 0
    t = synth.attention_inputs(qs, ks, 2, 1, torch.bfloat16, 1.0, 122, DEV, kv_padded_max_seq=2200)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, 2, 1, synth.QK_SCALE,
                      synth.MASK_CAUSAL)
    torch.cuda.synchronize()
    f = {k: x.double().cpu().numpy() for k, x in t.items()}
    for k in ("k", "k_rope", "v"):
        f[k] = f[k].reshape(2, 2200, 1, -1)
    want = oracle.attention(f["q"], f["q_rope"], f["k"], f["k_rope"], f["v"], qs, ks, 2, 1, synth.QK_SCALE,
                            synth.MASK_CAUSAL, None, kv_padded=True)
    check(out, want, "padded split")


def test_split_full_single_shape_16_heads_sampled():
    # The 4096-token causal shape at 16 heads (one GPU's share of an 8-way
    # split over heads): items of 40..64 tiles are cut in two. Rows are
    # sampled from every item, head by head, plus the first and last rows.
    H, n = 16, 4096
    assert split_tasks([n], [n], H, H, synth.MASK_CAUSAL) == 224
    _say("[gpu] split full size: 4096 causal, 16 heads")
    t = synth.attention_inputs([n], [n], H, H, torch.bfloat16, 1.0, 123, DEV)
    qs = np.array([n], np.int32)
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, qs, H, H, synth.QK_SCALE,
                      synth.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    got = out.double().cpu().numpy()
    f = lambda x: x.double().cpu().numpy()
    rng = np.random.default_rng(124)
    errs = []
    for h in range(H):
        rows = np.array(sorted({0, n - 1} | {int(256 * it + rng.integers(0, 256)) for it in range(16)}), np.int64)
        want = oracle.attention_head(f(t["q"][:, h]), f(t["q_rope"][:, h]), f(t["k"][:, h]), f(t["k_rope"][:, h]),
                                     f(t["v"][:, h]), synth.QK_SCALE, synth.MASK_CAUSAL, rows=rows)
        errs.append(np.abs(got[rows, h] - want))
    e = np.concatenate(errs)
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS, f"max {e.max():.3e} mean {e.mean():.3e}"


def test_split_run_is_deterministic():
    qs = np.array([2048], np.int32)
    t = synth.attention_inputs([2048], [2048], 2, 2, torch.bfloat16, 1.0, 125, DEV)
    a = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, qs, 2, 2, synth.QK_SCALE,
                    synth.MASK_CAUSAL)
    b = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, qs, 2, 2, synth.QK_SCALE,
                    synth.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
