"""MASK_FREE with the tile's 64-key row blocks classified (all 0, all -inf,
or mixed): a wave whose rows lie in one 512-key block takes the unmasked
path for a leading run of all-zero tiles of that block and skips the tiles
past its last live one. Results must equal, bit for bit, those of
mla_prefill_no_alloc, which runs without the classes (every diagonal-block
tile through the per-element path), and the fp64 oracle to the attention
bar. Tiles here are built from blocks of each class in patterns a causal
tile never has: zero blocks after a mixed one, dead blocks between live
ones, rows with every block dead. Sequences stay at most 1024 keys, so
neither call splits an item (mla_prefill_no_alloc never does) and the two
run the same tasks.
"""
import numpy as np
import pytest
import torch

import mla_varlen_prefill_amd as mla
from mla_varlen_prefill_amd import synth
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def block_tile(seed, dtype):
    """512 x 512 tile: block (row, k) of 64 entries is 0, -inf, or random
    (N(0, 4) with 20% -inf), by a seeded draw per (32-row group, k) with a
    few rows overridden, so both wave-uniform and per-row patterns occur."""
    rng = np.random.default_rng(seed)
    t = np.zeros((512, 512), np.float32)
    kinds = rng.choice(3, size=(16, 8), p=[0.45, 0.3, 0.25])
    for g in range(16):
        for k in range(8):
            rows, cols = slice(32 * g, 32 * g + 32), slice(64 * k, 64 * k + 64)
            if kinds[g, k] == 1:
                t[rows, cols] = -np.inf
            elif kinds[g, k] == 2:
                v = rng.normal(0.0, 2.0, (32, 64)).astype(np.float32)
                v[rng.random((32, 64)) < 0.2] = -np.inf
                t[rows, cols] = v
    t[rng.choice(512, 12, replace=False)] = -np.inf  # rows that see no key of their diagonal block
    t[5, 64:128] = 1.5                              # one row's block breaks its group's zero run
    return torch.from_numpy(t).to(dtype).to(DEV)


def run_pair(t, qs, ks, h, hk, tile, scale):
    a = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, h, hk, scale, synth.MASK_FREE, tile)
    b = torch.full_like(a, float("nan"))
    mla.mla_prefill_no_alloc(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, tile, h, scale, hk,
                             synth.MASK_FREE, 0, b)
    torch.cuda.synchronize()
    return a, b


CASES = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, dtype, tile dtype, scale
    ("self-bf16", [700, 1024, 90], [700, 1024, 90], 2, 2, torch.bfloat16, torch.bfloat16, synth.QK_SCALE),
    ("suffix-fp16-grouped", [300, 530], [1000, 530], 8, 2, torch.float16, torch.float16, synth.QK_SCALE),
    ("offset-rows-scale1", [333], [1000], 2, 1, torch.bfloat16, torch.float16, 1.0),
]


def splits(qs, ks, h, hk, mt):
    _, items, tasks = mla.mla_prefill_plan_host(qs, ks, h, hk, mt)
    real = tasks[tasks[:, 0] >= 0]
    return bool(((real[:, 2] != 0) | (real[:, 3] != items[real[:, 0], 2])).any())


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_classified_mask_free_tile(case):
    name, qs, ks, h, hk, dt, tdt, scale = case
    print(f"[gpu] mask classes {name}", flush=True)
    assert not splits(qs, ks, h, hk, synth.MASK_FREE)
    t = synth.attention_inputs(qs, ks, h, hk, dt, 1.0, len(name) + 300, DEV)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    tile = block_tile(len(name), tdt)
    a, b = run_pair(t, qs, ks, h, hk, tile, scale)
    assert torch.equal(a, b), f"{name}: classified run differs from the per-element run"
    f = {k: x.double().cpu().numpy() for k, x in t.items()}
    want = oracle.attention(f["q"], f["q_rope"], f["k"], f["k_rope"], f["v"], qs, ks, h, hk, scale,
                            synth.MASK_FREE, tile.double().cpu().numpy())
    g = a.double().cpu().numpy()
    assert np.isfinite(g).all()
    err = np.abs(g - want)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, f"{name}: max {err.max():.3e} mean {err.mean():.3e}"


def test_causal_tile_runs_the_causal_counts():
    # with the causal tile the classified MASK_FREE run equals the
    # per-element run and CAUSAL bit for bit (no split at these lengths)
    qs, ks = [1000, 300], [1000, 900]
    print("[gpu] mask classes: causal tile vs CAUSAL, 2 heads", flush=True)
    assert not splits(qs, ks, 2, 2, synth.MASK_FREE) and not splits(qs, ks, 2, 2, synth.MASK_CAUSAL)
    t = synth.attention_inputs(qs, ks, 2, 2, torch.bfloat16, 1.0, 301, DEV)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    tile = synth.causal_mask_tile(torch.float16, DEV)
    a, b = run_pair(t, qs, ks, 2, 2, tile, synth.QK_SCALE)
    assert torch.equal(a, b)
    c = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, 2, 2, synth.QK_SCALE,
                    synth.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(a, c)
