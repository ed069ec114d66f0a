"""GPU parity of fused paged attention over a seeded sweep: each case draws
a batch (ragged, empty, query shorter or longer than its keys), a head
layout, a block size (64, 128, 192, 256), a mask type (MASK_FREE with a
random tile), a dtype, embeddimV 64 or 128 and a scale; the caches hold each
sequence's keys behind a seeded permuted block table with NaN in every
unused slot. mla_prefill_paged is compared with the fp64 oracle (gather by
definition, then attention) to the attention bar, and with gather +
mla_prefill bit for bit (both plan the same items, split the same way).
Case n is drawn from numpy's default_rng(2000 + n).
"""
import numpy as np
import pytest
import torch

from mla_varlen_prefill_amd import synth

from test_gpu_paged import make_paged, to_dev, run_paged, run_two_step, oracle_paged, assert_close

pytestmark = pytest.mark.gpu

N_CASES = 32
MAX_PAIRS = 3_000_000


def draw(n):
    rng = np.random.default_rng(2000 + n)
    while True:
        batch = int(rng.integers(1, 5))
        ks = [int(rng.choice([rng.integers(0, 200), rng.integers(200, 1500), rng.integers(1500, 4000)]))
              for _ in range(batch)]
        kind = rng.choice(["self", "suffix", "longer"])
        if kind == "self":
            qs = list(ks)
        elif kind == "suffix":
            qs = [int(rng.integers(0, k + 1)) for k in ks]
        else:
            qs = [k + int(rng.integers(1, 150)) for k in ks]
        kv_heads = int(rng.choice([1, 2, 3]))
        heads = kv_heads * int(rng.choice([1, 2, 4]))
        if sum(qs) == 0 or sum(q * k for q, k in zip(qs, ks)) * heads > MAX_PAIRS:
            continue
        return dict(qs=qs, ks=ks, heads=heads, kv_heads=kv_heads, block=int(rng.choice([64, 128, 192, 256])),
                    mask=int(rng.choice([synth.MASK_UNDEFINED, synth.MASK_SPEC, synth.MASK_CAUSAL,
                                         synth.MASK_FREE])),
                    dtype=rng.choice(["bf16", "fp16"]), d=int(rng.choice([64, 128])),
                    scale=float(rng.choice([synth.QK_SCALE, 1.0, -0.3])), seed=int(rng.integers(0, 1 << 20)))


@pytest.mark.parametrize("n", range(N_CASES), ids=[f"case-{n:02d}" for n in range(N_CASES)])
def test_random_paged_problem(n):
    c = draw(n)
    print(f"[gpu] paged sweep case {n}: {c}", flush=True)
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float16
    t, qs, ks = make_paged(c["qs"], c["ks"], c["heads"], c["kv_heads"], c["block"], dt, seed=c["seed"], dim=c["d"])
    tile = None
    if c["mask"] == synth.MASK_FREE:
        tile = synth.random_mask_tile(c["seed"], dt, "cpu")
    td = to_dev(t)
    tile_d = tile.to("cuda") if tile is not None else None
    out = run_paged(td, qs, ks, c["heads"], c["kv_heads"], c["mask"], tile_d, c["scale"])
    assert_close(out, oracle_paged(t, qs, ks, c["heads"], c["kv_heads"], c["mask"], tile, c["scale"]), f"case {n}")
    two = run_two_step(td, qs, ks, c["heads"], c["kv_heads"], c["mask"], tile_d, c["scale"])
    assert torch.equal(out, two), f"case {n}: fused differs from gather + prefill"
