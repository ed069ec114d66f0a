"""GPU parity of the MLA prolog over a seeded sweep: each case draws the
token count, h (a multiple of 128, so that the first product's split over K
takes every divisor structure), q_lora_rank, the head count and whether the
weights are packed once, and compares mla_prolog (or mla_prolog_prepacked)
with the fp64 oracle to the prolog tolerance, and the prepacked outputs with
the packing call's bit for bit. Case n is drawn from numpy's
default_rng(3000 + n).
"""
import numpy as np
import pytest
import torch

import mla_varlen_prefill_amd as mla
from mla_varlen_prefill_amd import synth

from test_gpu_prolog import run_gpu, run_oracle, assert_close

pytestmark = pytest.mark.gpu

N_CASES = 16


def draw(n):
    rng = np.random.default_rng(3000 + n)
    return dict(t=int(rng.choice([rng.integers(1, 40), rng.integers(40, 400), rng.integers(400, 1500)])),
                h=128 * int(rng.choice([1, 2, 3, 5, 8, 9, 12, 32])), q_lora_rank=512 * int(rng.integers(1, 4)),
                num_heads=int(rng.integers(1, 9)), seed=int(rng.integers(0, 1 << 20)))


@pytest.mark.parametrize("n", range(N_CASES), ids=[f"case-{n:02d}" for n in range(N_CASES)])
def test_random_prolog_problem(n):
    c = draw(n)
    print(f"[gpu] prolog sweep case {n}: {c}", flush=True)
    d = synth.prolog_inputs(c["t"], h=c["h"], q_lora_rank=c["q_lora_rank"], num_heads=c["num_heads"],
                            seed=c["seed"] % 1000, device="cuda")
    q, kv, cq = run_gpu(d)
    rq, rkv, rcq = run_oracle(d)
    assert_close(q, rq, f"case {n} q")
    assert_close(kv, rkv, f"case {n} kv")
    assert_close(cq, rcq, f"case {n} c^Q")
    packed = mla.pack_prolog_weights(d["wq_a"], d["wq_b"], d["wkv"])
    pp = mla.prolog(d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"], d["gamma_cq"],
                    d["gamma_ckv"], synth.PROLOG_EPS, packed=packed)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "kv", "cq"), (q, kv, cq), pp):
        assert torch.equal(a, b), f"case {n}: prepacked {name} differs"
