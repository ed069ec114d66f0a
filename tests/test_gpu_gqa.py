"""GPU parity of grouped-query attention (headNum > kvHeadNum) through the C ABI.

When several query heads share a KV head, one workgroup runs rows of up to
8 of them against the same K/V tiles in LDS (the planner's heads per task).
Checks:
  * against the fp64 oracle, every element, for group sizes that give 8, 4,
    2 and 1 heads per workgroup, MQA, ragged and empty sequences, queries
    longer and shorter than keys, each mask type, fp16 and bf16, and a
    negative scale;
  * bit-exact against the same inputs with K/V repeated per query head and
    run as plain multi-head attention (one head per workgroup): each query
    row sees the same key tiles in the same order either way;
  * a full-size grouped workload (4096-token causal, 128 query heads over 16
    and over 1 KV heads) on sampled rows.
Tolerances as in test_gpu_parity: max |gpu - oracle| <= 2e-2, mean <= 2e-3.
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


def run(t, qs, ks, heads, kv_heads, mask_type, mask=None, scale=synth.QK_SCALE):
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, heads, kv_heads, scale,
                      mask_type, mask)
    torch.cuda.synchronize()
    return out


def expand_kv(t, heads, kv_heads):
    """K, KRope and V repeated so that query head h has its own copy of kv
    head h // (heads / kv_heads)."""
    g = heads // kv_heads
    e = dict(t)
    for n in ("k", "k_rope", "v"):
        e[n] = t[n].repeat_interleave(g, dim=1).contiguous()
    return e


def oracle_out(t, qs, ks, heads, kv_heads, mask_type, mask=None, scale=synth.QK_SCALE):
    d = {n: x.double().cpu().numpy() for n, x in t.items()}
    tile = mask.double().cpu().numpy() if mask is not None else None
    return oracle.attention(d["q"], d["q_rope"], d["k"], d["k_rope"], d["v"], qs, ks, heads, kv_heads, scale,
                            mask_type, tile)


def assert_close(gpu, ref, what):
    g = gpu.double().cpu().numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    assert err.max() <= MAX_ABS, f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean abs err {err.mean():.3e}"


CASES = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, dtype, mask_type  (heads per workgroup)
    ("g8-causal", [1, 31, 32, 33, 65, 300], [1, 31, 32, 33, 65, 300], 16, 2, torch.bfloat16,
     synth.MASK_CAUSAL),  # 8
    ("mqa16-chunked", [100, 33], [700, 260], 16, 1, torch.bfloat16, synth.MASK_CAUSAL),  # 8
    ("g4-undefined-fp16", [5, 130, 257], [77, 130, 190], 8, 2, torch.float16, synth.MASK_UNDEFINED),  # 4
    ("g6-spec", [64, 200], [64, 200], 12, 2, torch.bfloat16, synth.MASK_SPEC),  # 2
    ("g3-causal", [150, 40], [150, 90], 12, 4, torch.bfloat16, synth.MASK_CAUSAL),  # 1
    ("g16-q-longer-than-kv", [200, 70], [50, 0], 32, 2, torch.bfloat16, synth.MASK_CAUSAL),  # 8
    ("g8-empty-and-single-query", [0, 1, 45, 1], [10, 1000, 45, 3], 8, 1, torch.float16,
     synth.MASK_SPEC),  # 8
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_matches_oracle_and_expanded_mha(case):
    name, qs, ks, h, hk, dt, mt = case
    _say(f"[gpu] gqa {name}: q={qs} kv={ks} H={h} Hkv={hk} {dt} mask={mt}")
    t = synth.attention_inputs(qs, ks, h, hk, dt, 1.0, len(name) + 40, DEV)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    out = run(t, qs, ks, h, hk, mt)
    assert_close(out, oracle_out(t, qs, ks, h, hk, mt), name)
    mha = run(expand_kv(t, h, hk), qs, ks, h, h, mt)
    assert torch.equal(out, mha), f"{name}: grouped run differs from the expanded multi-head run"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_grouped_mask_free_random_tile(dtype):
    qs, ks = [300, 530], [700, 530]
    _say(f"[gpu] gqa mask-free random tile {dtype}")
    t = synth.attention_inputs(qs, ks, 16, 4, dtype, 1.0, 61, DEV)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    tile = synth.random_mask_tile(9, dtype, DEV)
    out = run(t, qs, ks, 16, 4, synth.MASK_FREE, tile)
    assert_close(out, oracle_out(t, qs, ks, 16, 4, synth.MASK_FREE, tile), "gqa mask-free")
    assert torch.equal(out, run(expand_kv(t, 16, 4), qs, ks, 16, 16, synth.MASK_FREE, tile))


def test_grouped_negative_scale():
    # a negative scale is folded into Q (and Q-rope in LDS); with several heads
    # per workgroup every head's rows must be flipped exactly once
    qs = [90, 257]
    _say("[gpu] gqa negative scale")
    t = synth.attention_inputs(qs, qs, 8, 1, torch.bfloat16, 1.0, 62, DEV)
    qs = np.asarray(qs, np.int32)
    out = run(t, qs, qs, 8, 1, synth.MASK_CAUSAL, scale=-0.1)
    assert_close(out, oracle_out(t, qs, qs, 8, 1, synth.MASK_CAUSAL, scale=-0.1), "negative scale")


@pytest.mark.parametrize("kv_heads", [16, 1])
def test_grouped_full_size_single_sampled(kv_heads):
    # 4096-token causal prefill, 128 query heads over kv_heads KV heads, bf16
    H, n = 128, 4096
    _say(f"[gpu] gqa full size: 4096 causal, H=128, Hkv={kv_heads}")
    t = synth.attention_inputs([n], [n], H, kv_heads, torch.bfloat16, 1.0, 63, DEV)
    qs = np.array([n], np.int32)
    out = run(t, qs, qs, H, kv_heads, synth.MASK_CAUSAL)
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(64)
    g = H // kv_heads
    errs = []
    for k in range(6):
        h = int(rng.integers(0, H)) if k else H - 1
        hk = h // g
        rows = np.array(sorted(set(int(x) for x in rng.integers(0, n, size=24)) | {0, 1, 31, 32, n - 1}),
                        np.int64)
        ref = oracle.attention_head(t["q"][:, h].double().cpu().numpy(), t["q_rope"][:, h].double().cpu().numpy(),
                                    t["k"][:, hk].double().cpu().numpy(), t["k_rope"][:, hk].double().cpu().numpy(),
                                    t["v"][:, hk].double().cpu().numpy(), synth.QK_SCALE, synth.MASK_CAUSAL,
                                    rows=rows)
        got = out[torch.from_numpy(rows).to(DEV), h].double().cpu().numpy()
        errs.append(np.abs(got - ref).ravel())
    err = np.concatenate(errs)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
