"""GPU parity at the library's size limits (through the C ABI).

  * fused paged attention with one sequence of exactly PAGED_MAX_KEYS keys
    (the most the kernel's LDS tile table addresses), 64 queries at its end,
    causal, sampled rows against the oracle's host gather + attention;
  * contiguous attention over a 65536-key sequence (256 queries at the end,
    causal and UNDEFINED), sampled rows against the oracle;
  * the paged gather with the largest batch the kernel's LDS offset table
    holds (GATHER_MAX_BATCH sequences), every row bit for bit;
  * 5000 sequences of 0 to 3 tokens: the planner's many small items, every
    element against the oracle.
One past each limit is rejected on the host (tests/test_abi_cpu.py).
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
GATHER_MAX_BATCH = 8192


def _say(msg):
    print(msg, flush=True)


def _check(err):
    err = np.concatenate([e.ravel() for e in err])
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


def test_paged_attention_at_max_keys():
    n, ql, bs = mla.PAGED_MAX_KEYS, 64, 128
    _say(f"[gpu] fused paged attention, {n} keys (limit), {ql} queries")
    c = synth.paged_inputs([n], heads=1, block_size=bs, seed=91, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(92)
    q = torch.randn((ql, 1, 128), generator=g, device=DEV).to(torch.bfloat16)
    qr = torch.randn((ql, 1, 64), generator=g, device=DEV).to(torch.bfloat16)
    qs, ks = np.array([ql], np.int32), np.array([n], np.int32)
    out = mla.prefill_paged(q, qr, c["key_cache"], c["rope_cache"], c["value_cache"], c["block_tables"], qs, ks,
                            1, 1, synth.QK_SCALE, synth.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    table = c["block_tables"].cpu().numpy()
    f = lambda x: x.double().cpu().numpy()
    k, _ = oracle.paged_cache_load(f(c["key_cache"]), None, table, ks)
    kr, _ = oracle.paged_cache_load(f(c["rope_cache"]), None, table, ks)
    v, _ = oracle.paged_cache_load(f(c["value_cache"]), None, table, ks)
    rows = np.array([0, 1, 17, 31, 32, 62, 63], np.int64)
    ref = oracle.attention_head(f(q)[:, 0], f(qr)[:, 0], k[:, 0], kr[:, 0], v[:, 0], synth.QK_SCALE,
                                synth.MASK_CAUSAL, rows=rows)
    _check([np.abs(f(out)[rows, 0] - ref)])


@pytest.mark.parametrize("mask_type", [synth.MASK_CAUSAL, synth.MASK_UNDEFINED])
def test_contiguous_attention_long_sequence(mask_type):
    n, ql = 65536, 256
    _say(f"[gpu] contiguous attention, {n} keys, {ql} queries, mask {mask_type}")
    t = synth.attention_inputs([ql], [n], 2, 1, torch.bfloat16, 1.0, 93, DEV)
    qs, ks = np.array([ql], np.int32), np.array([n], np.int32)
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, 2, 1, synth.QK_SCALE, mask_type)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    f = lambda x: x.double().cpu().numpy()
    rows = np.array([0, 1, 100, 254, 255], np.int64)
    errs = []
    for h in range(2):
        ref = oracle.attention_head(f(t["q"][:, h]), f(t["q_rope"][:, h]), f(t["k"][:, 0]), f(t["k_rope"][:, 0]),
                                    f(t["v"][:, 0]), synth.QK_SCALE, mask_type, rows=rows)
        errs.append(np.abs(f(out)[rows, h] - ref))
    _check(errs)


def test_gather_at_max_batch():
    rng = np.random.default_rng(94)
    lens = rng.integers(0, 40, size=GATHER_MAX_BATCH).astype(np.int32)
    _say(f"[gpu] paged gather, batch {GATHER_MAX_BATCH} (limit), {int(lens.sum())} tokens")
    c = synth.paged_inputs(lens, heads=2, head_size_k=16, head_size_v=16, block_size=16, seed=95, device=DEV,
                           with_rope=False)
    total = int(lens.sum())
    key = torch.empty((total, 2, 16), dtype=torch.bfloat16, device=DEV)
    value = torch.empty_like(key)
    mla.paged_cache_load(c["key_cache"], c["value_cache"], c["block_tables"], c["context_lens"], key, value)
    torch.cuda.synchronize()
    rk, rv = oracle.paged_cache_load(c["key_cache"].view(torch.int16).cpu().numpy(),
                                     c["value_cache"].view(torch.int16).cpu().numpy(),
                                     c["block_tables"].cpu().numpy(), lens)
    assert np.array_equal(key.view(torch.int16).cpu().numpy(), rk)
    assert np.array_equal(value.view(torch.int16).cpu().numpy(), rv)


def test_many_tiny_sequences():
    rng = np.random.default_rng(96)
    qs = rng.integers(0, 4, size=5000).astype(np.int32)
    ks = qs + rng.integers(0, 3, size=5000).astype(np.int32)
    _say(f"[gpu] 5000 sequences of 0..3 queries, {int(qs.sum())} query rows")
    t = synth.attention_inputs(qs, ks, 2, 2, torch.bfloat16, 1.0, 97, DEV)
    out = mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], qs, ks, 2, 2, synth.QK_SCALE,
                      synth.MASK_CAUSAL)
    torch.cuda.synchronize()
    d = {n: x.double().cpu().numpy() for n, x in t.items()}
    ref = oracle.attention(d["q"], d["q_rope"], d["k"], d["k_rope"], d["v"], qs, ks, 2, 2, synth.QK_SCALE,
                           synth.MASK_CAUSAL)
    _check([np.abs(out.double().cpu().numpy() - ref)])
