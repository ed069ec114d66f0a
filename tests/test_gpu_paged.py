"""GPU parity of fused paged attention (``mla_prefill_paged``, through the C ABI).

Expected values come from the oracle's ``paged_attention``: the plain gather
of each cache followed by plain attention. Every cache block no sequence uses
holds NaN, so a tile read from the wrong block shows up as a non-finite
output. The fused result must also equal, bit for bit, the two-step path
(``paged_cache_load`` then ``mla_prefill``) on the same data: both run the
same arithmetic and differ only in where the key rows are read from.
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


def make_paged(qs, ks, heads, kv_heads, block_size, dtype=torch.bfloat16, seed=0, spare_blocks=3, dim=128):
    """Q/QRope plus ND caches holding each sequence's keys behind a seeded,
    permuted block table; unused blocks (and unused slots) are NaN."""
    rng = np.random.default_rng(seed)
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    cols = max(1, max(-(-int(k) // block_size) for k in ks))
    nb = len(ks) * cols + spare_blocks
    table = rng.permutation(nb)[:len(ks) * cols].reshape(len(ks), cols).astype(np.int32)
    g = torch.Generator(device="cpu").manual_seed(seed * 100 + 1)

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)

    caches = {}
    for name, d in (("key_cache", dim), ("krope_cache", 64), ("value_cache", dim)):
        c = torch.full((nb, block_size, kv_heads, d), float("nan"), dtype=dtype)
        for b, n in enumerate(ks):
            for t0 in range(0, int(n), block_size):
                m = min(block_size, int(n) - t0)
                c[table[b][t0 // block_size], :m] = randn(m, kv_heads, d)
        caches[name] = c
    q = randn(int(qs.sum()), heads, dim)
    qr = randn(int(qs.sum()), heads, 64)
    return dict(q=q, q_rope=qr, block_tables=torch.from_numpy(table), **caches), qs, ks


def to_dev(t):
    return {k: v.to(DEV) for k, v in t.items()}


def run_paged(td, qs, ks, heads, kv_heads, mask_type, mask=None, scale=synth.QK_SCALE):
    out = mla.prefill_paged(td["q"], td["q_rope"], td["key_cache"], td["krope_cache"], td["value_cache"],
                            td["block_tables"], qs, ks, heads, kv_heads, scale, mask_type, mask)
    torch.cuda.synchronize()
    return out


def run_two_step(td, qs, ks, heads, kv_heads, mask_type, mask=None, scale=synth.QK_SCALE):
    n = int(ks.sum())
    ctx = torch.from_numpy(ks).to(DEV)
    k = torch.empty((n, kv_heads, td["q"].shape[-1]), dtype=td["q"].dtype, device=DEV)
    v = torch.empty_like(k)
    kr = torch.empty((n, kv_heads, 64), dtype=td["q"].dtype, device=DEV)
    mla.paged_cache_load(td["key_cache"], td["value_cache"], td["block_tables"], ctx, k, v)
    mla.paged_cache_load(td["krope_cache"], None, td["block_tables"], ctx, kr, None)
    out = mla.prefill(td["q"], td["q_rope"], k, kr, v, qs, ks, heads, kv_heads, scale, mask_type, mask)
    torch.cuda.synchronize()
    return out


def oracle_paged(t, qs, ks, heads, kv_heads, mask_type, mask=None, scale=synth.QK_SCALE):
    f = lambda x: x.double().numpy()
    tile = mask.double().cpu().numpy() if mask is not None else None
    return oracle.paged_attention(f(t["q"]), f(t["q_rope"]), f(t["key_cache"]), f(t["krope_cache"]),
                                  f(t["value_cache"]), t["block_tables"].numpy(), qs, ks, heads, kv_heads, scale,
                                  mask_type, tile)


def assert_close(gpu, ref, what):
    g = gpu.double().cpu().numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    assert err.max() <= MAX_ABS, f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean abs err {err.mean():.3e}"


CASES = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, block_size, dtype, mask_type
    ("causal-bs64", [1, 63, 130, 300], [1, 63, 130, 300], 2, 2, 64, torch.bfloat16, synth.MASK_CAUSAL),
    ("chunked-gqa-bs128", [100, 33], [700, 260], 8, 2, 128, torch.bfloat16, synth.MASK_CAUSAL),
    ("undefined-fp16-bs192", [5, 130], [77, 190], 3, 3, 192, torch.float16, synth.MASK_UNDEFINED),
    ("empty-and-mqa-bs64", [0, 45, 3], [10, 45, 0], 2, 1, 64, torch.bfloat16, synth.MASK_CAUSAL),
    ("spec-bs256", [1, 200], [1000, 200], 4, 4, 256, torch.bfloat16, synth.MASK_SPEC),
]

# head dim 64 (embeddimV), and the page's default qkScale of 1.0 (scores of
# standard deviation near 14, so the running max moves often)
CASES_MORE = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, block_size, dtype, mask_type, head dim, scale
    ("causal-d64-bs64", [1, 63, 130, 300], [1, 63, 130, 300], 2, 2, 64, torch.bfloat16, synth.MASK_CAUSAL, 64,
     synth.QK_SCALE),
    ("gqa-d64-fp16-bs128", [100, 33], [700, 260], 8, 2, 128, torch.float16, synth.MASK_CAUSAL, 64, synth.QK_SCALE),
    ("causal-scale1-bs64", [70, 300], [70, 300], 2, 2, 64, torch.bfloat16, synth.MASK_CAUSAL, 128, 1.0),
    ("gqa-scale1-fp16-bs128", [100, 33], [700, 260], 8, 2, 128, torch.float16, synth.MASK_UNDEFINED, 128, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_matches_oracle_and_two_step(case):
    name, qs, ks, h, hk, bs, dtype, mt = case
    _say(f"[gpu] paged {name}")
    t, qs, ks = make_paged(qs, ks, h, hk, bs, dtype, seed=len(name))
    td = to_dev(t)
    out = run_paged(td, qs, ks, h, hk, mt)
    assert_close(out, oracle_paged(t, qs, ks, h, hk, mt), name)
    assert torch.equal(out, run_two_step(td, qs, ks, h, hk, mt)), f"{name}: fused differs from gather + prefill"


@pytest.mark.parametrize("case", CASES_MORE, ids=[c[0] for c in CASES_MORE])
def test_paged_head_dim_and_scale(case):
    name, qs, ks, h, hk, bs, dtype, mt, dim, scale = case
    _say(f"[gpu] paged {name}")
    t, qs, ks = make_paged(qs, ks, h, hk, bs, dtype, seed=len(name) + 50, dim=dim)
    td = to_dev(t)
    out = run_paged(td, qs, ks, h, hk, mt, scale=scale)
    assert_close(out, oracle_paged(t, qs, ks, h, hk, mt, scale=scale), name)
    assert torch.equal(out, run_two_step(td, qs, ks, h, hk, mt, scale=scale)), f"{name}: fused differs from gather + prefill"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_paged_mask_free_random_tile(dtype):
    _say(f"[gpu] paged MASK_FREE random tile {dtype}")
    t, qs, ks = make_paged([600, 70], [600, 900], 2, 2, 128, dtype, seed=11)
    tile = synth.random_mask_tile(5, torch.float16, "cpu")
    td = to_dev(t)
    out = run_paged(td, qs, ks, 2, 2, synth.MASK_FREE, tile.to(DEV))
    assert_close(out, oracle_paged(t, qs, ks, 2, 2, synth.MASK_FREE, tile), "mask-free")
    assert torch.equal(out, run_two_step(td, qs, ks, 2, 2, synth.MASK_FREE, tile.to(DEV)))


def test_paged_out_of_range_block_reads_zeros():
    # A block id outside [0, num_blocks) makes its 64-key tiles read as zero
    # rows (documented); sequences whose tables are valid are unaffected.
    _say("[gpu] paged out-of-range block id")
    t, qs, ks = make_paged([50, 80], [200, 300], 2, 2, 64, seed=5)
    good = run_paged(to_dev(t), qs, ks, 2, 2, synth.MASK_CAUSAL)
    bad = dict(t)
    bt = t["block_tables"].clone()
    bt[0, 1] = 10 ** 6
    bt[0, 2] = -3
    bad["block_tables"] = bt
    out = run_paged(to_dev(bad), qs, ks, 2, 2, synth.MASK_CAUSAL)
    assert torch.isfinite(out).all()
    assert torch.equal(out[50:], good[50:])


def test_paged_medium_workload_sampled():
    # 8 sequences of 1024..8192 keys, 16 heads (a tensor-parallel share of 128),
    # bf16, causal, block size 128; rows sampled per (sequence, head) and checked
    # against the oracle's gather + attention, head by head on the host.
    _say("[gpu] paged medium workload, sampled rows")
    rng = np.random.default_rng(21)
    ks = rng.integers(1024, 8193, size=8).astype(np.int32)
    qs = ks.copy()
    H = HK = 16
    bs = 128
    cols = int(-(-ks.max() // bs))
    nb = len(ks) * cols
    table = rng.permutation(nb).astype(np.int32).reshape(len(ks), cols)
    g = torch.Generator(device=DEV).manual_seed(2100)
    td = dict(
        q=torch.randn((int(qs.sum()), H, 128), generator=g, device=DEV).to(torch.bfloat16),
        q_rope=torch.randn((int(qs.sum()), H, 64), generator=g, device=DEV).to(torch.bfloat16),
        key_cache=torch.randn((nb, bs, HK, 128), generator=g, device=DEV).to(torch.bfloat16),
        krope_cache=torch.randn((nb, bs, HK, 64), generator=g, device=DEV).to(torch.bfloat16),
        value_cache=torch.randn((nb, bs, HK, 128), generator=g, device=DEV).to(torch.bfloat16),
        block_tables=torch.from_numpy(table).to(DEV))
    out = run_paged(td, qs, ks, H, HK, synth.MASK_CAUSAL)
    assert torch.isfinite(out).all()
    qoff = np.concatenate([[0], np.cumsum(qs)])
    errs = []
    for n in range(6):
        b, h = int(rng.integers(0, len(ks))), int(rng.integers(0, H))
        caches = {k: td[k][:, :, h].unsqueeze(2).double().cpu().numpy()
                  for k in ("key_cache", "krope_cache", "value_cache")}
        one = np.array([int(ks[b])], np.int32)
        kk, _ = oracle.paged_cache_load(caches["key_cache"], None, table[b:b + 1], one)
        kr, _ = oracle.paged_cache_load(caches["krope_cache"], None, table[b:b + 1], one)
        vv, _ = oracle.paged_cache_load(caches["value_cache"], None, table[b:b + 1], one)
        ql = int(qs[b])
        rows = np.array(sorted(set(int(x) for x in rng.integers(0, ql, size=16)) | {0, ql - 1}), np.int64)
        sl = slice(int(qoff[b]), int(qoff[b]) + ql)
        ref = oracle.attention_head(td["q"][sl, h].double().cpu().numpy(), td["q_rope"][sl, h].double().cpu().numpy(),
                                    kk[:, 0], kr[:, 0], vv[:, 0], synth.QK_SCALE, synth.MASK_CAUSAL, rows=rows)
        got = out[int(qoff[b]) + torch.from_numpy(rows).to(DEV), h].double().cpu().numpy()
        errs.append(np.abs(got - ref).ravel())
    err = np.concatenate(errs)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


def test_paged_full_workload_sampled_rows():
    """Fused paged attention on the full paged workload (32 sequences of 1024 ..
    32768 keys from the seeded lengths, 128 heads, block size 128, the seeded
    permuted block table, causal, bf16): seeded (sequence, head, row) samples
    plus each sequence's first and last row, against the oracle's gather and
    attention for that head (``oracle.paged_cache_load`` then
    ``oracle.attention_head``)."""
    lens, _ = synth.workload_seqlens("paged")
    total = int(lens.sum())
    _say(f"[gpu] fused paged attention, full paged workload, {total} tokens x 128 heads")
    c = synth.paged_inputs(lens, device=DEV, with_rope=True)
    H = c["key_cache"].shape[2]
    q = synth._randn((total, H, 128), torch.bfloat16, 1.0, 4 * 100 + 8, DEV)
    qr = synth._randn((total, H, 64), torch.bfloat16, 1.0, 4 * 100 + 9, DEV)
    qs = ks = np.asarray(lens, np.int32)
    td = dict(q=q, q_rope=qr, key_cache=c["key_cache"], krope_cache=c["rope_cache"], value_cache=c["value_cache"],
              block_tables=c["block_tables"])
    out = run_paged(td, qs, ks, H, H, synth.MASK_CAUSAL)
    table = c["block_tables"].cpu().numpy()
    qoff = np.concatenate([[0], np.cumsum(qs)])
    rng = np.random.default_rng(31)
    heads = sorted(set(int(x) for x in rng.integers(0, H, size=4)) | {0, H - 1})
    errs = []
    for h in heads:
        hc = {k: td[k][:, :, h].unsqueeze(2).contiguous().cpu().double().numpy()
              for k in ("key_cache", "krope_cache", "value_cache")}
        for b in sorted(set(int(x) for x in rng.integers(0, len(lens), size=6)) | {0, len(lens) - 1}):
            one = np.array([int(ks[b])], np.int32)
            kk, _ = oracle.paged_cache_load(hc["key_cache"], None, table[b:b + 1], one)
            kr, _ = oracle.paged_cache_load(hc["krope_cache"], None, table[b:b + 1], one)
            vv, _ = oracle.paged_cache_load(hc["value_cache"], None, table[b:b + 1], one)
            ql = int(qs[b])
            rows = np.array(sorted(set(int(x) for x in rng.integers(0, ql, size=24)) | {0, 1, ql - 1}), np.int64)
            sl = slice(int(qoff[b]), int(qoff[b]) + ql)
            ref = oracle.attention_head(q[sl, h].double().cpu().numpy(), qr[sl, h].double().cpu().numpy(), kk[:, 0],
                                        kr[:, 0], vv[:, 0], synth.QK_SCALE, synth.MASK_CAUSAL, rows=rows)
            got = out[int(qoff[b]) + torch.from_numpy(rows).to(DEV), h].double().cpu().numpy()
            errs.append(np.abs(got - ref).ravel())
        del hc
    err = np.concatenate(errs)
    _say(f"[gpu]   {len(err) // 128} rows compared, max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


SPLIT_CASES = [
    # name, q_seqlen, kv_seqlen, heads, kv_heads, block_size, dtype, mask_type, head dim
    ("causal-bs128", [3000], [3000], 2, 2, 128, torch.bfloat16, synth.MASK_CAUSAL, 128),
    ("q-longer-bs64", [2000], [1500], 2, 1, 64, torch.float16, synth.MASK_CAUSAL, 128),
    ("undefined-d64-bs192", [300, 100], [3000, 2000], 4, 2, 192, torch.bfloat16, synth.MASK_UNDEFINED, 64),
]


def _split_tasks(qs, ks, h, hk, mt):
    _, items, tasks = mla.mla_prefill_plan_host(qs, ks, h, hk, mt)
    real = tasks[tasks[:, 0] >= 0]
    return int(((real[:, 2] != 0) | (real[:, 3] != items[real[:, 0], 2])).sum())


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_paged_split_items(case):
    # few heads over long sequences: long items run as several key-tile runs
    # (the run's first tile sits above the sequence index in the launch
    # record); the result matches the oracle and gather + prefill bit for bit
    name, qs, ks, h, hk, bs, dtype, mt, dim = case
    n = _split_tasks(qs, ks, h, hk, mt)
    _say(f"[gpu] paged split {name}: {n} split tasks")
    assert n > 0
    t, qs, ks = make_paged(qs, ks, h, hk, bs, dtype, seed=len(name) + 70, dim=dim)
    td = to_dev(t)
    out = run_paged(td, qs, ks, h, hk, mt)
    assert_close(out, oracle_paged(t, qs, ks, h, hk, mt), name)
    assert torch.equal(out, run_two_step(td, qs, ks, h, hk, mt)), f"{name}: fused differs from gather + prefill"


def test_paged_mask_free_split_random_tile():
    qs, ks = [1500, 200], [2600, 900]
    assert _split_tasks(qs, ks, 4, 2, synth.MASK_FREE) > 0
    _say("[gpu] paged split MASK_FREE random tile")
    t, qs, ks = make_paged(qs, ks, 4, 2, 128, torch.bfloat16, seed=77)
    tile = synth.random_mask_tile(78, torch.float16)
    td = to_dev(t)
    out = run_paged(td, qs, ks, 4, 2, synth.MASK_FREE, tile.to(DEV))
    assert_close(out, oracle_paged(t, qs, ks, 4, 2, synth.MASK_FREE, tile), "mask-free split")
    assert torch.equal(out, run_two_step(td, qs, ks, 4, 2, synth.MASK_FREE, tile.to(DEV)))
