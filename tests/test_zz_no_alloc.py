"""mla_prefill_no_alloc, the entry point that keeps its work list in the
library's fixed per-GPU array, against mla_prefill with a workspace from the
caller. Both run the same kernels; where mla_prefill runs every item whole the
plans are the same and the outputs must agree bit for bit, and where it
splits long items over runs of keys (little work for the compute units) they
must agree to the attention parity bar (max abs 2e-2, mean abs 2e-3). Each
pair of no-alloc calls runs back to back on one stream with no
synchronisation between them, the second on a smaller problem, so a work
list left behind by the first call, or a copy that overtakes the first
call's kernel, would show in the second result."""
import numpy as np
import pytest
import torch

import mla_varlen_prefill_amd as mla
from mla_varlen_prefill_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def case(qs, ks, heads, kv_heads, dtype, seed, mask_type, mask=None, d=128, padded=0):
    qs, ks = np.asarray(qs, np.int32), np.asarray(ks, np.int32)
    t = synth.attention_inputs(qs, ks, heads, kv_heads, dtype, 1.0, seed, DEV, d_nope=d, kv_padded_max_seq=padded)
    out = torch.full((int(qs.sum()), heads, d), float("nan"), dtype=dtype, device=DEV)
    return dict(q=t["q"], q_rope=t["q_rope"], k=t["k"], k_rope=t["k_rope"], v=t["v"], q_seqlen=qs, kv_seqlen=ks,
                mask=mask, head_num=heads, qk_scale=synth.QK_SCALE, kv_head_num=kv_heads, mask_type=mask_type,
                cache_mode=0, atten_out=out)


def with_workspace(a):
    """The same problem through mla_prefill with a workspace of its own."""
    b = dict(a, atten_out=torch.full_like(a["atten_out"], float("nan")))
    size = mla.mla_prefill_get_workspace_size(**b)
    ws = torch.empty(max(size, 1), dtype=torch.uint8, device=DEV)
    mla.mla_prefill(**b, workspace=ws)
    torch.cuda.synchronize()
    return b["atten_out"]


def splits(a):
    """Does mla_prefill cut any item of this problem into runs of keys?"""
    _, items, tasks = mla.mla_prefill_plan_host(a["q_seqlen"], a["kv_seqlen"], a["head_num"], a["kv_head_num"],
                                                a["mask_type"])
    real = tasks[tasks[:, 0] >= 0]
    return bool(((real[:, 2] != 0) | (real[:, 3] != items[real[:, 0], 2])).any())


def run_pair(big, small):
    stream = torch.cuda.current_stream()
    mla.mla_prefill_no_alloc(**big, stream=stream)
    mla.mla_prefill_no_alloc(**small, stream=stream)
    torch.cuda.synchronize()
    for name, a in (("first (larger)", big), ("second (smaller)", small)):
        want = with_workspace(a)
        got = a["atten_out"]
        assert torch.isfinite(want).all() and torch.isfinite(got).all(), name
        if splits(a):
            err = (got.float() - want.float()).abs()
            assert err.max().item() <= 2e-2 and err.mean().item() <= 2e-3, f"{name}: {err.max().item()}"
        else:
            assert torch.equal(got, want), f"{name} call differs from mla_prefill"


def test_no_alloc_varlen_then_tiny():
    # The varlen workload (16 sequences of 128..8192 rows, 128 heads, fp16),
    # then the tiny one (2 sequences, 4 heads, bf16).
    _say("[gpu] no-alloc: varlen workload, then tiny")
    vq, vk = synth.workload_seqlens("varlen")
    big = case(vq, vk, 128, 128, torch.float16, 2, synth.MASK_CAUSAL)
    tq, tk = synth.workload_seqlens("tiny")
    small = case(tq, tk, 4, 4, torch.bfloat16, 0, synth.MASK_CAUSAL)
    run_pair(big, small)


def test_no_alloc_grouped_mask_free_padded_then_head_dim_64():
    # Grouped heads (16 over 2), a MASK_FREE tile, padded K/V (a problem that
    # mla_prefill splits); then a smaller causal problem with embeddimV 64
    # whose launch has fewer workgroups.
    _say("[gpu] no-alloc: grouped MASK_FREE padded, then head-dim 64")
    tile = synth.random_mask_tile(5, torch.bfloat16, DEV)
    big = case([700, 1500], [3000, 2100], 16, 2, torch.bfloat16, 7, synth.MASK_FREE, mask=tile, padded=3072)
    small = case([33, 1], [33, 90], 8, 8, torch.float16, 8, synth.MASK_CAUSAL, d=64)
    assert splits(big) and not splits(small)
    run_pair(big, small)


def test_no_alloc_full_single_workload_twice():
    # The single workload (4096 rows, 128 heads) twice, the second call with
    # its first 1000 rows and keys only.
    _say("[gpu] no-alloc: single workload, then its first 1000 rows")
    big = case([4096], [4096], 128, 128, torch.bfloat16, 1, synth.MASK_CAUSAL)
    small = case([1000], [1000], 128, 128, torch.bfloat16, 1, synth.MASK_CAUSAL)
    run_pair(big, small)
