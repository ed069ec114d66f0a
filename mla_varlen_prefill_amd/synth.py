"""Seeded synthetic workloads for MLA varlen prefill and the paged gather.

This module only draws inputs: lengths, random tensors, block tables and mask
tiles. It holds none of the attention or gather arithmetic, so the CPU oracle
and the HIP path can both be fed from it without sharing any computation.

Workloads (shapes follow the Ascend Transformer Boost "MLA Prefill" and
"PagedCacheLoadOperation" pages' Members tables; the pages name no dataset,
so these synthetic inputs are the workload):

  tiny      batch 2, q = kv = {17, 40}, 4 heads, bf16 N(0, 1), causal
  single    batch 1, q = kv = 4096, 128 heads, bf16 N(0, 1), causal
  varlen    16 sequences, q = kv ~ U{128..8192}, 128 heads, fp16 N(0, 0.5), causal
  chunked   batch 8, kv = 16384, q = 2048 (last 2048 positions), 128 heads, bf16
  paged     32 sequences, ctx ~ U{1024..32768}, block size 128, 128 heads, bf16,
            block tables = a seeded permutation of all block ids

All use embeddimV = 128, rope 64 and qkScale = 1/sqrt(192).
"""
from __future__ import annotations

import math

import numpy as np
import torch

D_NOPE = 128
D_ROPE = 64
MASK_TILE = 512
BLOCK_SIZE = 128

MASK_UNDEFINED, MASK_SPEC, MASK_CAUSAL, MASK_FREE = 0, 1, 2, 3

WORKLOADS = {
    "tiny": dict(batch=2, heads=4, kv_heads=4, dtype=torch.bfloat16, sigma=1.0, seed=0),
    "single": dict(batch=1, heads=128, kv_heads=128, dtype=torch.bfloat16, sigma=1.0, seed=1),
    "varlen": dict(batch=16, heads=128, kv_heads=128, dtype=torch.float16, sigma=0.5, seed=2),
    "chunked": dict(batch=8, heads=128, kv_heads=128, dtype=torch.bfloat16, sigma=1.0, seed=3),
    "paged": dict(batch=32, heads=128, kv_heads=128, dtype=torch.bfloat16, sigma=1.0, seed=4),
}

QK_SCALE = 1.0 / math.sqrt(D_NOPE + D_ROPE)


def workload_seqlens(name: str, seed: int | None = None):
    """(q_seqlen, kv_seqlen) int32 numpy arrays of a named workload."""
    w = WORKLOADS[name]
    seed = w["seed"] if seed is None else seed
    if name == "tiny":
        q = np.array([17, 40], dtype=np.int32)
        return q, q.copy()
    if name == "single":
        q = np.array([4096], dtype=np.int32)
        return q, q.copy()
    if name == "varlen":
        rng = np.random.default_rng(seed)
        q = rng.integers(128, 8192, size=16, endpoint=True).astype(np.int32)
        return q, q.copy()
    if name == "chunked":
        return np.full(8, 2048, dtype=np.int32), np.full(8, 16384, dtype=np.int32)
    if name == "paged":
        rng = np.random.default_rng(seed)
        ctx = rng.integers(1024, 32768, size=32, endpoint=True).astype(np.int32)
        return ctx, ctx.copy()
    raise KeyError(name)


def _randn(shape, dtype, sigma, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(dtype)


def attention_inputs(q_seqlen, kv_seqlen, heads, kv_heads, dtype=torch.bfloat16, sigma=1.0,
                     seed=0, device="cpu", d_nope=D_NOPE, d_rope=D_ROPE, kv_padded_max_seq=0):
    """Seeded Q, QRope, K, KRope, V in packed varlen layout.

    Q [sum q, H, D], QRope [sum q, H, 64]; K, V [sum kv, Hkv, D], KRope
    [sum kv, Hkv, 64]. With kv_padded_max_seq > 0, K/KRope/V are instead
    [batch, max_seq, Hkv * dim] with rows past each sequence's length drawn too.
    Values: N(0, sigma^2) drawn in fp32 from torch.Generator(seed * 100 + k),
    k = 0..4, then rounded to dtype.
    """
    nq = int(np.sum(q_seqlen))
    nk = int(np.sum(kv_seqlen))
    base = int(seed) * 100
    t = {}
    t["q"] = _randn((nq, heads, d_nope), dtype, sigma, base + 0, device)
    t["q_rope"] = _randn((nq, heads, d_rope), dtype, sigma, base + 1, device)
    if kv_padded_max_seq:
        b = len(q_seqlen)
        m = int(kv_padded_max_seq)
        t["k"] = _randn((b, m, kv_heads * d_nope), dtype, sigma, base + 2, device)
        t["k_rope"] = _randn((b, m, kv_heads * d_rope), dtype, sigma, base + 3, device)
        t["v"] = _randn((b, m, kv_heads * d_nope), dtype, sigma, base + 4, device)
    else:
        t["k"] = _randn((nk, kv_heads, d_nope), dtype, sigma, base + 2, device)
        t["k_rope"] = _randn((nk, kv_heads, d_rope), dtype, sigma, base + 3, device)
        t["v"] = _randn((nk, kv_heads, d_nope), dtype, sigma, base + 4, device)
    return t


def workload_inputs(name: str, device="cpu", seed: int | None = None):
    """Inputs of a named workload: (tensors, q_seqlen, kv_seqlen, params)."""
    w = WORKLOADS[name]
    seed = w["seed"] if seed is None else seed
    qs, ks = workload_seqlens(name, seed)
    t = attention_inputs(qs, ks, w["heads"], w["kv_heads"], w["dtype"], w["sigma"], seed, device)
    params = dict(head_num=w["heads"], kv_head_num=w["kv_heads"], qk_scale=QK_SCALE,
                  mask_type=MASK_CAUSAL)
    return t, qs, ks, params


def causal_mask_tile(dtype=torch.float16, device="cpu"):
    """512 x 512 tile: 0 where column <= row, -inf above the diagonal."""
    tile = torch.zeros((MASK_TILE, MASK_TILE), dtype=torch.float32)
    upper = torch.ones((MASK_TILE, MASK_TILE), dtype=torch.bool).triu(1)
    tile[upper] = float("-inf")
    return tile.to(dtype).to(device)


def random_mask_tile(seed, dtype=torch.float16, device="cpu", p_masked=0.2, scale=2.0):
    """Seeded 512 x 512 tile of finite N(0, scale^2) values with a fraction of -inf
    entries, the diagonal kept finite so every query row keeps a visible key."""
    rng = np.random.default_rng(seed)
    tile = rng.standard_normal((MASK_TILE, MASK_TILE)) * scale
    tile[rng.random((MASK_TILE, MASK_TILE)) < p_masked] = -np.inf
    np.fill_diagonal(tile, rng.standard_normal(MASK_TILE))
    return torch.from_numpy(tile.astype(np.float32)).to(dtype).to(device)


def extreme_mask_tile(seed, dtype=torch.bfloat16, device="cpu"):
    """Seeded 512 x 512 tile with entries at the far ends of the dtype's range,
    on top of random_mask_tile's pattern: in a quarter of the rows 30% of the
    entries are the most negative finite value of the dtype (-3e38 for bf16,
    -65504 for fp16); in another quarter 20% are -1e30 (bf16) or -6e4 (fp16);
    in an eighth of the rows one entry is +1e30 (bf16) or +6e4 (fp16). Every
    row keeps its diagonal entry small and finite, so it keeps a visible key of
    moderate score, and has at most one large positive entry."""
    rng = np.random.default_rng(seed)
    tile = rng.standard_normal((MASK_TILE, MASK_TILE)) * 2.0
    tile[rng.random((MASK_TILE, MASK_TILE)) < 0.2] = -np.inf
    lowest = -3.0e38 if dtype == torch.bfloat16 else -65504.0
    big = 1.0e30 if dtype == torch.bfloat16 else 6.0e4
    for r in range(MASK_TILE):
        u = rng.random()
        if u < 0.25:
            tile[r, rng.random(MASK_TILE) < 0.3] = lowest
        elif u < 0.5:
            tile[r, rng.random(MASK_TILE) < 0.2] = -big
        elif u < 0.625:
            tile[r, rng.integers(0, MASK_TILE)] = big
        tile[r, r] = rng.standard_normal()
    return torch.from_numpy(tile.astype(np.float32)).to(dtype).to(device)


def paged_inputs(context_lens, heads=128, head_size_k=D_NOPE, head_size_v=D_NOPE,
                 head_size_rope=D_ROPE, block_size=BLOCK_SIZE, dtype=torch.bfloat16,
                 seed=4, device="cpu", with_rope=True):
    """Paged caches and a block table for the given context lengths.

    num_blocks = batch * ceil(max_ctx / block_size); the table is a seeded
    permutation of all block ids reshaped to [batch, ceil(max_ctx / block_size)],
    so unused tail columns still hold valid ids. Caches are fully drawn.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    batch = len(ctx)
    cols = int(-(-int(ctx.max()) // block_size)) if batch else 1
    num_blocks = batch * cols
    rng = np.random.default_rng(seed)
    table = rng.permutation(num_blocks).astype(np.int32).reshape(batch, cols)
    base = int(seed) * 100
    out = {
        "block_tables": torch.from_numpy(table).to(device),
        "context_lens": torch.from_numpy(ctx.astype(np.int32)).to(device),
        "key_cache": _randn((num_blocks, block_size, heads, head_size_k), dtype, 1.0, base + 5, device),
        "value_cache": _randn((num_blocks, block_size, heads, head_size_v), dtype, 1.0, base + 6, device),
    }
    if with_rope:
        out["rope_cache"] = _randn((num_blocks, block_size, heads, head_size_rope), dtype, 1.0,
                                   base + 7, device)
    return out


# ---------------------------------------------------------------- MLA prolog
# Sizes the "MlaProlog" page's constraints name: hidden size h 4096,
# q_lora_rank 1024, 64 heads of head_dim 512, rope_dim 64.
PROLOG_SIZES = dict(h=4096, q_lora_rank=1024, num_heads=64, head_dim=512, rope_dim=64)
PROLOG_TOKENS = 16384  # tokens of the measured prolog workload (the page allows 1 .. 64k)
PROLOG_EPS = 1e-6


def rope_tables(positions, rope_dim=64, base=10000.0, dtype=torch.bfloat16, device="cpu"):
    """cos / sin [len(positions), rope_dim]: the pair (2i, 2i + 1) of position
    p shares the angle p * base^(-2i / rope_dim)."""
    pos = torch.as_tensor(np.asarray(positions, dtype=np.float64))
    inv = base ** (-torch.arange(0, rope_dim, 2, dtype=torch.float64) / rope_dim)
    ang = torch.repeat_interleave(pos[:, None] * inv[None, :], 2, dim=1)
    return torch.cos(ang).to(dtype).to(device), torch.sin(ang).to(dtype).to(device)


def prolog_inputs(t, h=4096, q_lora_rank=1024, num_heads=64, head_dim=512, rope_dim=64, seed=0, device="cpu",
                  position0=0):
    """Seeded bf16 prolog inputs. token_x ~ N(0, 1); each weight ~ N(0, 1/fan_in)
    (random init of the stated shapes; no trained weights); gammas ~ 1 + 0.1 N(0, 1);
    rope tables for positions position0 .. position0 + t - 1. Values from
    torch.Generator(seed * 100 + k), k = 10 .. 15."""
    base = int(seed) * 100
    d = dict(
        token_x=_randn((t, h), torch.bfloat16, 1.0, base + 10, device),
        wq_a=_randn((h, q_lora_rank), torch.bfloat16, 1.0 / math.sqrt(h), base + 11, device),
        wq_b=_randn((q_lora_rank, num_heads * head_dim), torch.bfloat16, 1.0 / math.sqrt(q_lora_rank), base + 12,
                    device),
        wkv=_randn((h, head_dim), torch.bfloat16, 1.0 / math.sqrt(h), base + 13, device),
    )
    g1 = _randn((q_lora_rank,), torch.float32, 0.1, base + 14, device)
    g2 = _randn((head_dim,), torch.float32, 0.1, base + 15, device)
    d["gamma_cq"] = (1.0 + g1).to(torch.bfloat16)
    d["gamma_ckv"] = (1.0 + g2).to(torch.bfloat16)
    d["rope_cos"], d["rope_sin"] = rope_tables(np.arange(position0, position0 + t), rope_dim, device=device)
    return d


def prolog_quant_inputs(t, h=4096, q_lora_rank=1024, num_heads=64, head_dim=512, rope_dim=64, seed=0,
                        device="cpu", position0=0):
    """Seeded inputs of the quantised prolog: those of prolog_inputs, with wq_b
    replaced by int8 integers uniform in [-127, 127] and wq_b_scale (float32
    [num_heads * head_dim, 1]) uniform in [0.75, 1.25] * sqrt(3 / q_lora_rank)
    / 127, so that wq_b * wq_b_scale has about the variance 1 / q_lora_rank of
    the plain prolog's weight. Values from torch.Generator(seed * 100 + k),
    k = 10 .. 17."""
    d = prolog_inputs(t, h, q_lora_rank, num_heads, head_dim, rope_dim, seed, device, position0)
    base = int(seed) * 100
    g = torch.Generator(device="cpu").manual_seed(base + 16)
    d["wq_b"] = torch.randint(-127, 128, (q_lora_rank, num_heads * head_dim), generator=g,
                              dtype=torch.int8).to(device)
    g = torch.Generator(device="cpu").manual_seed(base + 17)
    u = torch.rand((num_heads * head_dim, 1), generator=g, dtype=torch.float32)
    d["wq_b_scale"] = ((0.75 + 0.5 * u) * math.sqrt(3.0 / q_lora_rank) / 127.0).to(device)
    return d


PROLOG_FLOP_PER_TOKEN = 2 * (PROLOG_SIZES["h"] * (PROLOG_SIZES["q_lora_rank"] + PROLOG_SIZES["head_dim"])
                             + PROLOG_SIZES["q_lora_rank"] * PROLOG_SIZES["num_heads"] * PROLOG_SIZES["head_dim"])
