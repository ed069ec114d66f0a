"""Pins of the CPU attention oracle against things other than itself.

Each test ties the oracle to the "MLA Prefill" page (Ascend Transformer Boost
C API, AtbMLAPreFillGetWorkspaceSize Members table) through an independent
route: a float64 brute force built differently (tests/brute.py), torch's
scaled_dot_product_attention as a library special case, closed forms and
invariants that the definition fixes. Together they are chosen so that a
dropped rope term, a scale applied to part of the product, a wrong causal
offset, a swapped operand or a wrong head mapping fails at least one of them
(test_oracle_mutants.py plants such mistakes and checks that they do).
"""
import math

import numpy as np
import pytest
import torch

import brute
import oracle

UNDEF, SPEC, CAUSAL, FREE = 0, 1, 2, 3


def bf16_values(shape, rng, sigma=1.0):
    """Random values exactly representable in bf16, as float64."""
    x = torch.from_numpy(rng.standard_normal(shape) * sigma).to(torch.bfloat16)
    return x.double().numpy()


def make_problem(q_seqlen, kv_seqlen, heads, kv_heads, d=16, r=8, seed=0, sigma=1.0):
    rng = np.random.default_rng(seed)
    nq, nk = int(sum(q_seqlen)), int(sum(kv_seqlen))
    return dict(
        q=bf16_values((nq, heads, d), rng, sigma), qr=bf16_values((nq, heads, r), rng, sigma),
        k=bf16_values((nk, kv_heads, d), rng, sigma), kr=bf16_values((nk, kv_heads, r), rng, sigma),
        v=bf16_values((nk, kv_heads, d), rng, sigma))


def run_oracle(p, q_seqlen, kv_seqlen, heads, kv_heads, scale, mask_type, tile=None):
    return oracle.attention(p["q"], p["qr"], p["k"], p["kr"], p["v"], q_seqlen, kv_seqlen,
                            heads, kv_heads, scale, mask_type, tile)


def run_brute(p, q_seqlen, kv_seqlen, heads, kv_heads, scale, mask_type, tile=None):
    return brute.attention(p["q"], p["qr"], p["k"], p["kr"], p["v"], q_seqlen, kv_seqlen,
                           heads, kv_heads, scale, mask_type, tile)


def random_tile(seed):
    rng = np.random.default_rng(seed)
    t = rng.standard_normal((512, 512)) * 2.0
    t[rng.random((512, 512)) < 0.25] = -np.inf
    np.fill_diagonal(t, rng.standard_normal(512))
    return t


def causal_tile():
    return np.where(np.tril(np.ones((512, 512), dtype=bool)), 0.0, -np.inf)


CASES = [
    # (q_seqlen, kv_seqlen, heads, kv_heads)
    ([17, 40], [17, 40], 4, 4),
    ([5, 9, 1], [12, 9, 30], 4, 2),     # chunked (q < kv) and GQA
    ([7, 3], [4, 0], 2, 1),             # q > kv, empty kv, MQA
    ([0, 6], [3, 6], 2, 2),             # empty query sequence
]


@pytest.mark.parametrize("mask_type", [UNDEF, SPEC, CAUSAL])
@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_brute_force(oracle_lib, case, mask_type):
    qs, ks, h, hk = case
    p = make_problem(qs, ks, h, hk, seed=len(qs) * 10 + mask_type)
    scale = 1.0 / math.sqrt(24)
    got = run_oracle(p, qs, ks, h, hk, scale, mask_type)
    want = run_brute(p, qs, ks, h, hk, scale, mask_type)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("q_len,kv_len", [(600, 600), (300, 700), (1, 530)])
def test_oracle_mask_free_random_tile_matches_brute_force(oracle_lib, q_len, kv_len):
    """MASK_FREE with a tile that is neither 0 nor causal, across a 512 boundary."""
    p = make_problem([q_len], [kv_len], 1, 1, d=8, r=4, seed=q_len)
    tile = random_tile(q_len + kv_len)
    got = run_oracle(p, [q_len], [kv_len], 1, 1, 0.3, FREE, tile)
    want = run_brute(p, [q_len], [kv_len], 1, 1, 0.3, FREE, tile)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mask_type", [UNDEF, CAUSAL])
def test_oracle_matches_torch_sdpa(oracle_lib, mask_type):
    """Library special case: with Qc = [Q|QRope], Kc = [K|KRope] the result is
    torch's float64 scaled_dot_product_attention with an explicit bottom-right
    boolean mask (torch's own is_causal is top-left, so it is not used)."""
    ql, kl, h = 23, 57, 3
    p = make_problem([ql], [kl], h, h, d=32, r=16, seed=7)
    scale = 0.17
    got = run_oracle(p, [ql], [kl], h, h, scale, mask_type)
    qc = torch.from_numpy(np.concatenate([p["q"], p["qr"]], -1)).permute(1, 0, 2)
    kc = torch.from_numpy(np.concatenate([p["k"], p["kr"]], -1)).permute(1, 0, 2)
    vv = torch.from_numpy(p["v"]).permute(1, 0, 2)
    if mask_type == CAUSAL:
        keep = torch.ones(ql, kl, dtype=torch.bool).tril(kl - ql)
    else:
        keep = torch.ones(ql, kl, dtype=torch.bool)
    want = torch.nn.functional.scaled_dot_product_attention(qc, kc, vv, attn_mask=keep, scale=scale)
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mask_type", [UNDEF, CAUSAL, FREE])
def test_softmax_weights_sum_to_one(oracle_lib, mask_type):
    ql, kl = 40, 70
    p = make_problem([ql], [kl], 1, 1, seed=3)
    tile = random_tile(5) if mask_type == FREE else None
    _, w = oracle.attention_head(p["q"][:, 0], p["qr"][:, 0], p["k"][:, 0], p["kr"][:, 0],
                                 p["v"][:, 0], 0.25, mask_type, tile, return_weights=True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert (w >= 0).all()
    if mask_type == CAUSAL:
        for i in range(ql):
            assert (w[i, kl - ql + i + 1:] == 0).all()


def test_single_visible_key_returns_that_value_row(oracle_lib):
    p = make_problem([1], [1], 2, 2, seed=11)
    out = run_oracle(p, [1], [1], 2, 2, 0.5, UNDEF)
    assert np.array_equal(out, p["v"])
    # causal row 0 of a square sequence sees only key 0
    p = make_problem([9], [9], 2, 2, seed=12)
    out = run_oracle(p, [9], [9], 2, 2, 0.5, CAUSAL)
    assert np.array_equal(out[0], p["v"][0])


@pytest.mark.parametrize("mask_type", [UNDEF, CAUSAL])
def test_zero_query_gives_mean_of_visible_values(oracle_lib, mask_type):
    """Q = QRope = 0 makes every score equal, so row i is the plain mean of the
    values it can see."""
    ql, kl = 6, 10
    p = make_problem([ql], [kl], 1, 1, seed=13)
    p["q"][:] = 0.0
    p["qr"][:] = 0.0
    out = run_oracle(p, [ql], [kl], 1, 1, 0.7, mask_type)
    for i in range(ql):
        n = kl if mask_type == UNDEF else kl - ql + i + 1
        np.testing.assert_allclose(out[i, 0], p["v"][:n, 0].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_constant_values_give_that_constant(oracle_lib):
    p = make_problem([5], [8], 2, 2, seed=14)
    p["v"][:] = 0.375
    out = run_oracle(p, [5], [8], 2, 2, 0.3, CAUSAL)
    np.testing.assert_allclose(out, 0.375, rtol=1e-14)


def test_two_key_closed_form_scale_covers_rope(oracle_lib):
    """One query, two keys. Nope dots are 1 and 0, rope dots 2 and -1, so the
    full products are 3 and -1 and the first weight is sigmoid(4 * scale).
    A scale that skipped the rope term, or a dropped rope term, gives another
    value."""
    q = np.array([[1.0, 0.0]])
    qr = np.array([[1.0, 1.0]])
    k = np.array([[1.0, 0.0], [0.0, 1.0]])
    kr = np.array([[1.0, 1.0], [0.0, -1.0]])
    v = np.array([[2.0, 0.0], [0.0, 4.0]])
    scale = 0.5
    out, w = oracle.attention_head(q, qr, k, kr, v, scale, UNDEF, return_weights=True)
    w0 = 1.0 / (1.0 + math.exp(-4.0 * scale))
    np.testing.assert_allclose(w[0], [w0, 1 - w0], rtol=1e-14)
    np.testing.assert_allclose(out[0], [2 * w0, 4 * (1 - w0)], rtol=1e-14)


def test_mask_added_after_scale_closed_form(oracle_lib):
    """MASK_FREE tile entry m adds to scale * dot: with dots 0 and 0 and a tile
    entry of log(3) on the first key, the weights are 3/4 and 1/4 for any scale."""
    tile = np.zeros((512, 512))
    tile[0, 1] = -np.inf
    tile[1, 0] = math.log(3.0)
    q = np.zeros((2, 2))
    qr = np.zeros((2, 1))
    k = np.ones((2, 2))
    kr = np.ones((2, 1))
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    out = oracle.attention_head(q, qr, k, kr, v, 5.0, FREE, tile)
    np.testing.assert_allclose(out[1], [0.75, 0.25], rtol=1e-14)
    np.testing.assert_allclose(out[0], [1.0, 0.0], rtol=0, atol=0)


def test_rows_without_visible_keys_are_zero(oracle_lib):
    p = make_problem([6, 2], [3, 0], 1, 1, seed=15)
    out = run_oracle(p, [6, 2], [3, 0], 1, 1, 0.4, CAUSAL)
    assert (out[:3] == 0).all()          # positions -3..-1 see nothing
    assert (out[6:] == 0).all()          # empty kv sequence
    assert np.abs(out[3:6]).sum() > 0


@pytest.mark.parametrize("mask_type", [SPEC, CAUSAL])
def test_causal_invariance(oracle_lib, mask_type):
    """Changing keys/values after position p leaves rows at positions <= p
    bit-identical."""
    ql, kl = 12, 20
    p = make_problem([ql], [kl], 2, 2, seed=16)
    base = run_oracle(p, [ql], [kl], 2, 2, 0.3, mask_type)
    cut = 13
    for name in ("k", "kr", "v"):
        p2 = {n: a.copy() for n, a in p.items()}
        p2[name][cut + 1:] += 5.0
        out = run_oracle(p2, [ql], [kl], 2, 2, 0.3, mask_type)
        first_changed = cut - (kl - ql) + 1
        assert np.array_equal(out[:first_changed], base[:first_changed])
        assert not np.array_equal(out[first_changed:], base[first_changed:])


def test_batch_independence(oracle_lib):
    qs, ks = [9, 4, 11], [9, 15, 11]
    p = make_problem(qs, ks, 2, 2, seed=17)
    full = run_oracle(p, qs, ks, 2, 2, 0.3, CAUSAL)
    # sequence 1 alone
    one = {"q": p["q"][9:13], "qr": p["qr"][9:13], "k": p["k"][9:24], "kr": p["kr"][9:24],
           "v": p["v"][9:24]}
    alone = run_oracle(one, [4], [15], 2, 2, 0.3, CAUSAL)
    assert np.array_equal(full[9:13], alone)


def test_mask_free_with_causal_tile_equals_causal(oracle_lib):
    qs, ks = [700, 40], [1100, 40]
    p = make_problem(qs, ks, 1, 1, d=8, r=4, seed=18)
    a = run_oracle(p, qs, ks, 1, 1, 0.3, FREE, causal_tile())
    b = run_oracle(p, qs, ks, 1, 1, 0.3, CAUSAL)
    assert np.array_equal(a, b)


def test_spec_with_single_query_equals_undefined(oracle_lib):
    p = make_problem([1, 1], [30, 7], 2, 2, seed=19)
    a = run_oracle(p, [1, 1], [30, 7], 2, 2, 0.3, SPEC)
    b = run_oracle(p, [1, 1], [30, 7], 2, 2, 0.3, UNDEF)
    assert np.array_equal(a, b)


def test_grouped_heads_equal_expanded_heads(oracle_lib):
    qs, ks = [8, 5], [8, 9]
    p = make_problem(qs, ks, 6, 2, seed=20)
    a = run_oracle(p, qs, ks, 6, 2, 0.3, CAUSAL)
    e = dict(p)
    for n in ("k", "kr", "v"):
        e[n] = np.repeat(p[n], 3, axis=1)
    b = run_oracle(e, qs, ks, 6, 6, 0.3, CAUSAL)
    assert np.array_equal(a, b)


def test_padded_kv_layout_equals_packed(oracle_lib):
    qs, ks = [4, 6], [7, 3]
    p = make_problem(qs, ks, 2, 2, seed=21)
    packed = run_oracle(p, qs, ks, 2, 2, 0.3, CAUSAL)
    max_seq = 9
    pad = {"q": p["q"], "qr": p["qr"]}
    for n in ("k", "kr", "v"):
        a = np.full((2, max_seq) + p[n].shape[1:], np.nan)
        a[0, :7] = p[n][:7]
        a[1, :3] = p[n][7:]
        pad[n] = a
    got = oracle.attention(pad["q"], pad["qr"], pad["k"], pad["kr"], pad["v"], qs, ks, 2, 2, 0.3,
                           CAUSAL, kv_padded=True)
    assert np.array_equal(got, packed)


def test_oracle_rejects_bad_rows(oracle_lib):
    q = np.zeros((2, 4))
    with pytest.raises(ValueError):
        oracle.attention_head(q, q[:, :2], q, q[:, :2], q, 1.0, UNDEF, rows=[2])
