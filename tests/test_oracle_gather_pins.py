"""Pins of the paged-gather oracle ("PagedCacheLoadOperation" page, Members
table) against round trips and identities the page's definitions fix."""
import numpy as np
import pytest

import oracle


def scatter_to_cache(rows, lens, table, block_size, num_blocks, starts=None):
    """Place each sequence's contiguous rows into a paged cache (the inverse of
    the gather, written as a plain per-token loop)."""
    cache = np.full((num_blocks, block_size) + rows.shape[1:], -7, dtype=rows.dtype)
    off = 0
    for b, n in enumerate(lens):
        s = 0 if starts is None else int(starts[b])
        for t in range(n):
            pos = s + t
            cache[table[b][pos // block_size], pos % block_size] = rows[off + t]
        off += n
    return cache


def test_round_trip_through_permuted_table():
    rng = np.random.default_rng(0)
    bs, lens = 4, [5, 12, 1, 8]
    cols = max(-(-n // bs) for n in lens)
    nb = len(lens) * cols
    table = rng.permutation(nb).reshape(len(lens), cols).astype(np.int32)
    rows = rng.integers(-1000, 1000, size=(sum(lens), 3, 5)).astype(np.int16)
    cache = scatter_to_cache(rows, lens, table, bs, nb)
    key, value = oracle.paged_cache_load(cache, cache[:, :, :, :2], table, lens)
    assert np.array_equal(key, rows)
    assert np.array_equal(value, rows[:, :, :2])


def test_identity_table_is_a_reshape():
    rng = np.random.default_rng(1)
    bs, nbps = 8, 3
    cache = rng.integers(0, 255, size=(2 * nbps, bs, 2, 4)).astype(np.uint8)
    table = np.arange(2 * nbps, dtype=np.int32).reshape(2, nbps)
    key, _ = oracle.paged_cache_load(cache, None, table, [bs * nbps, bs * nbps])
    assert np.array_equal(key, cache.reshape(-1, 2, 4))


def test_cumsum_forms_equal_plain_lengths():
    rng = np.random.default_rng(2)
    bs, lens = 4, [3, 9, 0, 6]
    nb = 4 * 3
    table = rng.permutation(nb).reshape(4, 3).astype(np.int32)
    cache = rng.standard_normal((nb, bs, 2, 2)).astype(np.float32)
    plain, _ = oracle.paged_cache_load(cache, None, table, lens)
    inclusive = np.cumsum(lens)
    exclusive = np.concatenate([[0], inclusive])
    a, _ = oracle.paged_cache_load(cache, None, table, inclusive, is_seq_lens_cumsum=True)
    b, _ = oracle.paged_cache_load(cache, None, table, exclusive, is_seq_lens_cumsum=True)
    assert np.array_equal(a, plain) and np.array_equal(b, plain)


def test_seq_start_shift_identity():
    """gather(len, start s) equals gather(len + s, start 0) without its first s rows."""
    rng = np.random.default_rng(3)
    bs, nb = 4, 24
    table = rng.permutation(nb).reshape(3, 8).astype(np.int32)
    cache = rng.standard_normal((nb, bs, 1, 3)).astype(np.float32)
    lens, starts = [5, 7, 2], [3, 10, 0]
    shifted, _ = oracle.paged_cache_load(cache, None, table, lens, seq_starts=starts,
                                         has_seq_starts=True)
    longer, _ = oracle.paged_cache_load(cache, None, table, [n + s for n, s in zip(lens, starts)])
    off_long = np.concatenate([[0], np.cumsum([n + s for n, s in zip(lens, starts)])])
    expect = np.concatenate([longer[off_long[b] + starts[b]:off_long[b + 1]] for b in range(3)])
    assert np.array_equal(shifted, expect)
    # with has_seq_starts false the starts are ignored
    ignored, _ = oracle.paged_cache_load(cache, None, table, lens, seq_starts=starts,
                                         has_seq_starts=False)
    zero, _ = oracle.paged_cache_load(cache, None, table, lens, seq_starts=[0, 0, 0],
                                      has_seq_starts=True)
    assert np.array_equal(ignored, zero)


def test_round_trip_with_seq_starts():
    rng = np.random.default_rng(4)
    bs, lens, starts = 8, [9, 4], [6, 17]
    cols = 4
    table = rng.permutation(2 * cols).reshape(2, cols).astype(np.int32)
    rows = rng.standard_normal((sum(lens), 2, 2)).astype(np.float32)
    cache = scatter_to_cache(rows, lens, table, bs, 2 * cols, starts)
    key, _ = oracle.paged_cache_load(cache, None, table, lens, seq_starts=starts,
                                     has_seq_starts=True)
    assert np.array_equal(key, rows)


def test_page_block_table_width_formula():
    """The page gives blockTables as [len(contextLens), (max(contextLens) - 1)
    // block_size + 1]: the widest sequence uses exactly that many blocks."""
    lens, bs = [1, 128, 129, 300], 128
    width = (max(lens) - 1) // bs + 1
    assert width == 3
    assert all((n - 1) // bs + 1 <= width for n in lens)


@pytest.mark.parametrize("block_size", [3, 16])
def test_paged_attention_equals_attention_on_the_scattered_kv(block_size):
    # Fused paged attention is, by definition, the gather followed by attention:
    # scatter contiguous K/KRope/V into a permuted cache whose unused blocks
    # hold NaN, and the paged result must equal attention on the contiguous
    # tensors exactly (the same fp64 arithmetic on the same values).
    rng = np.random.default_rng(3)
    qlens, kvlens = [5, 9, 0, 4], [7, 9, 3, 11]
    H, HK, D, R = 4, 2, 8, 4
    cols = max(-(-n // block_size) for n in kvlens) + 1
    nb = len(kvlens) * cols + 2
    table = rng.permutation(nb)[:len(kvlens) * cols].reshape(len(kvlens), cols).astype(np.int32)
    q = rng.standard_normal((sum(qlens), H, D))
    qr = rng.standard_normal((sum(qlens), H, R))
    k = rng.standard_normal((sum(kvlens), HK, D))
    kr = rng.standard_normal((sum(kvlens), HK, R))
    v = rng.standard_normal((sum(kvlens), HK, D))

    def cache_of(rows):
        c = scatter_to_cache(rows, kvlens, table, block_size, nb)
        used = np.zeros((nb, block_size), bool)
        for b, n in enumerate(kvlens):
            for t in range(n):
                used[table[b][t // block_size], t % block_size] = True
        c[~used] = np.nan
        return c

    for mask_type in (oracle.MASK_CAUSAL, oracle.MASK_UNDEFINED):
        ref = oracle.attention(q, qr, k, kr, v, qlens, kvlens, H, HK, 0.3, mask_type)
        got = oracle.paged_attention(q, qr, cache_of(k), cache_of(kr), cache_of(v), table, qlens, kvlens, H, HK,
                                     0.3, mask_type)
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref)


def nd_to_nz(cache_nd, elems):
    """NZ form of an ND cache [nb, bs, H, hs]: each slot's H*hs row cut into
    chunks of ``elems``, chunk index moved in front of the slot index."""
    nb, bs, h, hs = cache_nd.shape
    return cache_nd.reshape(nb, bs, h * hs // elems, elems).transpose(0, 2, 1, 3).copy()


@pytest.mark.parametrize("dtype,elems", [(np.int16, 16), (np.int8, 32)])
def test_nz_gather_equals_nd_gather_reshaped(dtype, elems):
    rng = np.random.default_rng(7)
    bs, lens, heads, hs = 8, [5, 17, 0, 9], 4, 32
    cols = max(-(-n // bs) for n in lens)
    nb = len(lens) * cols + 1
    table = rng.permutation(nb)[:len(lens) * cols].reshape(len(lens), cols).astype(np.int32)
    nd = rng.integers(-100, 100, size=(nb, bs, heads, hs)).astype(dtype)
    nd_v = rng.integers(-100, 100, size=(nb, bs, heads, hs // 2)).astype(dtype)
    k_nd, v_nd = oracle.paged_cache_load(nd, nd_v, table, lens)
    k_nz, v_nz = oracle.paged_cache_load_nz(nd_to_nz(nd, elems), nd_to_nz(nd_v, elems), table, lens)
    assert np.array_equal(k_nz, k_nd.reshape(len(k_nd), -1))
    assert np.array_equal(v_nz, v_nd.reshape(len(v_nd), -1))


def test_nz_gather_worked_example():
    # 2 blocks, 2 chunks of 2 elements, block size 2; one sequence of 3 tokens
    # whose table row is [1, 0]: tokens 0, 1 sit in block 1 slots 0, 1, token 2
    # in block 0 slot 0. cache[k, c, s, e] = 1000k + 100c + 10s + e.
    cache = np.array([[[[1000 * k + 100 * c + 10 * s + e for e in range(2)] for s in range(2)] for c in range(2)]
                      for k in range(2)], dtype=np.int32)
    key, value = oracle.paged_cache_load_nz(cache, None, [[1, 0]], [3])
    assert value is None
    assert key.tolist() == [[1000, 1001, 1100, 1101],
                            [1010, 1011, 1110, 1111],
                            [0, 1, 100, 101]]
