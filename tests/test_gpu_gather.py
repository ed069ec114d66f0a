"""GPU parity of the paged gather against the numpy oracle: bit-exact."""
import numpy as np
import pytest
import torch

import mla_varlen_prefill_amd as mla
from mla_varlen_prefill_amd import synth
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def gather_gpu(caches, lens_dev, total, seq_starts=None, cumsum=False, has_starts=False, with_value=True,
               key_name="key_cache", value_name="value_cache"):
    kc = caches[key_name]
    vc = caches[value_name] if with_value else None
    key = torch.full((total,) + tuple(kc.shape[2:]), 77, dtype=kc.dtype, device=DEV) if kc.dtype == torch.int8 \
        else torch.full((total,) + tuple(kc.shape[2:]), float("nan"), dtype=kc.dtype, device=DEV)
    value = None
    if vc is not None:
        value = torch.zeros((total,) + tuple(vc.shape[2:]), dtype=vc.dtype, device=DEV)
    mla.paged_cache_load(kc, vc, caches["block_tables"], lens_dev, key, value, seq_starts,
                         mla.KV_CACHE_ND, cumsum, has_starts)
    torch.cuda.synchronize()
    return key, value


def as_bits(t):
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


def oracle_gather(caches, lens, starts=None, cumsum=False, has_starts=False, with_value=True,
                  key_name="key_cache", value_name="value_cache"):
    kc = as_bits(caches[key_name])
    vc = as_bits(caches[value_name]) if with_value else None
    table = caches["block_tables"].cpu().numpy()
    return oracle.paged_cache_load(kc, vc, table, lens, starts, cumsum, has_starts)


def test_gather_small_bit_exact():
    lens = [1, 127, 128, 129, 500, 3]
    _say(f"[gpu] gather lens={lens}")
    caches = synth.paged_inputs(lens, heads=4, head_size_k=128, head_size_v=128, block_size=128, seed=1,
                                device=DEV)
    key, value = gather_gpu(caches, caches["context_lens"], sum(lens))
    rk, rv = oracle_gather(caches, lens)
    assert np.array_equal(as_bits(key), rk) and np.array_equal(as_bits(value), rv)


@pytest.mark.parametrize("form", ["inclusive", "exclusive"])
def test_gather_cumsum_forms(form):
    lens = [7, 0, 300, 64]
    caches = synth.paged_inputs(lens, heads=2, block_size=64, seed=2, device=DEV)
    inc = np.cumsum(lens).astype(np.int32)
    ctx = inc if form == "inclusive" else np.concatenate([[0], inc]).astype(np.int32)
    key, value = gather_gpu(caches, torch.from_numpy(ctx).to(DEV), sum(lens), cumsum=True)
    rk, rv = oracle_gather(caches, lens)
    assert np.array_equal(as_bits(key), rk) and np.array_equal(as_bits(value), rv)


def test_gather_seq_starts():
    lens, starts = [50, 9, 200], [10, 120, 0]
    ctx = [n + s for n, s in zip(lens, starts)]
    caches = synth.paged_inputs(ctx, heads=2, block_size=32, seed=3, device=DEV)
    st = torch.tensor(starts, dtype=torch.int32, device=DEV)
    key, value = gather_gpu(caches, torch.tensor(lens, dtype=torch.int32, device=DEV), sum(lens), st,
                            has_starts=True)
    rk, rv = oracle_gather(caches, lens, starts, has_starts=True)
    assert np.array_equal(as_bits(key), rk) and np.array_equal(as_bits(value), rv)
    # has_seq_starts false ignores the starts
    key2, _ = gather_gpu(caches, torch.tensor(lens, dtype=torch.int32, device=DEV), sum(lens), st,
                         has_starts=False)
    rk2, _ = oracle_gather(caches, lens)
    assert np.array_equal(as_bits(key2), rk2)


def test_gather_keys_only_rope_cache():
    lens = [300, 17]
    caches = synth.paged_inputs(lens, heads=4, block_size=128, seed=4, device=DEV)
    key, value = gather_gpu(caches, caches["context_lens"], sum(lens), with_value=False, key_name="rope_cache")
    assert value is None
    rk, _ = oracle_gather(caches, lens, with_value=False, key_name="rope_cache")
    assert np.array_equal(as_bits(key), rk)


def test_gather_int8_and_odd_row_bytes():
    """int8 caches and rows that are not a multiple of 16 bytes (byte path)."""
    lens = [40, 13]
    nb, bs = 8, 16
    g = torch.Generator(device=DEV).manual_seed(5)
    kc = torch.randint(-128, 127, (nb, bs, 3, 5), dtype=torch.int8, device=DEV, generator=g)
    vc = torch.randint(-128, 127, (nb, bs, 3, 7), dtype=torch.int8, device=DEV, generator=g)
    table = torch.from_numpy(np.random.default_rng(5).permutation(nb).reshape(2, 4).astype(np.int32)).to(DEV)
    caches = {"key_cache": kc, "value_cache": vc, "block_tables": table}
    key, value = gather_gpu(caches, torch.tensor(lens, dtype=torch.int32, device=DEV), sum(lens))
    rk, rv = oracle_gather(caches, lens)
    assert np.array_equal(key.cpu().numpy(), rk) and np.array_equal(value.cpu().numpy(), rv)


def test_gather_skips_out_of_range_rows():
    """A block id outside the cache leaves its output rows untouched."""
    lens = [20]
    caches = synth.paged_inputs(lens, heads=2, block_size=8, seed=6, device=DEV)
    caches["block_tables"][0, 1] = 10_000
    key, _ = gather_gpu(caches, caches["context_lens"], 20)
    assert torch.isnan(key[8:16].float()).all()
    table = caches["block_tables"].cpu().numpy().copy()
    kc = as_bits(caches["key_cache"])
    for t in (0, 7, 16, 19):
        assert np.array_equal(as_bits(key[t]), kc[table[0, t // 8], t % 8])


def test_gather_full_paged_workload_sampled_rows():
    """The paged workload at full size (32 sequences, ctx up to 32768, 128 heads):
    seeded output tokens, plus each sequence's first and last token, compared
    bit for bit with the oracle's gather of those tokens. The oracle is given
    the cache blocks those tokens live in (copied whole to the host) and, per
    token, its sequence's table row (renumbered to the copied blocks) with
    a one-token length and the token's position as the start offset, so the
    block and slot arithmetic is the oracle's own."""
    lens, _ = synth.workload_seqlens("paged")
    total = int(lens.sum())
    _say(f"[gpu] full paged gather, total tokens {total}")
    caches = synth.paged_inputs(lens, device=DEV, with_rope=True)
    key, value = gather_gpu(caches, caches["context_lens"], total)
    rope, _ = gather_gpu(caches, caches["context_lens"], total, with_value=False, key_name="rope_cache")
    table = caches["block_tables"].cpu().numpy()
    bs = caches["key_cache"].shape[1]
    off = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(7)
    picks = set(int(x) for x in rng.integers(0, total, size=256))
    for b in range(len(lens)):
        picks |= {int(off[b]), int(off[b + 1] - 1)}
    picks = np.array(sorted(picks))
    b_of = np.searchsorted(off, picks, side="right") - 1
    t_of = picks - off[b_of]
    used = np.unique(table[b_of, t_of // bs])
    renum = np.full(caches["key_cache"].shape[0], -1, np.int64)
    renum[used] = np.arange(len(used))
    sub_table = renum[table[b_of]]  # one row per picked token: its sequence's row, renumbered
    sub_table[sub_table < 0] = 0    # blocks no picked token reads
    ones = np.ones(len(picks), np.int64)
    blk = torch.from_numpy(used).to(DEV)
    idx = torch.from_numpy(picks).to(DEV)
    for out, cache in ((key, "key_cache"), (value, "value_cache"), (rope, "rope_cache")):
        sub_cache = as_bits(caches[cache][blk])
        want, _ = oracle.paged_cache_load(sub_cache, None, sub_table, ones, seq_starts=t_of, has_seq_starts=True)
        assert np.array_equal(as_bits(out[idx]), want), cache


def test_gather_total_past_two_to_the_31():
    """Plain lengths whose total passes 2^31: sequences of 1.2e9 and 1.0e9
    tokens, rows of one bf16 element, block size 128, the table columns
    cycling over a seeded permutation of 64 cache blocks. The device sums the
    lengths in 64 bits, so the rows of the second sequence past 2^31 are
    written where they belong. Rows around 2^31, at both ends and at random
    are compared bit for bit with the oracle's gather of those tokens (each
    given as a one-token sequence whose block table is the window of its own
    table row that holds it, from a start position inside that window)."""
    lens = np.array([1_200_000_000, 1_000_000_000], np.int64)
    total = int(lens.sum())
    assert total > 2**31
    _say(f"[gpu] gather, total {total} tokens past 2^31")
    bs, nb = 128, 64
    cols = int(-(-lens.max() // bs))
    rng = np.random.default_rng(12)
    table = rng.permutation(nb).astype(np.int32)[np.arange(2 * cols) % nb].reshape(2, cols)
    g = torch.Generator(device=DEV).manual_seed(1200)
    cache = torch.randn((nb, bs, 1, 1), generator=g, device=DEV).to(torch.bfloat16)
    caches = {"key_cache": cache, "block_tables": torch.from_numpy(table).to(DEV)}
    key, _ = gather_gpu(caches, torch.from_numpy(lens.astype(np.int32)).to(DEV), total, with_value=False)
    off = np.array([0, lens[0], total])
    picks = {2**31 - 2, 2**31 - 1, 2**31, 2**31 + 1, 0, int(lens[0]) - 1, int(lens[0]), total - 1}
    picks |= set(int(x) for x in rng.integers(2**31, total, size=24))
    picks |= set(int(x) for x in rng.integers(0, total, size=24))
    picks = np.array(sorted(picks))
    b_of = np.searchsorted(off, picks, side="right") - 1
    t_of = picks - off[b_of]
    col = t_of // bs
    windows = table[b_of, col][:, None]          # the table column holding each token
    starts = t_of - col * bs                     # its position inside that window
    want, _ = oracle.paged_cache_load(as_bits(cache), None, windows, np.ones(len(picks), np.int64),
                                      seq_starts=starts, has_seq_starts=True)
    got = as_bits(key[torch.from_numpy(picks).to(DEV)])
    assert np.array_equal(got, want)


def test_gather_nd_reduced_paged_workload_bit_exact():
    """The paged workload's lengths and block table at 8 heads (K, V, KRope
    caches [8192, 128, 8, 128 | 128 | 64] bf16, ND): every output row compared
    bit for bit with the oracle."""
    lens, _ = synth.workload_seqlens("paged")
    total = int(lens.sum())
    _say(f"[gpu] ND gather, reduced paged workload, {total} tokens")
    c = synth.paged_inputs(lens, heads=8, device=DEV, with_rope=True)
    key, value = gather_gpu(c, c["context_lens"], total)
    rope, _ = gather_gpu(c, c["context_lens"], total, with_value=False, key_name="rope_cache")
    rk, rv = oracle_gather(c, lens)
    assert np.array_equal(as_bits(key), rk)
    assert np.array_equal(as_bits(value), rv)
    del rk, rv
    rr, _ = oracle_gather(c, lens, with_value=False, key_name="rope_cache")
    assert np.array_equal(as_bits(rope), rr)


# ---------------------------------------------------------------- NZ layout

def nd_to_nz(cache_nd, elems):
    """NZ form of an ND cache [nb, bs, H, hs] (the page's dimension table, NZ
    column): each slot's H*hs row cut into chunks of ``elems`` elements, the
    chunk index moved in front of the slot index."""
    nb, bs, h, hs = cache_nd.shape
    return cache_nd.reshape(nb, bs, h * hs // elems, elems).permute(0, 2, 1, 3).contiguous()


def gather_nz_gpu(kc, vc, table, lens_dev, total):
    key = torch.zeros((total, kc.shape[1] * kc.shape[3]), dtype=kc.dtype, device=DEV)
    value = None if vc is None else torch.zeros((total, vc.shape[1] * vc.shape[3]), dtype=vc.dtype, device=DEV)
    mla.paged_cache_load(kc, vc, table, lens_dev, key, value, None, mla.KV_CACHE_NZ, False, False)
    torch.cuda.synchronize()
    return key, value


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.int8])
def test_gather_nz_small_bit_exact(dtype):
    lens = [1, 31, 32, 33, 300, 0, 129]
    _say(f"[gpu] NZ gather {dtype} lens={lens}")
    bs, heads = 64, 4
    elems = 32 if dtype == torch.int8 else 16
    cols = max(-(-n // bs) for n in lens)
    nb = len(lens) * cols + 2
    rng = np.random.default_rng(5)
    table = torch.from_numpy(rng.permutation(nb)[:len(lens) * cols].reshape(len(lens), cols).astype(np.int32))
    g = torch.Generator().manual_seed(6)
    if dtype == torch.int8:
        kd = torch.randint(-128, 128, (nb, bs, heads, 128), generator=g, dtype=torch.int8)
        vd = torch.randint(-128, 128, (nb, bs, heads, 64), generator=g, dtype=torch.int8)
    else:
        kd = torch.randn((nb, bs, heads, 128), generator=g).to(dtype)
        vd = torch.randn((nb, bs, heads, 64), generator=g).to(dtype)
    kz, vz = nd_to_nz(kd, elems), nd_to_nz(vd, elems)
    lens_dev = torch.tensor(lens, dtype=torch.int32, device=DEV)
    key, value = gather_nz_gpu(kz.to(DEV), vz.to(DEV), table.to(DEV), lens_dev, sum(lens))
    rk, rv = oracle.paged_cache_load_nz(as_bits(kz), as_bits(vz), table.numpy(), lens)
    assert np.array_equal(as_bits(key), rk) and np.array_equal(as_bits(value), rv)
    # and the NZ gather equals the ND gather of the same data, reshaped
    caches = {"key_cache": kd.to(DEV), "value_cache": vd.to(DEV), "block_tables": table.to(DEV)}
    knd, vnd = gather_gpu(caches, lens_dev, sum(lens))
    assert torch.equal(as_bits_t(key), as_bits_t(knd.reshape(len(knd), -1)))
    assert torch.equal(as_bits_t(value), as_bits_t(vnd.reshape(len(vnd), -1)))


def as_bits_t(t):
    return t.view(torch.int16) if t.dtype in (torch.float16, torch.bfloat16) else t


def test_gather_nz_reduced_paged_workload_bit_exact():
    """The paged workload's lengths and table at 8 heads (the full one at 128
    heads is the bench's): K, V and KRope caches in NZ, every row compared with
    the oracle."""
    lens, _ = synth.workload_seqlens("paged")
    total = int(lens.sum())
    _say(f"[gpu] NZ gather, reduced paged workload, {total} tokens")
    c = synth.paged_inputs(lens, heads=8, device=DEV, with_rope=True)
    kz, vz, rz = (nd_to_nz(c[n], 16) for n in ("key_cache", "value_cache", "rope_cache"))
    del c["key_cache"], c["value_cache"], c["rope_cache"]
    lens_dev = torch.from_numpy(np.asarray(lens, np.int32)).to(DEV)
    table = c["block_tables"].cpu().numpy()
    key, value = gather_nz_gpu(kz, vz, c["block_tables"], lens_dev, total)
    rope, _ = gather_nz_gpu(rz, None, c["block_tables"], lens_dev, total)
    rk, rv = oracle.paged_cache_load_nz(as_bits(kz), as_bits(vz), table, lens)
    rr, _ = oracle.paged_cache_load_nz(as_bits(rz), None, table, lens)
    assert np.array_equal(as_bits(key), rk)
    assert np.array_equal(as_bits(value), rv)
    assert np.array_equal(as_bits(rope), rr)
