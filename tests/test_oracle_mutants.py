"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them.

The C oracle is copied to a temporary directory, one source line is changed
(a dropped rope term, a scale on part of the product, a top-left or
off-by-one causal rule, a reversed index, a flipped exponent sign, a missing
normalisation, a wrong MASK_FREE block rule or a transposed tile), the copy is
compiled, and the pins of test_oracle_pins.py are re-run against it: at least
one must fail. The Python parts (head grouping, gather spans and slots) are
mutated the same way in a private copy of the module. Nothing here touches the
real oracle files.
"""
import importlib.util
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import brute
import oracle

ORACLE_DIR = os.path.dirname(oracle.__file__)
UNDEF, SPEC, CAUSAL, FREE = 0, 1, 2, 3


def _problem(q_seqlen, kv_seqlen, heads, kv_heads, d=16, r=8, seed=0):
    rng = np.random.default_rng(seed)
    nq, nk = sum(q_seqlen), sum(kv_seqlen)

    def vals(shape):
        return np.round(rng.standard_normal(shape) * 64) / 64

    return dict(q=vals((nq, heads, d)), qr=vals((nq, heads, r)), k=vals((nk, kv_heads, d)),
                kr=vals((nk, kv_heads, r)), v=vals((nk, kv_heads, d)))


def _tile(seed):
    rng = np.random.default_rng(seed)
    t = rng.standard_normal((512, 512)) * 2.0
    t[rng.random((512, 512)) < 0.25] = -np.inf
    np.fill_diagonal(t, 0.5)
    return t


def _attention_pins(mod, lib):
    """Pins that compare an oracle (module ``mod`` driving library ``lib``)
    with the brute force and closed forms. Returns the names that fail; a
    mutant that crashes a pin counts as caught."""
    try:
        return _attention_pins_unguarded(mod, lib)
    except (IndexError, ValueError, AssertionError) as e:
        return [f"raised {type(e).__name__}"]


def _attention_pins_unguarded(mod, lib):
    failed = []
    cases = [([17, 9], [17, 30], 4, 2), ([7, 3], [4, 5], 2, 1)]
    for mask_type in (UNDEF, CAUSAL):
        for qs, ks, h, hk in cases:
            p = _problem(qs, ks, h, hk, seed=sum(qs))
            got = mod.attention(p["q"], p["qr"], p["k"], p["kr"], p["v"], qs, ks, h, hk, 0.2,
                                mask_type, lib=lib)
            want = brute.attention(p["q"], p["qr"], p["k"], p["kr"], p["v"], qs, ks, h, hk, 0.2,
                                   mask_type)
            if not np.allclose(got, want, rtol=1e-10, atol=1e-12):
                failed.append(f"brute mask={mask_type} case={qs}/{ks}")
    for ql, kl in ((600, 600), (300, 700)):
        p = _problem([ql], [kl], 1, 1, d=4, r=4, seed=ql)
        tile = _tile(kl)
        got = mod.attention(p["q"], p["qr"], p["k"], p["kr"], p["v"], [ql], [kl], 1, 1, 0.3, FREE,
                            tile, lib=lib)
        want = brute.attention(p["q"], p["qr"], p["k"], p["kr"], p["v"], [ql], [kl], 1, 1, 0.3,
                               FREE, tile)
        if not np.allclose(got, want, rtol=1e-10, atol=1e-12):
            failed.append(f"brute mask-free {ql}/{kl}")
    # closed form: one query, two keys, products 3 and -1
    q, qr = np.array([[1.0, 0.0]]), np.array([[1.0, 1.0]])
    k, kr = np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([[1.0, 1.0], [0.0, -1.0]])
    v = np.array([[2.0, 0.0], [0.0, 4.0]])
    w0 = 1.0 / (1.0 + math.exp(-2.0))
    out = mod.attention_head(q, qr, k, kr, v, 0.5, UNDEF, lib=lib)
    if not np.allclose(out[0], [2 * w0, 4 * (1 - w0)], rtol=1e-13):
        failed.append("closed form")
    return failed


def _gather_pins(mod):
    failed = []
    rng = np.random.default_rng(0)
    bs, lens = 4, [5, 12, 1, 8]
    table = rng.permutation(16).reshape(4, 4).astype(np.int32)
    rows = rng.integers(-1000, 1000, size=(sum(lens), 2, 3)).astype(np.int16)
    cache = np.zeros((16, bs, 2, 3), dtype=np.int16)
    off = 0
    for b, n in enumerate(lens):
        for t in range(n):
            cache[table[b][t // bs], t % bs] = rows[off + t]
        off += n
    key, _ = mod.paged_cache_load(cache, None, table, lens)
    if key.shape != rows.shape or not np.array_equal(key, rows):
        failed.append("round trip")
    inc = np.cumsum(lens)
    try:
        a, _ = mod.paged_cache_load(cache, None, table, inc, is_seq_lens_cumsum=True)
        b, _ = mod.paged_cache_load(cache, None, table, np.concatenate([[0], inc]),
                                    is_seq_lens_cumsum=True)
        if not (np.array_equal(a, rows) and np.array_equal(b, rows)):
            failed.append("cumsum")
    except (AssertionError, IndexError, ValueError):
        failed.append("cumsum raised")
    return failed


C_MUTANTS = {
    "drop rope term": ("dot += qr[i * d_rope + d] * kr[j * d_rope + d];", "dot += 0.0;"),
    "scale skips rope": ("dot += qr[i * d_rope + d] * kr[j * d_rope + d];",
                         "dot += qr[i * d_rope + d] * kr[j * d_rope + d] / scale;"),
    "mask inside scale": ("scale * dot + m;", "scale * (dot + m);"),
    "top-left causal": ("long p = kvlen - qlen + i;", "long p = i;"),
    "causal off by one": ("return (j <= p) ? 0.0 : -INFINITY;", "return (j < p) ? 0.0 : -INFINITY;"),
    "reversed key feature": ("dot += q[i * d_nope + d] * k[j * d_nope + d];",
                             "dot += q[i * d_nope + d] * k[j * d_nope + (d_nope - 1 - d)];"),
    "reversed value rows": ("o[d] += w * v[j * d_v + d];", "o[d] += w * v[(kvlen - 1 - j) * d_v + d];"),
    "exponent sign": ("exp(s[j] - row_max)", "exp(row_max - s[j])"),
    "no normalisation": ("double w = s[j] / denom;", "double w = s[j];"),
    "diagonal block fully visible": ("if (col_block < row_block)", "if (col_block <= row_block)"),
    "tile transposed": ("tile[(p % ORACLE_TILE) * ORACLE_TILE + (j % ORACLE_TILE)]",
                        "tile[(j % ORACLE_TILE) * ORACLE_TILE + (p % ORACLE_TILE)]"),
}

PY_MUTANTS = {
    "head grouping modulo": ("return h // (head_num // kv_head_num)", "return h % kv_head_num", "attn"),
    "head grouping by kv count": ("return h // (head_num // kv_head_num)", "return h // kv_head_num",
                                  "attn"),
    "slot from block index": ("slots = pos % block_size", "slots = pos // block_size", "gather"),
    "block from slot": ("blocks = block_tables[b, pos // block_size]",
                        "blocks = block_tables[b, pos % block_size]", "gather"),
    "inclusive cumsum off by one": ("spans.append((prev, ctx[b] - prev))",
                                    "spans.append((prev, ctx[b]))", "gather"),
}


@pytest.fixture(scope="module")
def real_pins_pass(oracle_lib):
    assert _attention_pins(oracle, oracle_lib) == []
    assert _gather_pins(oracle) == []
    return True


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(tmp_path, real_pins_pass, name):
    old, new = C_MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(path), "-o", so,
                    "-lm"], check=True)
    lib = oracle.load(so)
    assert _attention_pins(oracle, lib), f"mutant {name!r} passed every pin"


def _mutant_module(tmp_path, old, new):
    src = open(os.path.join(ORACLE_DIR, "__init__.py")).read()
    assert src.count(old) == 1
    d = tmp_path / "mutant_oracle"
    d.mkdir()
    (d / "__init__.py").write_text(src.replace(old, new))
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.c"), d / "oracle.c")
    spec = importlib.util.spec_from_file_location("mutant_oracle", str(d / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_is_caught(tmp_path, real_pins_pass, oracle_lib, name):
    old, new, kind = PY_MUTANTS[name]
    mod = _mutant_module(tmp_path, old, new)
    if kind == "attn":
        assert _attention_pins(mod, oracle_lib), f"mutant {name!r} passed every pin"
    else:
        assert _gather_pins(mod), f"mutant {name!r} passed every pin"
