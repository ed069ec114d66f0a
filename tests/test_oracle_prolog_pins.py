"""Pins of the MLA prolog oracle (``oracle.rms_norm``, ``oracle.rope_interleaved``,
``oracle.mla_prolog``) against things other than itself.

The "MlaProlog" page (formula section) gives c^Q = RmsNorm(x wq_a),
q = RmsNorm(c^Q wq_b) with weight 1, kv = RmsNorm(x wkv), and an interleaved
rope on the last rope_dim values of q and kv. The pins:
  * RmsNorm: torch's ``rms_norm`` as a library special case, the unit mean
    square it produces, invariance to the input's scale, gamma per element;
  * rope: the complex-number form of a rotation of adjacent pairs, a worked
    quarter turn, a pair worked by hand whose two cos/sin entries differ,
    norm preservation and composition of angles;
  * the prolog: a pure-Python brute force (tests/brute.py) on tiny sizes,
    unit norms of every rope'd head, independence of q from the scale of x
    and of gamma_cq (both RmsNorms remove it), no rotation at angle 0.
The quantised prolog (``oracle.quantize_per_token``,
``oracle.mla_prolog_quant``; "MlaProlog" page, mla_prolog_quant) is pinned by
a row quantised by hand (ties to even, a zero row), the brute force by
another route (Python's round and integer sums), the code range, q's
independence of the scale of x and of a head's dequantisation scales, and
the non-quantised prolog on the dequantised inputs within the bound that
rounding the codes allows.
The mutants at the end plant plausible mistakes in a private copy of the
oracle module (rope on split halves, a norm over all heads, a dropped gamma,
a sign flip, rope on the leading values, the odd element of a pair reading
the even element's table entry) and check that some pin fails.
"""
import importlib.util
import math
import os
import shutil

import numpy as np
import pytest
import torch

import brute
import oracle

ORACLE_DIR = os.path.dirname(oracle.__file__)


def rope_tables(t, rd, base=10000.0, offset=0):
    """cos / sin [t, rd] for positions offset .. offset + t - 1, the two
    elements of each pair sharing one angle pos * base^(-2i / rd)."""
    inv = base ** (-np.arange(0, rd, 2) / rd)
    ang = np.repeat((np.arange(t) + offset)[:, None] * inv[None, :], 2, axis=1)
    return np.cos(ang), np.sin(ang)


def tiny_problem(t=3, h=8, r=8, heads=2, hd=8, rd=4, seed=0):
    rng = np.random.default_rng(seed)
    cos, sin = rope_tables(t, rd, offset=5)
    return dict(x=rng.standard_normal((t, h)), wq_a=rng.standard_normal((h, r)) / math.sqrt(h),
                wq_b=rng.standard_normal((r, heads * hd)) / math.sqrt(r),
                wkv=rng.standard_normal((h, hd)) / math.sqrt(h), cos=cos, sin=sin,
                gamma_cq=1 + 0.2 * rng.standard_normal(r), gamma_ckv=1 + 0.2 * rng.standard_normal(hd),
                heads=heads)


def run(mod, p, eps=1e-6, **over):
    p = dict(p, **over)
    return mod.mla_prolog(p["x"], p["wq_a"], p["wq_b"], p["wkv"], p["cos"], p["sin"], p["gamma_cq"],
                          p["gamma_ckv"], p["heads"], eps)


# ------------------------------------------------------------------ pin sets

def rms_pins(mod):
    failed = []
    rng = np.random.default_rng(1)
    y = rng.standard_normal((5, 24)) * 3.0
    g = 1 + 0.3 * rng.standard_normal(24)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(y), (24,), torch.from_numpy(g), eps=1e-6).numpy()
    if not np.allclose(mod.rms_norm(y, g, 1e-6), ref, rtol=1e-12, atol=1e-12):
        failed.append("torch rms_norm")
    out = mod.rms_norm(y, None, 0.0)
    if not np.allclose(np.mean(out * out, axis=-1), 1.0, rtol=1e-12):
        failed.append("unit mean square")
    if not np.allclose(mod.rms_norm(7.5 * y, None, 0.0), out, rtol=1e-12):
        failed.append("scale invariance")
    if not np.allclose(mod.rms_norm(y, g, 0.0) / out, np.broadcast_to(g, y.shape), rtol=1e-12):
        failed.append("gamma per element")
    return failed


def rope_pins(mod):
    failed = []
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 16))
    cos, sin = rope_tables(4, 16, offset=3)
    got = mod.rope_interleaved(x, cos, sin)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * np.arctan2(sin[:, 0::2], cos[:, 0::2]))
    if not np.allclose(got[:, 0::2], z.real, atol=1e-12) or not np.allclose(got[:, 1::2], z.imag, atol=1e-12):
        failed.append("complex rotation")
    # worked example: a quarter turn maps the pair (a, b) to (-b, a)
    quarter = mod.rope_interleaved(np.array([1.0, 2.0, 3.0, 4.0]), np.zeros(4), np.ones(4))
    if not np.allclose(quarter, [-2.0, 1.0, -4.0, 3.0], atol=1e-15):
        failed.append("quarter turn")
    if not np.allclose(np.hypot(got[:, 0::2], got[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]), rtol=1e-12):
        failed.append("pair norms")
    # worked by hand, with the two entries of a pair's cos/sin different (the
    # page's rope_cos / rope_sin have one value per element): the even element
    # takes cos[2i], sin[2i], the odd one cos[2i + 1], sin[2i + 1]
    #   (a, b) = (1, 2), cos = (1/2, 1/4), sin = (3/4, -1/8):
    #   out[0] = 1 * 1/2 - 2 * 3/4    = -1
    #   out[1] = 2 * 1/4 + 1 * (-1/8) = 3/8
    pair = mod.rope_interleaved(np.array([1.0, 2.0]), np.array([0.5, 0.25]), np.array([0.75, -0.125]))
    if not np.array_equal(pair, [-1.0, 0.375]):
        failed.append("pair-unequal tables")
    c2, s2 = rope_tables(4, 16, offset=11)
    ang = np.arctan2(sin, cos) + np.arctan2(s2, c2)
    if not np.allclose(mod.rope_interleaved(got, c2, s2), mod.rope_interleaved(x, np.cos(ang), np.sin(ang)),
                       atol=1e-12):
        failed.append("composition")
    return failed


def prolog_pins(mod):
    failed = []
    p = tiny_problem()
    q, kv, cq = run(mod, p)
    bq, bkv, bcq = brute.mla_prolog(p["x"], p["wq_a"], p["wq_b"], p["wkv"], p["cos"], p["sin"], p["gamma_cq"],
                                    p["gamma_ckv"], p["heads"], 1e-6)
    if not (np.allclose(q, bq, atol=1e-12) and np.allclose(kv, bkv, atol=1e-12) and np.allclose(cq, bcq, atol=1e-12)):
        failed.append("brute force")
    # with eps = 0 every head of q has squared norm head_dim (RmsNorm, then a rotation)
    q0, kv0, _ = run(mod, p, eps=0.0, gamma_ckv=np.ones(8))
    if not np.allclose(np.sum(q0 * q0, axis=-1), 8.0, rtol=1e-12):
        failed.append("q head norms")
    if not np.allclose(np.sum(kv0 * kv0, axis=-1), 8.0, rtol=1e-12):
        failed.append("kv norms")
    # both RmsNorms remove the scale of x; the second removes that of gamma_cq
    q1, kv1, _ = run(mod, p, eps=0.0, x=3.0 * p["x"], gamma_cq=0.25 * p["gamma_cq"])
    q2, kv2, _ = run(mod, p, eps=0.0)
    if not (np.allclose(q1, q2, rtol=1e-10, atol=1e-12) and np.allclose(kv1, kv2, rtol=1e-10, atol=1e-12)):
        failed.append("scale invariance")
    # at angle 0 nothing rotates: q and kv are the plain RmsNorms
    t = p["x"].shape[0]
    qz, kvz, cqz = run(mod, p, cos=np.ones((t, 4)), sin=np.zeros((t, 4)))
    plain_q = (cqz @ p["wq_b"]).reshape(t, 2, 8)
    plain_q = plain_q / np.sqrt(np.mean(plain_q ** 2, axis=-1, keepdims=True) + 1e-6)
    if not np.allclose(qz, plain_q, atol=1e-12):
        failed.append("angle 0")
    return failed


def quant_problem(seed=1, t=4, r=8, heads=2, hd=8):
    p = tiny_problem(t=t, r=r, heads=heads, hd=hd, seed=seed)
    rng = np.random.default_rng(seed + 10)
    p["wq_b8"] = rng.integers(-127, 128, size=(r, heads * hd))
    p["wq_b_scale"] = rng.uniform(0.5, 2.0, size=(heads * hd, 1)) / (127 * math.sqrt(r))
    return p


def run_quant(mod, p, eps=1e-6, **over):
    p = dict(p, **over)
    return mod.mla_prolog_quant(p["x"], p["wq_a"], p["wq_b8"], p["wkv"], p["cos"], p["sin"], p["gamma_cq"],
                                p["gamma_ckv"], p["wq_b_scale"], p["heads"], eps)


def quant_pins(mod):
    failed = []
    # a row worked by hand: max |c| = 254 gives scale 2; -63.5, 2.5 and 1.5
    # round to the even neighbours -64, 2 and 2; a zero row has scale 0
    codes, scale = mod.quantize_per_token(np.array([[254.0, -127.0, 5.0, 0.0, 3.0], [0.0] * 5]))
    if not (np.array_equal(codes, [[127, -64, 2, 0, 2], [0] * 5]) and np.array_equal(scale, [2.0, 0.0])):
        failed.append("hand quantisation")
    p = quant_problem()
    q, kv, qr, sc = run_quant(mod, p)
    bq, bkv, bqr, bsc = brute.mla_prolog_quant(p["x"], p["wq_a"], p["wq_b8"], p["wkv"], p["cos"], p["sin"],
                                               p["gamma_cq"], p["gamma_ckv"], p["wq_b_scale"], p["heads"], 1e-6)
    if not (np.array_equal(qr, bqr) and np.allclose(sc, bsc, rtol=1e-14) and np.allclose(q, bq, atol=1e-12)
            and np.allclose(kv, bkv, atol=1e-12)):
        failed.append("quant brute force")
    if not (np.abs(qr).max() == 127 and (np.abs(qr).max(axis=1) == 127).all()):
        failed.append("code range")
    # q does not depend on the scale of x, nor on a common factor of one
    # head's dequantisation scales (its RmsNorm removes it; eps = 0)
    w2 = p["wq_b_scale"].copy()
    w2[:8] *= 3.0
    q1, _, qr1, _ = run_quant(mod, p, eps=0.0, x=2.0 * p["x"], wq_b_scale=w2)
    q2, _, qr2, _ = run_quant(mod, p, eps=0.0)
    if not (np.array_equal(qr1, qr2) and np.allclose(q1, q2, rtol=1e-10, atol=1e-12)):
        failed.append("quant scale invariance")
    # against the non-quantised prolog on dequantised weights: the codes
    # differ from c^Q / s by at most 1/2, so each product entry moves by at
    # most s * 1/2 * sum_k |wq_b[k, n]| * wq_b_scale[n]
    wdq = p["wq_b8"] * p["wq_b_scale"].reshape(1, -1)
    rq, _, cq = run(mod, p, eps=0.0, wq_b=wdq)
    yq = (qr @ p["wq_b8"]) * sc[:, None] * p["wq_b_scale"].reshape(1, -1)
    yr = cq @ wdq
    bound = 0.5 * sc[:, None] * (np.abs(p["wq_b8"]).sum(axis=0) * p["wq_b_scale"].reshape(-1))[None, :]
    if not (np.abs(yq - yr) <= bound * (1 + 1e-9)).all():
        failed.append("dequantised product bound")
    q0, _, _, _ = run_quant(mod, p, eps=0.0)
    if not np.allclose(q0, rq, atol=0.15):
        failed.append("close to the non-quantised prolog")
    return failed


def test_rms_norm_pins():
    assert rms_pins(oracle) == []


def test_rope_pins():
    assert rope_pins(oracle) == []


def test_prolog_pins():
    assert prolog_pins(oracle) == []


def test_quant_prolog_pins():
    assert quant_pins(oracle) == []


def test_prolog_page_sizes_shapes():
    # the page's sizes (head_dim 512, h 4096, q_lora_rank 1024, 64 heads,
    # rope_dim 64) at t = 2: output shapes and unit head norms
    rng = np.random.default_rng(3)
    t, h, r, heads, hd, rd = 2, 4096, 1024, 64, 512, 64
    cos, sin = rope_tables(t, rd)
    q, kv, cq = oracle.mla_prolog(rng.standard_normal((t, h)), rng.standard_normal((h, r)) / 64,
                                  rng.standard_normal((r, heads * hd)) / 32, rng.standard_normal((h, hd)) / 64,
                                  cos, sin, np.ones(r), np.ones(hd), heads, 0.0)
    assert q.shape == (t, heads, hd) and kv.shape == (t, hd) and cq.shape == (t, r)
    assert np.allclose(np.sum(q * q, axis=-1), hd) and np.allclose(np.sum(kv * kv, axis=-1), hd)


# ------------------------------------------------------------------ mutants

MUTANTS = {
    "rope on split halves": ("partner[..., 0::2] = -x[..., 1::2]\n    partner[..., 1::2] = x[..., 0::2]",
                             "h = x.shape[-1] // 2\n    partner[..., :h] = -x[..., h:]\n    partner[..., h:] = x[..., :h]"),
    "rope sign flipped": ("partner[..., 0::2] = -x[..., 1::2]", "partner[..., 0::2] = x[..., 1::2]"),
    "rms without mean": ("np.mean(y * y, axis=-1, keepdims=True)", "np.sum(y * y, axis=-1, keepdims=True)"),
    "q norm over all heads": ("q = rms_norm((cq @ np.asarray(wq_b, dtype=np.float64)).reshape(t, num_heads, head_dim), None, eps)",
                              "q = rms_norm(cq @ np.asarray(wq_b, dtype=np.float64), None, eps).reshape(t, num_heads, head_dim)"),
    "gamma_ckv dropped": ("kv = rms_norm(x @ np.asarray(wkv, dtype=np.float64), gamma_ckv, eps)",
                          "kv = rms_norm(x @ np.asarray(wkv, dtype=np.float64), None, eps)"),
    "odd element reads the even table entry": ("    return x * cos + partner * sin",
                                               "    return (x * np.repeat(cos[..., 0::2], 2, axis=-1)\n"
                                               "            + partner * np.repeat(sin[..., 0::2], 2, axis=-1))"),
    "rope on leading values": ("kv[:, head_dim - rd:] = rope_interleaved(kv[:, head_dim - rd:], rope_cos, rope_sin)",
                               "kv[:, :rd] = rope_interleaved(kv[:, :rd], rope_cos, rope_sin)"),
}

QUANT_MUTANTS = {
    "ties away from zero": ("np.rint(c / safe[:, None])", "np.sign(c) * np.floor(np.abs(c / safe[:, None]) + 0.5)"),
    "scale over 128": ("scale = np.max(np.abs(c), axis=-1) / 127.0", "scale = np.max(np.abs(c), axis=-1) / 128.0"),
    "codes truncated": ("np.rint(c / safe[:, None])", "np.trunc(c / safe[:, None])"),
    "channel scale dropped": ("y = acc * s[:, None] * np.asarray(wq_b_scale, dtype=np.float64).reshape(1, -1)",
                              "y = acc * s[:, None]"),
    "quantised before gamma": ("    cq = rms_norm(x @ np.asarray(wq_a, dtype=np.float64), gamma_cq, eps)\n    qr, s = quantize_per_token(cq)",
                               "    cq = rms_norm(x @ np.asarray(wq_a, dtype=np.float64), None, eps)\n    qr, s = quantize_per_token(cq)"),
    "quant q norm over all heads": ("    q = rms_norm(y.reshape(t, num_heads, head_dim), None, eps)",
                                    "    q = rms_norm(y, None, eps).reshape(t, num_heads, head_dim)"),
}


def _mutant(tmp_path, old, new):
    src = open(os.path.join(ORACLE_DIR, "__init__.py")).read()
    assert src.count(old) == 1, old
    d = tmp_path / "mutant_prolog"
    d.mkdir()
    (d / "__init__.py").write_text(src.replace(old, new))
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.c"), d / "oracle.c")
    spec = importlib.util.spec_from_file_location("mutant_prolog", str(d / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quant_prolog_mutant_is_caught(tmp_path, name):
    mod = _mutant(tmp_path, *QUANT_MUTANTS[name])
    try:
        failed = quant_pins(mod)
    except (ValueError, IndexError) as e:
        failed = [f"raised {type(e).__name__}"]
    assert failed, f"mutant {name!r} passed every pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prolog_mutant_is_caught(tmp_path, name):
    mod = _mutant(tmp_path, *MUTANTS[name])
    try:
        failed = rms_pins(mod) + rope_pins(mod) + prolog_pins(mod)
    except (ValueError, IndexError) as e:
        failed = [f"raised {type(e).__name__}"]
    assert failed, f"mutant {name!r} passed every pin"
