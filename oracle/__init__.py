"""CPU oracle for MLA varlen prefill and the paged cache gather.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``. The product package never imports
it, and it shares no code, tables or helpers with the HIP path.

* ``attention_head`` / ``attention`` wrap ``oracle.c``: plain fp64 softmax
  attention written from the Ascend Transformer Boost "MLA Prefill" C API page
  (Definition; AtbMLAPreFillGetWorkspaceSize Members table).
* ``paged_cache_load`` is a plain numpy gather written from the Ascend
  Transformer Boost "PagedCacheLoadOperation" page (Members table: keyCache,
  valueCache, blockTables, contextLens, seqStarts, isSeqLensCumsumType,
  hasSeqStarts), ND cache layout.
* ``paged_attention`` is the composition of the two: gather K, KRope and V
  out of ND caches, then attention on the gathered tensors.
* ``paged_cache_load_nz`` is the same gather for the NZ cache layout of the
  "PagedCacheLoadOperation" page's dimension table (keyCache / valueCache /
  key / value rows, NZ column).
* ``rms_norm``, ``rope_interleaved`` and ``mla_prolog`` follow the "MlaProlog"
  page (cann-recipes-infer operator notes: formula section, parameter and
  return lists, constraints), non-quantised: plain numpy in float64, with
  ``numpy.matmul`` as the only library step.

Mask-type codes (the page names the modes but prints no integer values):
UNDEFINED 0, SPEC 1, CAUSAL 2, MASK_FREE 3.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")
# ORACLE_LIBRARY selects another build (the sanitizer build of build_sanitized)
LIB = os.environ.get("ORACLE_LIBRARY") or DEFAULT_LIB
ASAN_LIB = os.path.join(HERE, "liboracle_asan.so")

MASK_UNDEFINED, MASK_SPEC, MASK_CAUSAL, MASK_FREE = 0, 1, 2, 3
MASK_TILE = 512

_lib = None


def build(src: str = SRC, out: str = DEFAULT_LIB) -> str:
    """Compile the C oracle with gcc (IEEE arithmetic: no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def build_sanitized(src: str = SRC, out: str = ASAN_LIB) -> str:
    """The same oracle built with clang under AddressSanitizer and
    UndefinedBehaviorSanitizer (for the sanitizer run of the CPU tests)."""
    clang = os.environ.get("CLANG", "/opt/rocm/llvm/bin/clang")
    cmd = [clang, "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared-libasan", src, "-o", out, "-lm",
           "-Wl,-rpath,/opt/rocm/llvm/lib"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB):
    """Load a compiled oracle library (building it first if it is missing)."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        if path != DEFAULT_LIB:
            raise RuntimeError(f"{path} is missing")
        build(out=path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_long)
    lib.oracle_attention_head.argtypes = [dp, dp, dp, dp, dp, ctypes.c_long, ctypes.c_long,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                          ctypes.c_int, dp, lp, ctypes.c_long, dp, dp]
    lib.oracle_attention_head.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    if path == LIB:
        _lib = lib
    return lib


def num_threads() -> int:
    """Threads the oracle's parallel loops run on (OMP_NUM_THREADS or all cores)."""
    return int(load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the parallel loops the calling thread runs from now on."""
    load().oracle_set_num_threads(int(n))


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attention_head(q, qr, k, kr, v, qk_scale, mask_type, mask=None, rows=None,
                   return_weights=False, lib=None):
    """Attention for one (sequence, query head).

    q [qlen, D], qr [qlen, R], k [kvlen, D], kr [kvlen, R], v [kvlen, Dv]: values
    already converted exactly to float64. ``rows`` selects query rows (default
    all). Query row i sits at key position kvlen - qlen + i. Returns
    out [n_rows, Dv] (and the softmax weights [n_rows, kvlen] if asked).
    """
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    qr = np.ascontiguousarray(qr, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    kr = np.ascontiguousarray(kr, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    qlen, d_nope = q.shape
    kvlen = k.shape[0]
    d_rope = qr.shape[1]
    d_v = v.shape[1]
    assert qr.shape == (qlen, d_rope) and kr.shape == (kvlen, d_rope)
    assert k.shape == (kvlen, d_nope) and v.shape[0] == kvlen
    rows = np.arange(qlen, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), d_v), dtype=np.float64)
    weights = np.zeros((len(rows), kvlen), dtype=np.float64) if return_weights else None
    tile = None
    if mask_type == MASK_FREE:
        tile = np.ascontiguousarray(mask, dtype=np.float64)
        assert tile.shape == (MASK_TILE, MASK_TILE)
    rc = lib.oracle_attention_head(
        _dptr(q), _dptr(qr), _dptr(k), _dptr(kr), _dptr(v), qlen, kvlen, d_nope, d_rope, d_v,
        float(qk_scale), int(mask_type), _dptr(tile) if tile is not None else None,
        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), len(rows), _dptr(out),
        _dptr(weights) if weights is not None else None)
    if rc != 0:
        raise ValueError("oracle_attention_head rejected its arguments")
    return (out, weights) if return_weights else out


def kv_head_of(h: int, head_num: int, kv_head_num: int) -> int:
    """Query head h reads kv head h // (headNum / kvHeadNum): contiguous groups."""
    return h // (head_num // kv_head_num)


def attention(q, qr, k, kr, v, q_seqlen, kv_seqlen, head_num, kv_head_num, qk_scale,
              mask_type, mask=None, kv_padded=False, lib=None):
    """Full varlen problem.

    q [sum qlen, H, D], qr [sum qlen, H, R]; k/kr/v packed [sum kvlen, Hkv, *] or,
    with ``kv_padded``, [batch, max_seq, Hkv, *]. Returns [sum qlen, H, Dv] float64.
    """
    q_seqlen = [int(x) for x in q_seqlen]
    kv_seqlen = [int(x) for x in kv_seqlen]
    assert len(q_seqlen) == len(kv_seqlen)
    assert head_num > 0 and kv_head_num > 0 and head_num % kv_head_num == 0
    d_v = v.shape[-1]
    out = np.zeros((q.shape[0], head_num, d_v), dtype=np.float64)
    qoff = 0
    koff = 0
    for b, (ql, kl) in enumerate(zip(q_seqlen, kv_seqlen)):
        for h in range(head_num):
            hk = kv_head_of(h, head_num, kv_head_num)
            if kv_padded:
                ks, krs, vs = k[b, :kl, hk], kr[b, :kl, hk], v[b, :kl, hk]
            else:
                ks, krs, vs = k[koff:koff + kl, hk], kr[koff:koff + kl, hk], v[koff:koff + kl, hk]
            out[qoff:qoff + ql, h] = attention_head(q[qoff:qoff + ql, h], qr[qoff:qoff + ql, h],
                                                    ks, krs, vs, qk_scale, mask_type, mask, lib=lib)
        qoff += ql
        koff += kl
    return out


def sequence_spans(context_lens, batch, is_cumsum):
    """(offset, length) of each batch's rows in the packed gather output.

    Plain mode: contextLens[b] is the length, offsets are running sums.
    Cumsum mode: contextLens holds running totals, either [batch + 1] with a
    leading 0 or [batch] inclusive totals.
    """
    ctx = [int(x) for x in context_lens]
    spans = []
    if not is_cumsum:
        assert len(ctx) == batch
        off = 0
        for n in ctx:
            spans.append((off, n))
            off += n
    elif len(ctx) == batch + 1:
        spans = [(ctx[b], ctx[b + 1] - ctx[b]) for b in range(batch)]
    else:
        assert len(ctx) == batch
        prev = 0
        for b in range(batch):
            spans.append((prev, ctx[b] - prev))
            prev = ctx[b]
    return spans


def paged_cache_load(key_cache, value_cache, block_tables, context_lens, seq_starts=None,
                     is_seq_lens_cumsum=False, has_seq_starts=False):
    """Gather each sequence's tokens out of a block-paged ND cache.

    key_cache [num_blocks, block_size, heads, head_size_k] (any dtype: a byte
    copy), block_tables [batch, max_blocks] int, context_lens [batch] or
    [batch+1]. Token t of sequence b is cache position s_b + t, which lives in
    block block_tables[b][(s_b + t) // block_size] at slot (s_b + t) % block_size;
    s_b = seq_starts[b] when has_seq_starts, else 0. Returns (key, value); value
    is None when value_cache is None.
    """
    block_tables = np.asarray(block_tables)
    batch = block_tables.shape[0]
    block_size = key_cache.shape[1]
    spans = sequence_spans(context_lens, batch, is_seq_lens_cumsum)
    total = sum(n for _, n in spans)
    key = np.zeros((total,) + key_cache.shape[2:], dtype=key_cache.dtype)
    value = None if value_cache is None else np.zeros((total,) + value_cache.shape[2:], dtype=value_cache.dtype)
    for b, (off, n) in enumerate(spans):
        start = int(seq_starts[b]) if has_seq_starts else 0
        pos = start + np.arange(n)
        blocks = block_tables[b, pos // block_size]
        slots = pos % block_size
        key[off:off + n] = key_cache[blocks, slots]
        if value is not None:
            value[off:off + n] = value_cache[blocks, slots]
    return key, value


def paged_attention(q, qr, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen, head_num,
                    kv_head_num, qk_scale, mask_type, mask=None, lib=None):
    """MLA prefill attention over K, KRope and V kept in block-paged ND caches.

    By definition the gather of each cache ("PagedCacheLoadOperation" page,
    Members table: ND layout, plain contextLens = kv_seqlen, every sequence
    starting at position 0 of its table row) followed by ``attention`` on the
    packed result ("MLA Prefill" page, Definition). Returns [sum qlen, H, Dv]
    float64.
    """
    k, _ = paged_cache_load(key_cache, None, block_tables, kv_seqlen)
    kr, _ = paged_cache_load(krope_cache, None, block_tables, kv_seqlen)
    v, _ = paged_cache_load(value_cache, None, block_tables, kv_seqlen)
    return attention(q, qr, k, kr, v, q_seqlen, kv_seqlen, head_num, kv_head_num, qk_scale, mask_type, mask,
                     lib=lib)


def paged_cache_load_nz(key_cache, value_cache, block_tables, context_lens):
    """Gather out of block-paged caches in the NZ layout.

    The page's dimension table gives the NZ cache as [num_blocks,
    num_heads * head_size // E, block_size, E] (E = 32 for int8, else 16) and
    the gathered tensor as [sum(contextLens), num_heads * head_size]: a token's
    row is cut into chunks of E elements, and chunk c of the token in slot s of
    block k sits at cache[k, c, s, :]. Plain lengths only (the page supports
    seqStarts and cumulative lengths in the ND layout only). Returns
    (key, value); value is None when value_cache is None.
    """
    block_tables = np.asarray(block_tables)
    batch = block_tables.shape[0]
    block_size = key_cache.shape[2]
    spans = sequence_spans(context_lens, batch, False)
    total = sum(n for _, n in spans)

    def gather(cache):
        chunks, elems = cache.shape[1], cache.shape[3]
        out = np.zeros((total, chunks * elems), dtype=cache.dtype)
        for b, (off, n) in enumerate(spans):
            for t in range(n):
                k, s = block_tables[b, t // block_size], t % block_size
                out[off + t] = cache[k, :, s, :].reshape(-1)
        return out

    return gather(key_cache), None if value_cache is None else gather(value_cache)


def rms_norm(y, gamma=None, eps=1e-6):
    """RmsNorm over the last axis ("MlaProlog" page, formula section):
    y / sqrt(mean(y^2) + eps), times gamma when one is given (the page's second
    RmsNorm has weight 1). The page prints neither the formula's body nor eps;
    this is the usual definition, and eps is an argument."""
    y = np.asarray(y, dtype=np.float64)
    out = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return out if gamma is None else out * np.asarray(gamma, dtype=np.float64)


def rope_interleaved(x, cos, sin):
    """Interleaved rotary embedding ("MlaProlog" page, formula section: "inplace
    interleaved rope" of the last rope_dim values). Elements 2i and 2i + 1
    form a pair that is rotated:
        out[2i]     = x[2i]     * cos[2i]     - x[2i + 1] * sin[2i]
        out[2i + 1] = x[2i + 1] * cos[2i + 1] + x[2i]     * sin[2i + 1]
    cos and sin hold one value per element (the page's rope_cos / rope_sin are
    [t, rope_dim]) and broadcast against x."""
    x = np.asarray(x, dtype=np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    partner = np.empty_like(x)
    partner[..., 0::2] = -x[..., 1::2]
    partner[..., 1::2] = x[..., 0::2]
    return x * cos + partner * sin


def prolog_kv(token_x, wkv, rope_cos, rope_sin, gamma_ckv, eps=1e-6):
    """The key-value half of the MLA prolog ("MlaProlog" page, formula
    section), the same in the plain and the quantised operator:
        kv = RmsNorm(x . wkv) * gamma_ckv, kv[..., -rope_dim:] = ROPE(kv[..., -rope_dim:])
    [t, head_dim], float64."""
    x = np.asarray(token_x, dtype=np.float64)
    head_dim = wkv.shape[1]
    rd = rope_cos.shape[1]
    kv = rms_norm(x @ np.asarray(wkv, dtype=np.float64), gamma_ckv, eps)
    kv[:, head_dim - rd:] = rope_interleaved(kv[:, head_dim - rd:], rope_cos, rope_sin)
    return kv


def mla_prolog(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, num_heads, eps=1e-6):
    """The MLA prolog, non-quantised ("MlaProlog" page, formula section; shapes
    from its parameter and return lists):
        c^Q = RmsNorm(x . wq_a) * gamma_cq                       [t, q_lora_rank]
        q   = RmsNorm(c^Q . wq_b), per head over head_dim (weight 1)
        q[..., -rope_dim:]  = ROPE(q[..., -rope_dim:])           [t, num_heads, head_dim]
        kv  = RmsNorm(x . wkv) * gamma_ckv
        kv[..., -rope_dim:] = ROPE(kv[..., -rope_dim:])          [t, head_dim]
    with rope_dim = rope_cos.shape[1] and head_dim = wkv.shape[1]. Everything
    in float64; returns (q, kv, c^Q)."""
    x = np.asarray(token_x, dtype=np.float64)
    t = x.shape[0]
    head_dim = wkv.shape[1]
    rd = rope_cos.shape[1]
    cq = rms_norm(x @ np.asarray(wq_a, dtype=np.float64), gamma_cq, eps)
    q = rms_norm((cq @ np.asarray(wq_b, dtype=np.float64)).reshape(t, num_heads, head_dim), None, eps)
    q[..., head_dim - rd:] = rope_interleaved(q[..., head_dim - rd:], np.asarray(rope_cos)[:, None, :],
                                              np.asarray(rope_sin)[:, None, :])
    kv = prolog_kv(x, wkv, rope_cos, rope_sin, gamma_ckv, eps)
    return q, kv, cq


def quantize_per_token(c):
    """Per-token symmetric int8 quantisation of c^Q ("MlaProlog" page,
    mla_prolog_quant return list: qr_out int8 [t, q_lora_rank] and
    qr_scale_out float32 [t, 1]). The page names these outputs and their types
    only. Reading: a row's scale is its largest magnitude over 127, so that
    c ~ code * scale, and each code is c / scale rounded to the nearest integer
    with ties to even, which keeps it in [-127, 127]; a row of zeros has scale
    0 and codes 0. Returns (codes as int64 [t, r], scale as float64 [t])."""
    c = np.asarray(c, dtype=np.float64)
    scale = np.max(np.abs(c), axis=-1) / 127.0
    safe = np.where(scale > 0, scale, 1.0)
    codes = np.where(scale[:, None] > 0, np.rint(c / safe[:, None]), 0.0)
    return codes.astype(np.int64), scale


def mla_prolog_quant(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, num_heads,
                     eps=1e-6):
    """The quantised MLA prolog ("MlaProlog" page, mla_prolog_quant: wq_b is
    int8 [q_lora_rank, num_heads * head_dim] with the per-channel
    dequantisation scale wq_b_scale [num_heads * head_dim, 1]; c^Q leaves as
    int8 codes plus a per-token scale):
        c^Q      = RmsNorm(x . wq_a) * gamma_cq
        (qr, s)  = quantize_per_token(c^Q)                       [t, q_lora_rank], [t]
        q        = RmsNorm((qr . wq_b) * s[t] * wq_b_scale[n]), per head (weight 1)
        q[..., -rope_dim:] = ROPE(q[..., -rope_dim:])
        kv       as in mla_prolog
    The product qr . wq_b is taken exactly: both factors hold integers of
    magnitude at most 128, so every partial sum is an integer far below 2^53
    and a float64 product cannot round. Returns (q, kv, qr, s), q and kv in
    float64."""
    x = np.asarray(token_x, dtype=np.float64)
    t = x.shape[0]
    head_dim = wkv.shape[1]
    rd = rope_cos.shape[1]
    cq = rms_norm(x @ np.asarray(wq_a, dtype=np.float64), gamma_cq, eps)
    qr, s = quantize_per_token(cq)
    w8 = np.asarray(wq_b, dtype=np.float64)
    assert qr.shape[1] * 128 * 128 < 2 ** 53 and np.abs(w8).max(initial=0) <= 128
    acc = qr.astype(np.float64) @ w8
    y = acc * s[:, None] * np.asarray(wq_b_scale, dtype=np.float64).reshape(1, -1)
    q = rms_norm(y.reshape(t, num_heads, head_dim), None, eps)
    q[..., head_dim - rd:] = rope_interleaved(q[..., head_dim - rd:], np.asarray(rope_cos)[:, None, :],
                                              np.asarray(rope_sin)[:, None, :])
    kv = prolog_kv(x, wkv, rope_cos, rope_sin, gamma_ckv, eps)
    return q, kv, qr, s
