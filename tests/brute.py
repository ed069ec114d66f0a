"""Float64 brute force for MLA prefill attention, used to pin the C oracle.

Built by a different route from ``oracle/oracle.c`` on purpose:
* queries and keys are concatenated ([Q | QRope], [K | KRope]) and multiplied
  as whole matrices;
* KV heads are expanded with ``np.repeat`` instead of an index formula;
* the mask is materialised as a full [q_len, kv_len] matrix, causal via
  ``np.tril`` with a diagonal offset and MASK_FREE by pasting the 512 x 512
  tile into a block matrix of key-position space.
Follows the "MLA Prefill" page's Members table (Q, QRope, K, kRope, V,
qkScale, Mask, maskType) read as: scale the whole product, then add the mask.
"""
import math

import numpy as np

TILE = 512
UNDEFINED, SPEC, CAUSAL, FREE = 0, 1, 2, 3


def mask_matrix(q_len, kv_len, mask_type, tile=None):
    if mask_type == UNDEFINED:
        return np.zeros((q_len, kv_len))
    if mask_type in (SPEC, CAUSAL):
        keep = np.tril(np.ones((q_len, kv_len), dtype=bool), k=kv_len - q_len)
        return np.where(keep, 0.0, -np.inf)
    assert mask_type == FREE
    nblk = max(1, -(-kv_len // TILE))
    big = np.full((nblk * TILE, nblk * TILE), -np.inf)
    for rb in range(nblk):
        rows = slice(rb * TILE, (rb + 1) * TILE)
        big[rows, : rb * TILE] = 0.0
        big[rows, rb * TILE:(rb + 1) * TILE] = tile
    m = np.full((q_len, kv_len), -np.inf)
    for i in range(q_len):
        p = kv_len - q_len + i
        if p >= 0:
            m[i] = big[p, :kv_len]
    return m


def attention(q, qr, k, kr, v, q_seqlen, kv_seqlen, heads, kv_heads, scale, mask_type, tile=None):
    q_all = np.concatenate([q, qr], axis=-1)
    k_all = np.repeat(np.concatenate([k, kr], axis=-1), heads // kv_heads, axis=1)
    v_all = np.repeat(v, heads // kv_heads, axis=1)
    out = np.zeros((q.shape[0], heads, v.shape[-1]))
    qo = ko = 0
    for ql, kl in zip(q_seqlen, kv_seqlen):
        ql, kl = int(ql), int(kl)
        m = mask_matrix(ql, kl, mask_type, tile)
        for h in range(heads):
            s = scale * (q_all[qo:qo + ql, h] @ k_all[ko:ko + kl, h].T) + m
            for i in range(ql):
                row = s[i]
                if kl == 0 or not np.isfinite(row).any():
                    continue
                e = np.exp(row - row.max())
                out[qo + i, h] = (e / e.sum()) @ v_all[ko:ko + kl, h]
        qo += ql
        ko += kl
    return out


# ---------------------------------------------------------------- MLA prolog
# Float64 brute force of the "MlaProlog" page's formulas (formula section),
# built by another route than oracle.mla_prolog: matrix products as explicit
# loops, the RmsNorm with math.fsum, and the interleaved rope as a complex
# multiplication of (x[2i] + i x[2i+1]) by cos + i sin (cos and sin taken from
# the even element of each pair, which the inputs fill equally).

def _matmul(a, b):
    n, k = len(a), len(b)
    m = len(b[0])
    return [[math.fsum(a[i][kk] * b[kk][j] for kk in range(k)) for j in range(m)] for i in range(n)]


def _rms(row, gamma, eps):
    r = math.sqrt(math.fsum(v * v for v in row) / len(row) + eps)
    return [row[i] / r * (1.0 if gamma is None else gamma[i]) for i in range(len(row))]


def _rope_complex(vals, cos, sin):
    out = []
    for i in range(0, len(vals), 2):
        z = complex(vals[i], vals[i + 1]) * complex(cos[i], sin[i])
        out += [z.real, z.imag]
    return out


def mla_prolog(x, wq_a, wq_b, wkv, cos, sin, gamma_cq, gamma_ckv, num_heads, eps):
    x, wq_a, wq_b, wkv = (np.asarray(a).tolist() for a in (x, wq_a, wq_b, wkv))
    cos, sin = np.asarray(cos).tolist(), np.asarray(sin).tolist()
    gamma_cq, gamma_ckv = np.asarray(gamma_cq).tolist(), np.asarray(gamma_ckv).tolist()
    t, hd, rd = len(x), len(wkv[0]), len(cos[0])
    cq = [_rms(row, gamma_cq, eps) for row in _matmul(x, wq_a)]
    qf = _matmul(cq, wq_b)
    q = np.zeros((t, num_heads, hd))
    for i in range(t):
        for h in range(num_heads):
            head = _rms(qf[i][h * hd:(h + 1) * hd], None, eps)
            q[i, h] = head[:hd - rd] + _rope_complex(head[hd - rd:], cos[i], sin[i])
    kvf = _matmul(x, wkv)
    kv = np.zeros((t, hd))
    for i in range(t):
        row = _rms(kvf[i], gamma_ckv, eps)
        kv[i] = row[:hd - rd] + _rope_complex(row[hd - rd:], cos[i], sin[i])
    return q, kv, np.array(cq)


# Quantised prolog by the same route: c^Q as above, each code by Python's
# round() (ties to even) of c / (max|c| / 127), the product as a sum of Python
# integers, then the dequantisation and the per-head RmsNorm and rope.
def mla_prolog_quant(x, wq_a, wq_b, wkv, cos, sin, gamma_cq, gamma_ckv, wq_b_scale, num_heads, eps):
    x, wq_a, wkv = (np.asarray(a).tolist() for a in (x, wq_a, wkv))
    wq_b = [[int(v) for v in row] for row in np.asarray(wq_b)]
    wsc = [float(v) for v in np.asarray(wq_b_scale).reshape(-1)]
    cos, sin = np.asarray(cos).tolist(), np.asarray(sin).tolist()
    gamma_cq, gamma_ckv = np.asarray(gamma_cq).tolist(), np.asarray(gamma_ckv).tolist()
    t, hd, rd = len(x), len(wkv[0]), len(cos[0])
    cq = [_rms(row, gamma_cq, eps) for row in _matmul(x, wq_a)]
    codes, scales = [], []
    for row in cq:
        s = max(abs(v) for v in row) / 127.0
        scales.append(s)
        codes.append([round(v / s) if s > 0 else 0 for v in row])
    n = len(wq_b[0])
    q = np.zeros((t, num_heads, hd))
    for i in range(t):
        acc = [sum(codes[i][k] * wq_b[k][j] for k in range(len(wq_b))) for j in range(n)]
        y = [acc[j] * scales[i] * wsc[j] for j in range(n)]
        for h in range(num_heads):
            head = _rms(y[h * hd:(h + 1) * hd], None, eps)
            q[i, h] = head[:hd - rd] + _rope_complex(head[hd - rd:], cos[i], sin[i])
    kvf = _matmul(x, wkv)
    kv = np.zeros((t, hd))
    for i in range(t):
        row = _rms(kvf[i], gamma_ckv, eps)
        kv[i] = row[:hd - rd] + _rope_complex(row[hd - rd:], cos[i], sin[i])
    return q, kv, np.array(codes, dtype=np.int64), np.array(scales)
