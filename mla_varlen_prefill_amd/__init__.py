"""MLA varlen prefill on MI355X (gfx950): Python binding of the C ABI.

The functions below carry the names of the C entry points declared in
``include/mla_prefill.h`` and only marshal arguments: torch tensors become
``mla_tensor`` descriptors (data pointer, dtype code, shape), host length
arrays are passed as int32 pointers, and the current torch stream is passed as
the HIP stream. Every step of the computation runs in the HIP library
``libmla_prefill.so`` built from ``csrc/``; there is no other code path, and a
missing library is an error.

``prefill`` is a convenience wrapper that allocates the output and the
workspace with torch and calls the two-phase pair.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "MASK_UNDEFINED", "MASK_SPEC", "MASK_CAUSAL", "MASK_FREE", "KV_CACHE_NZ", "KV_CACHE_ND",
    "MlaError", "mla_prefill_get_workspace_size", "mla_prefill", "paged_cache_load",
    "mla_last_error", "mla_prefill_plan_host", "prefill", "library_path",
    "mla_prefill_paged_get_workspace_size", "mla_prefill_paged", "prefill_paged",
    "mla_prolog_get_workspace_size", "mla_prolog", "prolog",
    "mla_prolog_quant_get_workspace_size", "mla_prolog_quant", "prolog_quant",
    "mla_prolog_weights_size", "mla_prolog_pack_weights", "mla_prolog_prepacked_workspace_size",
    "mla_prolog_prepacked", "mla_prolog_quant_prepacked", "pack_prolog_weights",
]

# MLA_PREFILL_LIBRARY selects another build of the same library (the host
# sanitizer build of build.py is run this way).
LIB_PATH = os.environ.get("MLA_PREFILL_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                                  "libmla_prefill.so")

MASK_UNDEFINED, MASK_SPEC, MASK_CAUSAL, MASK_FREE = 0, 1, 2, 3
KV_CACHE_NZ, KV_CACHE_ND = 0, 1
PLAN_Q_ROWS, PLAN_KV_COLS = 256, 64
PAGED_MAX_KEYS = 2048 * 64

STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_VALUE", -5: "MLA_ERR_UNSUPPORTED", -6: "MLA_ERR_WORKSPACE",
          -7: "MLA_ERR_RUNTIME"}

_DTYPE = {torch.float16: 1, torch.bfloat16: 2, torch.int8: 3, torch.int32: 4, torch.float32: 5,
          np.dtype(np.int32): 4, np.dtype(np.int8): 3, np.dtype(np.float16): 1, np.dtype(np.float32): 5}


class MlaError(RuntimeError):
    """A C entry point returned a non-zero status."""

    def __init__(self, fn, code, message):
        self.code = code
        self.status = STATUS.get(code, str(code))
        super().__init__(f"{fn}: {self.status}: {message}")


class MlaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_varlen_prefill_amd.build`"
                           " (there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    T = ctypes.POINTER(MlaTensor)
    lib.mla_prefill_get_workspace_size.argtypes = [T, T, T, T, T, T, T, T, ctypes.c_int32, ctypes.c_float,
                                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_uint8, T,
                                                   ctypes.POINTER(ctypes.c_uint64)]
    lib.mla_prefill.argtypes = [T, T, T, T, T, T, T, T, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_uint8, T, ctypes.c_void_p, ctypes.c_uint64,
                                ctypes.c_void_p]
    lib.mla_prefill_no_alloc.argtypes = [T, T, T, T, T, T, T, T, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_uint8, T, ctypes.c_void_p]
    lib.paged_cache_load.argtypes = [T, T, T, T, T, T, T, ctypes.c_int8, ctypes.c_bool, ctypes.c_bool,
                                     ctypes.c_void_p]
    lib.mla_prefill_paged_get_workspace_size.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int32, ctypes.c_float,
                                                         ctypes.c_int32, ctypes.c_int32, T,
                                                         ctypes.POINTER(ctypes.c_uint64)]
    lib.mla_prefill_paged.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                      ctypes.c_int32, T, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.mla_prolog_get_workspace_size.argtypes = [T] * 8 + [ctypes.c_float, T, T, T,
                                                             ctypes.POINTER(ctypes.c_uint64)]
    lib.mla_prolog.argtypes = [T] * 8 + [ctypes.c_float, T, T, T, ctypes.c_void_p, ctypes.c_uint64,
                                         ctypes.c_void_p]
    lib.mla_prolog_quant_get_workspace_size.argtypes = [T] * 9 + [ctypes.c_float, T, T, T, T,
                                                                   ctypes.POINTER(ctypes.c_uint64)]
    lib.mla_prolog_quant.argtypes = [T] * 9 + [ctypes.c_float, T, T, T, T, ctypes.c_void_p, ctypes.c_uint64,
                                               ctypes.c_void_p]
    lib.mla_prolog_weights_size.argtypes = [T, T, T, ctypes.POINTER(ctypes.c_uint64)]
    lib.mla_prolog_pack_weights.argtypes = [T, T, T, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.mla_prolog_prepacked_workspace_size.argtypes = [T, T, ctypes.POINTER(ctypes.c_uint64)]
    lib.mla_prolog_prepacked.argtypes = [T] * 8 + [ctypes.c_float, T, T, T, ctypes.c_void_p, ctypes.c_uint64,
                                                   ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.mla_prolog_quant_prepacked.argtypes = [T] * 9 + [ctypes.c_float, T, T, T, T, ctypes.c_void_p,
                                                         ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                                         ctypes.c_void_p]
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_prefill_plan_host.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_uint64, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32)]
    for fn in ("mla_prefill_get_workspace_size", "mla_prefill", "mla_prefill_no_alloc", "paged_cache_load",
               "mla_prefill_plan_host",
               "mla_prefill_paged_get_workspace_size", "mla_prefill_paged", "mla_prolog_get_workspace_size",
               "mla_prolog", "mla_prolog_quant_get_workspace_size", "mla_prolog_quant", "mla_prolog_weights_size",
               "mla_prolog_pack_weights", "mla_prolog_prepacked_workspace_size", "mla_prolog_prepacked",
               "mla_prolog_quant_prepacked"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def mla_last_error() -> str:
    return _load().mla_last_error().decode()


def _check(fn, rc):
    if rc != 0:
        raise MlaError(fn, rc, mla_last_error())


def _on_device(named, stream=None):
    """Raise ValueError unless every (name, tensor) pair that is not None is a
    torch tensor in GPU memory, all on one device (the stream's, when a torch
    stream is given). The C entry points take raw pointers and cannot tell host
    memory from device memory; a host pointer handed to a kernel faults the
    GPU, so this is checked before any launching call."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            kind = type(t).__name__ if not isinstance(t, torch.Tensor) else f"tensor on {t.device}"
            raise ValueError(f"{name} must be a torch tensor in GPU memory (got {kind})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other device arguments on {dev}")
    if dev is not None and isinstance(stream, torch.cuda.Stream) and stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")


def _desc(t, keep):
    """mla_tensor descriptor of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("host arrays must be C-contiguous")
        keep.append(t)
        ptr, shape, dt = t.ctypes.data, t.shape, _DTYPE.get(t.dtype, 0)
    else:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (row-major)")
        ptr, shape, dt = t.data_ptr(), tuple(t.shape), _DTYPE.get(t.dtype, 0)
    if len(shape) > 4:
        raise ValueError("at most 4 dimensions")
    d = MlaTensor()
    d.data = ptr if ptr else None
    d.dtype = dt
    d.ndim = len(shape)
    for i, s in enumerate(shape):
        d.shape[i] = int(s)
    keep.append(d)
    return ctypes.pointer(d)


def _host_int32(x):
    """Host int32 array of lengths (list, numpy array or CPU tensor)."""
    if isinstance(x, torch.Tensor):
        if x.is_cuda:
            raise ValueError("q_seqlen / kv_seqlen are host arrays")
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _stream_ptr(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _prefill_args(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                  mask_type, cache_mode, atten_out, keep):
    qs, ks = _host_int32(q_seqlen), _host_int32(kv_seqlen)
    return [_desc(q, keep), _desc(q_rope, keep), _desc(k, keep), _desc(k_rope, keep), _desc(v, keep),
            _desc(qs, keep), _desc(ks, keep), _desc(mask, keep), int(head_num), float(qk_scale),
            int(kv_head_num), int(mask_type), int(cache_mode), _desc(atten_out, keep)]


def mla_prefill_get_workspace_size(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale,
                                   kv_head_num, mask_type, cache_mode, atten_out) -> int:
    """Bytes of device workspace ``mla_prefill`` needs (host-only planning call)."""
    lib = _load()
    keep = []
    args = _prefill_args(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                         mask_type, cache_mode, atten_out, keep)
    size = ctypes.c_uint64(0)
    _check("mla_prefill_get_workspace_size", lib.mla_prefill_get_workspace_size(*args, ctypes.byref(size)))
    return int(size.value)


def mla_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                mask_type, cache_mode, atten_out, workspace, stream=None) -> None:
    """Enqueue MLA prefill attention on ``stream`` (default: torch's current stream)."""
    lib = _load()
    _on_device([("q", q), ("q_rope", q_rope), ("k", k), ("k_rope", k_rope), ("v", v), ("atten_out", atten_out),
                ("mask", mask if mask_type == MASK_FREE else None), ("workspace", workspace)], stream)
    keep = []
    args = _prefill_args(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                         mask_type, cache_mode, atten_out, keep)
    ws_ptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    ws_size = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_prefill", lib.mla_prefill(*args, ctypes.c_void_p(ws_ptr), ctypes.c_uint64(ws_size),
                                          _stream_ptr(stream)))


def mla_prefill_no_alloc(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                         mask_type, cache_mode, atten_out, stream=None) -> None:
    """``mla_prefill`` without a workspace: the work list goes into the
    library's fixed per-GPU array (``MLA_NO_ALLOC_WORKSPACE_BYTES``), so the
    call allocates no device memory. Calls that overlap on one GPU race."""
    lib = _load()
    _on_device([("q", q), ("q_rope", q_rope), ("k", k), ("k_rope", k_rope), ("v", v), ("atten_out", atten_out),
                ("mask", mask if mask_type == MASK_FREE else None)], stream)
    keep = []
    args = _prefill_args(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                         mask_type, cache_mode, atten_out, keep)
    _check("mla_prefill_no_alloc", lib.mla_prefill_no_alloc(*args, _stream_ptr(stream)))


def _paged_args(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen, mask, head_num,
                qk_scale, kv_head_num, mask_type, atten_out, keep):
    qs, ks = _host_int32(q_seqlen), _host_int32(kv_seqlen)
    return [_desc(q, keep), _desc(q_rope, keep), _desc(key_cache, keep), _desc(krope_cache, keep),
            _desc(value_cache, keep), _desc(block_tables, keep), _desc(qs, keep), _desc(ks, keep),
            _desc(mask, keep), int(head_num), float(qk_scale), int(kv_head_num), int(mask_type),
            _desc(atten_out, keep)]


def mla_prefill_paged_get_workspace_size(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen,
                                         kv_seqlen, mask, head_num, qk_scale, kv_head_num, mask_type,
                                         atten_out) -> int:
    """Bytes of device workspace ``mla_prefill_paged`` needs (host-only planning call)."""
    lib = _load()
    keep = []
    args = _paged_args(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen, mask,
                       head_num, qk_scale, kv_head_num, mask_type, atten_out, keep)
    size = ctypes.c_uint64(0)
    _check("mla_prefill_paged_get_workspace_size",
           lib.mla_prefill_paged_get_workspace_size(*args, ctypes.byref(size)))
    return int(size.value)


def mla_prefill_paged(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen, mask,
                      head_num, qk_scale, kv_head_num, mask_type, atten_out, workspace, stream=None) -> None:
    """Enqueue MLA prefill attention reading K, KRope and V through block tables."""
    lib = _load()
    _on_device([("q", q), ("q_rope", q_rope), ("key_cache", key_cache), ("krope_cache", krope_cache),
                ("value_cache", value_cache), ("block_tables", block_tables), ("atten_out", atten_out),
                ("mask", mask if mask_type == MASK_FREE else None), ("workspace", workspace)], stream)
    keep = []
    args = _paged_args(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen, mask,
                       head_num, qk_scale, kv_head_num, mask_type, atten_out, keep)
    ws_ptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    ws_size = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_prefill_paged", lib.mla_prefill_paged(*args, ctypes.c_void_p(ws_ptr), ctypes.c_uint64(ws_size),
                                                      _stream_ptr(stream)))


def paged_cache_load(key_cache, value_cache, block_tables, context_lens, key, value, seq_starts=None,
                     kv_cache_cfg=KV_CACHE_ND, is_seq_lens_cumsum_type=False, has_seq_starts=False,
                     stream=None) -> None:
    """Enqueue the paged K/V gather on ``stream`` (default: torch's current stream).
    Every tensor argument, context_lens and seq_starts included, is device memory."""
    lib = _load()
    _on_device([("key_cache", key_cache), ("value_cache", value_cache), ("block_tables", block_tables),
                ("context_lens", context_lens), ("key", key), ("value", value),
                ("seq_starts", seq_starts if has_seq_starts else None)], stream)
    keep = []
    _check("paged_cache_load", lib.paged_cache_load(
        _desc(key_cache, keep), _desc(value_cache, keep), _desc(block_tables, keep), _desc(context_lens, keep),
        _desc(key, keep), _desc(value, keep), _desc(seq_starts, keep), int(kv_cache_cfg),
        bool(is_seq_lens_cumsum_type), bool(has_seq_starts), _stream_ptr(stream)))


def mla_prefill_plan_host(q_seqlen, kv_seqlen, head_num, kv_head_num, mask_type, kv_padded_max_seq=0):
    """The work list mla_prefill would copy to its workspace, decoded.

    Returns (seqs [batch, 4] int32 = q_offset, kv_offset, q_len, kv_len;
    items [n, 4] int32 = batch, first_q_row, kv_tiles, q_rows;
    tasks [m, 4] int32 = item (-1: padding), first head, first tile, end tile
    -- task i is workgroup i and runs PLAN_Q_ROWS // q_rows heads from its
    first head over key tiles [first tile, end tile) of the item; an item cut
    into several such runs is merged after the attention launch).
    """
    lib = _load()
    qs, ks = _host_int32(q_seqlen), _host_int32(kv_seqlen)
    batch = len(qs)
    n_items, n_tasks = ctypes.c_int32(0), ctypes.c_int32(0)
    args = (qs.ctypes.data, ks.ctypes.data, batch, int(head_num), int(kv_head_num), int(mask_type),
            int(kv_padded_max_seq))
    rc = lib.mla_prefill_plan_host(*args, None, 0, ctypes.byref(n_items), ctypes.byref(n_tasks))
    if rc not in (0, -6):  # -6: buffer too small, counts are filled in
        _check("mla_prefill_plan_host", rc)

    def up(x):
        return (x + 255) // 256 * 256

    off_items = up(batch * 16)
    off_tasks = off_items + up(n_items.value * 16)
    buf = np.zeros(max(1, off_tasks + n_tasks.value * 16), dtype=np.uint8)
    _check("mla_prefill_plan_host", lib.mla_prefill_plan_host(*args, buf.ctypes.data, buf.nbytes,
                                                              ctypes.byref(n_items), ctypes.byref(n_tasks)))
    seqs = buf[:batch * 16].view(np.int32).reshape(batch, 4).copy()
    items = buf[off_items:off_items + n_items.value * 16].view(np.int32).reshape(n_items.value, 4).copy()
    tasks = buf[off_tasks:off_tasks + n_tasks.value * 16].view(np.int32).reshape(n_tasks.value, 4).copy()
    return seqs, items, tasks


def prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, head_num, kv_head_num, qk_scale=1.0,
            mask_type=MASK_UNDEFINED, mask=None, out=None, stream=None):
    """Allocate the output and workspace with torch and run the two-phase pair."""
    if out is None:
        d = q.shape[-1] if q.dim() == 3 else q.shape[1] // head_num
        out = torch.empty((q.shape[0], head_num, d), dtype=q.dtype, device=q.device)
    ws = mla_prefill_get_workspace_size(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale,
                                        kv_head_num, mask_type, 0, out)
    workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
    mla_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num, mask_type,
                0, out, workspace, stream)
    if stream is not None and isinstance(stream, torch.cuda.Stream):
        workspace.record_stream(stream)
    return out


def prefill_paged(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen, head_num,
                  kv_head_num, qk_scale=1.0, mask_type=MASK_UNDEFINED, mask=None, out=None, stream=None):
    """Paged form of ``prefill``: allocate output and workspace, run the two-phase pair."""
    if out is None:
        d = q.shape[-1] if q.dim() == 3 else q.shape[1] // head_num
        out = torch.empty((q.shape[0], head_num, d), dtype=q.dtype, device=q.device)
    ws = mla_prefill_paged_get_workspace_size(q, q_rope, key_cache, krope_cache, value_cache, block_tables,
                                              q_seqlen, kv_seqlen, mask, head_num, qk_scale, kv_head_num,
                                              mask_type, out)
    workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
    mla_prefill_paged(q, q_rope, key_cache, krope_cache, value_cache, block_tables, q_seqlen, kv_seqlen, mask,
                      head_num, qk_scale, kv_head_num, mask_type, out, workspace, stream)
    if stream is not None and isinstance(stream, torch.cuda.Stream):
        workspace.record_stream(stream)
    return out


def _prolog_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out, qr_out,
                 keep):
    return ([_desc(x, keep) for x in (token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv)]
            + [ctypes.c_float(eps)] + [_desc(x, keep) for x in (q_out, kv_out, qr_out)])


def mla_prolog_get_workspace_size(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out,
                                  kv_out, qr_out) -> int:
    """Bytes of device workspace ``mla_prolog`` needs for these shapes."""
    lib = _load()
    keep = []
    size = ctypes.c_uint64(0)
    _check("mla_prolog_get_workspace_size", lib.mla_prolog_get_workspace_size(
        *_prolog_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out, qr_out,
                      keep), ctypes.byref(size)))
    return int(size.value)


def mla_prolog(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out, qr_out,
               workspace, stream=None) -> None:
    """Enqueue the non-quantised MLA prolog (q, kv and c^Q from hidden states)."""
    lib = _load()
    _on_device([("token_x", token_x), ("wq_a", wq_a), ("wq_b", wq_b), ("wkv", wkv), ("rope_cos", rope_cos),
                ("rope_sin", rope_sin), ("gamma_cq", gamma_cq), ("gamma_ckv", gamma_ckv), ("q_out", q_out),
                ("kv_out", kv_out), ("qr_out", qr_out), ("workspace", workspace)], stream)
    keep = []
    ws_ptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    ws_size = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_prolog", lib.mla_prolog(
        *_prolog_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out, qr_out,
                      keep), ctypes.c_void_p(ws_ptr), ctypes.c_uint64(ws_size), _stream_ptr(stream)))


def prolog(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps=1e-6, stream=None, packed=None):
    """Allocate outputs and workspace with torch and run the prolog. Returns
    (q [t, num_heads, head_dim], kv [t, head_dim], c^Q [t, q_lora_rank]).
    With ``packed`` (``pack_prolog_weights`` of these weights) the weights are
    not rearranged again."""
    t, hd, r = token_x.shape[0], wkv.shape[1], wq_a.shape[1]
    heads = wq_b.shape[1] // hd
    dev = token_x.device
    q = torch.empty((t, heads, hd), dtype=torch.bfloat16, device=dev)
    kv = torch.empty((t, hd), dtype=torch.bfloat16, device=dev)
    cq = torch.empty((t, r), dtype=torch.bfloat16, device=dev)
    if packed is not None:
        ws = mla_prolog_prepacked_workspace_size(token_x, wq_a)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        mla_prolog_prepacked(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q, kv, cq, packed,
                             workspace, stream)
    else:
        ws = mla_prolog_get_workspace_size(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q,
                                           kv, cq)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        mla_prolog(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q, kv, cq, workspace,
                   stream)
    if stream is not None and isinstance(stream, torch.cuda.Stream):
        workspace.record_stream(stream)
    return q, kv, cq


def _prolog_quant_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps, q_out,
                       kv_out, qr_out, qr_scale_out, keep):
    return ([_desc(x, keep) for x in (token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale)]
            + [ctypes.c_float(eps)] + [_desc(x, keep) for x in (q_out, kv_out, qr_out, qr_scale_out)])


def mla_prolog_quant_get_workspace_size(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv,
                                        wq_b_scale, eps, q_out, kv_out, qr_out, qr_scale_out) -> int:
    """Bytes of device workspace ``mla_prolog_quant`` needs for these shapes."""
    lib = _load()
    keep = []
    size = ctypes.c_uint64(0)
    _check("mla_prolog_quant_get_workspace_size", lib.mla_prolog_quant_get_workspace_size(
        *_prolog_quant_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps,
                            q_out, kv_out, qr_out, qr_scale_out, keep), ctypes.byref(size)))
    return int(size.value)


def mla_prolog_quant(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps, q_out,
                     kv_out, qr_out, qr_scale_out, workspace, stream=None) -> None:
    """Enqueue the quantised MLA prolog: int8 wq_b with per-column scales;
    q, kv, and c^Q as int8 codes with a per-token scale."""
    lib = _load()
    _on_device([("token_x", token_x), ("wq_a", wq_a), ("wq_b", wq_b), ("wkv", wkv), ("rope_cos", rope_cos),
                ("rope_sin", rope_sin), ("gamma_cq", gamma_cq), ("gamma_ckv", gamma_ckv),
                ("wq_b_scale", wq_b_scale), ("q_out", q_out), ("kv_out", kv_out), ("qr_out", qr_out),
                ("qr_scale_out", qr_scale_out), ("workspace", workspace)], stream)
    keep = []
    ws_ptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    ws_size = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_prolog_quant", lib.mla_prolog_quant(
        *_prolog_quant_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps,
                            q_out, kv_out, qr_out, qr_scale_out, keep),
        ctypes.c_void_p(ws_ptr), ctypes.c_uint64(ws_size), _stream_ptr(stream)))


def prolog_quant(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps=1e-6,
                 stream=None, packed=None):
    """Allocate outputs and workspace with torch and run the quantised prolog.
    Returns (q [t, num_heads, head_dim] bf16, kv [t, head_dim] bf16,
    c^Q codes [t, q_lora_rank] int8, c^Q scales [t, 1] float32). With
    ``packed`` (``pack_prolog_weights`` of these weights) the weights are not
    rearranged again."""
    t, hd, r = token_x.shape[0], wkv.shape[1], wq_a.shape[1]
    heads = wq_b.shape[1] // hd
    dev = token_x.device
    q = torch.empty((t, heads, hd), dtype=torch.bfloat16, device=dev)
    kv = torch.empty((t, hd), dtype=torch.bfloat16, device=dev)
    qr = torch.empty((t, r), dtype=torch.int8, device=dev)
    qs = torch.empty((t, 1), dtype=torch.float32, device=dev)
    if packed is not None:
        ws = mla_prolog_prepacked_workspace_size(token_x, wq_a)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        mla_prolog_quant_prepacked(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps,
                                   q, kv, qr, qs, packed, workspace, stream)
    else:
        ws = mla_prolog_quant_get_workspace_size(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv,
                                                 wq_b_scale, eps, q, kv, qr, qs)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        mla_prolog_quant(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps, q, kv,
                         qr, qs, workspace, stream)
    if stream is not None and isinstance(stream, torch.cuda.Stream):
        workspace.record_stream(stream)
    return q, kv, qr, qs


def _buf(t):
    """(pointer or None, size in bytes) of an optional device buffer tensor."""
    if t is None:
        return None, 0
    return (t.data_ptr() if t.numel() else None), t.numel() * t.element_size()


def mla_prolog_weights_size(wq_a, wq_b, wkv) -> int:
    """Bytes of the packed prolog weights (bf16 or int8 wq_b)."""
    lib = _load()
    keep = []
    size = ctypes.c_uint64(0)
    _check("mla_prolog_weights_size", lib.mla_prolog_weights_size(_desc(wq_a, keep), _desc(wq_b, keep),
                                                                   _desc(wkv, keep), ctypes.byref(size)))
    return int(size.value)


def mla_prolog_pack_weights(wq_a, wq_b, wkv, packed, stream=None) -> None:
    """Enqueue the rearrangement of the three prolog weights into ``packed``."""
    lib = _load()
    _on_device([("wq_a", wq_a), ("wq_b", wq_b), ("wkv", wkv), ("packed", packed)], stream)
    keep = []
    ptr, size = _buf(packed)
    _check("mla_prolog_pack_weights", lib.mla_prolog_pack_weights(
        _desc(wq_a, keep), _desc(wq_b, keep), _desc(wkv, keep), ctypes.c_void_p(ptr), ctypes.c_uint64(size),
        _stream_ptr(stream)))


def pack_prolog_weights(wq_a, wq_b, wkv, stream=None):
    """Allocate (torch) and fill the packed prolog weights; reuse the result
    for every call with these weights."""
    packed = torch.empty(max(mla_prolog_weights_size(wq_a, wq_b, wkv), 1), dtype=torch.uint8, device=wq_a.device)
    mla_prolog_pack_weights(wq_a, wq_b, wkv, packed, stream)
    return packed


def mla_prolog_prepacked_workspace_size(token_x, wq_a) -> int:
    """Workspace bytes of the prepacked prolog operators for these shapes."""
    lib = _load()
    keep = []
    size = ctypes.c_uint64(0)
    _check("mla_prolog_prepacked_workspace_size", lib.mla_prolog_prepacked_workspace_size(
        _desc(token_x, keep), _desc(wq_a, keep), ctypes.byref(size)))
    return int(size.value)


def mla_prolog_prepacked(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out,
                         qr_out, packed, workspace, stream=None) -> None:
    """``mla_prolog`` reading the weights from ``packed`` (mla_prolog_pack_weights)."""
    lib = _load()
    _on_device([("token_x", token_x), ("wq_a", wq_a), ("wq_b", wq_b), ("wkv", wkv), ("rope_cos", rope_cos),
                ("rope_sin", rope_sin), ("gamma_cq", gamma_cq), ("gamma_ckv", gamma_ckv), ("q_out", q_out),
                ("kv_out", kv_out), ("qr_out", qr_out), ("packed", packed), ("workspace", workspace)], stream)
    keep = []
    pk, pk_size = _buf(packed)
    ws, ws_size = _buf(workspace)
    _check("mla_prolog_prepacked", lib.mla_prolog_prepacked(
        *_prolog_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, eps, q_out, kv_out, qr_out,
                      keep), ctypes.c_void_p(pk), ctypes.c_uint64(pk_size), ctypes.c_void_p(ws),
        ctypes.c_uint64(ws_size), _stream_ptr(stream)))


def mla_prolog_quant_prepacked(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps,
                               q_out, kv_out, qr_out, qr_scale_out, packed, workspace, stream=None) -> None:
    """``mla_prolog_quant`` reading the weights from ``packed`` (mla_prolog_pack_weights)."""
    lib = _load()
    _on_device([("token_x", token_x), ("wq_a", wq_a), ("wq_b", wq_b), ("wkv", wkv), ("rope_cos", rope_cos),
                ("rope_sin", rope_sin), ("gamma_cq", gamma_cq), ("gamma_ckv", gamma_ckv),
                ("wq_b_scale", wq_b_scale), ("q_out", q_out), ("kv_out", kv_out), ("qr_out", qr_out),
                ("qr_scale_out", qr_scale_out), ("packed", packed), ("workspace", workspace)], stream)
    keep = []
    pk, pk_size = _buf(packed)
    ws, ws_size = _buf(workspace)
    _check("mla_prolog_quant_prepacked", lib.mla_prolog_quant_prepacked(
        *_prolog_quant_args(token_x, wq_a, wq_b, wkv, rope_cos, rope_sin, gamma_cq, gamma_ckv, wq_b_scale, eps,
                            q_out, kv_out, qr_out, qr_scale_out, keep),
        ctypes.c_void_p(pk), ctypes.c_uint64(pk_size), ctypes.c_void_p(ws), ctypes.c_uint64(ws_size),
        _stream_ptr(stream)))
