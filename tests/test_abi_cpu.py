"""Host-side tests of the C ABI: exports, validation, the work planner.

These run without a GPU: every call here either fails validation before any
HIP call, or only plans on the host.
"""
import ctypes
import glob
import json
import os
import re

import numpy as np
import pytest
import torch

import mla_varlen_prefill_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_contract.json")


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M):
            names.append(m.group(1))
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"mla_prefill_get_workspace_size", "mla_prefill", "paged_cache_load"} <= set(names)
    lib = ctypes.CDLL(mla.library_path())
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_binding_uses_the_c_names():
    for n in declared_functions():
        assert callable(getattr(mla, n, None)), f"binding lacks {n}"


# ------------------------------------------------------------------ validation

def tensors(qs=(17, 40), ks=None, h=4, hk=4, d=128, dtype=torch.bfloat16):
    ks = qs if ks is None else ks
    nq, nk = sum(qs), sum(ks)
    z = lambda *s, dt=dtype: torch.zeros(s, dtype=dt)
    return dict(q=z(nq, h, d), q_rope=z(nq, h, 64), k=z(nk, hk, d), k_rope=z(nk, hk, 64), v=z(nk, hk, d),
                q_seqlen=np.array(qs, np.int32), kv_seqlen=np.array(ks, np.int32), mask=None, head_num=h,
                qk_scale=0.1, kv_head_num=hk, mask_type=mla.MASK_CAUSAL, cache_mode=0, atten_out=z(nq, h, d))


def ws_size(t):
    return mla.mla_prefill_get_workspace_size(**t)


def status_of(t):
    try:
        ws_size(t)
        return "MLA_OK"
    except mla.MlaError as e:
        return e.status


def test_valid_problem_plans():
    assert ws_size(tensors()) > 0
    assert ws_size(tensors(qs=(0, 0), ks=(5, 0))) == 0  # no query rows: nothing to do


@pytest.mark.parametrize("mutate,status", [
    (lambda t: t.update(head_num=0), "MLA_ERR_VALUE"),                      # page default 0 is invalid
    (lambda t: t.update(kv_head_num=0), "MLA_ERR_VALUE"),
    (lambda t: t.update(kv_head_num=3), "MLA_ERR_VALUE"),                   # 4 % 3 != 0
    (lambda t: t.update(qk_scale=float("nan")), "MLA_ERR_VALUE"),
    (lambda t: t.update(mask_type=7), "MLA_ERR_VALUE"),
    (lambda t: t.update(cache_mode=1), "MLA_ERR_UNSUPPORTED"),
    (lambda t: t.update(q_seqlen=np.array([17, 41], np.int32)), "MLA_ERR_SHAPE"),
    (lambda t: t.update(kv_seqlen=np.array([17], np.int32)), "MLA_ERR_SHAPE"),
    (lambda t: t.update(kv_seqlen=np.array([-1, 58], np.int32)), "MLA_ERR_VALUE"),
    (lambda t: t.update(q_rope=torch.zeros(57, 4, 32, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),
    (lambda t: t.update(v=torch.zeros(57, 4, 128, dtype=torch.float16)), "MLA_ERR_DTYPE"),
    (lambda t: t.update(atten_out=torch.zeros(57, 4, 64, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),
    (lambda t: t.update(k=torch.zeros(57, 2, 128, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),
    (lambda t: t.update(mask_type=mla.MASK_FREE), "MLA_ERR_NULL"),         # MASK_FREE needs the tile
    (lambda t: t.update(mask_type=mla.MASK_FREE, mask=torch.zeros(256, 512, dtype=torch.float16)),
     "MLA_ERR_SHAPE"),
    (lambda t: t.update(mask_type=mla.MASK_FREE, mask=torch.zeros(512, 512, dtype=torch.float32)),
     "MLA_ERR_DTYPE"),
    # device tensors must be 16-byte aligned (the kernel reads tile rows in 16-byte runs)
    (lambda t: t.update(mask_type=mla.MASK_FREE,
                        mask=torch.zeros(512 * 512 + 8, dtype=torch.float16)[1:1 + 512 * 512].view(512, 512)),
     "MLA_ERR_VALUE"),
    (lambda t: t.update(q=torch.zeros(57, 4, 128, dtype=torch.float32)), "MLA_ERR_DTYPE"),
])
def test_validation_errors(mutate, status):
    t = tensors()
    mutate(t)
    assert status_of(t) == status
    assert mla.mla_last_error() != ""


def test_head_dims_64_and_128_only_after_shape_checks():
    assert status_of(tensors(d=64)) == "MLA_OK"
    assert status_of(tensors(d=128)) == "MLA_OK"
    for d in (32, 96, 192, 256):
        assert status_of(tensors(d=d)) == "MLA_ERR_UNSUPPORTED"


def test_mask_ignored_unless_mask_free():
    t = tensors()
    t["mask"] = torch.zeros(3, dtype=torch.float32)  # would be invalid for MASK_FREE
    assert status_of(t) == "MLA_OK"


def test_two_dimensional_forms_and_padded_kv_accepted():
    t = tensors()
    t["q"] = t["q"].reshape(57, -1)
    t["atten_out"] = t["atten_out"].reshape(57, -1)
    t["q_rope"] = t["q_rope"].reshape(57, -1)
    assert status_of(t) == "MLA_OK"
    t = tensors(qs=(17, 40), ks=(30, 50))
    t["k"] = torch.zeros(2, 64, 4 * 128, dtype=torch.bfloat16)
    t["k_rope"] = torch.zeros(2, 64, 4 * 64, dtype=torch.bfloat16)
    t["v"] = torch.zeros(2, 64, 4 * 128, dtype=torch.bfloat16)
    assert status_of(t) == "MLA_OK"
    t["v"] = torch.zeros(80, 4, 128, dtype=torch.bfloat16)  # packed while k is padded
    assert status_of(t) == "MLA_ERR_SHAPE"


# The launching entry points are called here straight through ctypes, with
# descriptors built the binding's way: the binding itself refuses host memory
# for device arguments before it reaches the C call (tested below), and these
# tests are about the C library's own validation, which runs before any HIP
# call and never dereferences a tensor pointer.

def c_status(rc):
    return mla.STATUS.get(rc, str(rc))


def c_mla_prefill(t, workspace):
    keep = []
    args = mla._prefill_args(**t, keep=keep)
    ptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    size = workspace.numel() if workspace is not None else 0
    return c_status(mla._load().mla_prefill(*args, ctypes.c_void_p(ptr), ctypes.c_uint64(size), None))


def c_paged_cache_load(key_cache, value_cache, block_tables, context_lens, key, value, seq_starts, kv_cache_cfg,
                       is_seq_lens_cumsum_type, has_seq_starts):
    keep = []
    d = lambda x: mla._desc(x, keep)
    return c_status(mla._load().paged_cache_load(d(key_cache), d(value_cache), d(block_tables), d(context_lens),
                                                 d(key), d(value), d(seq_starts), int(kv_cache_cfg),
                                                 bool(is_seq_lens_cumsum_type), bool(has_seq_starts), None))


def c_mla_prolog(kw, workspace):
    keep = []
    args = mla._prolog_args(**kw, keep=keep)
    return c_status(mla._load().mla_prolog(*args, None, ctypes.c_uint64(0), None))


def test_workspace_checks_before_any_launch():
    t = tensors()
    need = ws_size(t)
    small = torch.zeros(need - 1, dtype=torch.uint8)
    assert c_mla_prefill(t, small) == "MLA_ERR_WORKSPACE"


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful where no GPU is present")
def test_no_device_is_a_runtime_error():
    t = tensors()
    ws = torch.zeros(ws_size(t), dtype=torch.uint8)
    assert c_mla_prefill(t, ws) == "MLA_ERR_RUNTIME"


# ----------------------------------------------- mla_prefill_no_alloc's limit

NO_ALLOC_BYTES = 4 << 20  # MLA_NO_ALLOC_WORKSPACE_BYTES
LAUNCH_RECORD_BYTES = 32


def c_no_alloc_on_shapes(nq, heads):
    """mla_prefill_no_alloc on one causal bf16 sequence of nq rows and keys
    with `heads` query and KV heads, given as descriptors whose data pointers
    are placeholders: a call that fails validation or the size check returns
    before any HIP call and reads no tensor memory."""
    def desc(*shape):
        d = mla.MlaTensor()
        d.data = 1 << 20
        d.dtype = 2  # MLA_BF16
        d.ndim = len(shape)
        for i, n in enumerate(shape):
            d.shape[i] = n
        return ctypes.pointer(d)
    lens = np.array([nq], np.int32)
    keep = []
    q, qr, out = desc(nq, heads, 128), desc(nq, heads, 64), desc(nq, heads, 128)
    k, kr, v = desc(nq, heads, 128), desc(nq, heads, 64), desc(nq, heads, 128)
    rc = mla._load().mla_prefill_no_alloc(q, qr, k, kr, v, mla._desc(lens, keep), mla._desc(lens, keep), None,
                                          heads, 0.1, heads, mla.MASK_CAUSAL, 0, out, None)
    return c_status(rc)


def launch_records(nq, heads):
    _, _, tasks = mla.mla_prefill_plan_host([nq], [nq], heads, heads, mla.MASK_CAUSAL)
    return len(tasks)


def test_no_alloc_rejects_work_lists_beyond_its_array():
    # 128 heads over 1024 items of 256 rows fill the array exactly; one more
    # item does not fit.
    assert launch_records(1024 * 256, 128) * LAUNCH_RECORD_BYTES == NO_ALLOC_BYTES
    assert launch_records(1024 * 256 + 1, 128) * LAUNCH_RECORD_BYTES > NO_ALLOC_BYTES
    assert c_no_alloc_on_shapes(1024 * 256 + 1, 128) == "MLA_ERR_WORKSPACE"
    assert "mla_prefill_no_alloc holds at most 4194304 bytes" in mla.mla_last_error()
    assert c_no_alloc_on_shapes(1024 * 256 + 1, 0) == "MLA_ERR_VALUE"  # validation still comes first


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful where no GPU is present")
def test_no_alloc_at_its_limit_passes_the_size_check():
    # A work list of exactly the array's size passes the check and reaches the
    # device lookup, which fails here for want of a GPU.
    assert c_no_alloc_on_shapes(1024 * 256, 128) == "MLA_ERR_RUNTIME"
    assert "hipGetDevice" in mla.mla_last_error() or "hip" in mla.mla_last_error().lower()


# ------------------------------------------------------- binding: device memory

def test_binding_refuses_host_memory_for_device_arguments():
    """A host pointer given to a kernel faults the GPU: the binding raises
    ValueError before the C call when a device argument is a numpy array or a
    CPU tensor (these would otherwise pass the C validation, which reads only
    shapes and dtypes)."""
    t = tensors()
    ws = torch.zeros(ws_size(t), dtype=torch.uint8)
    with pytest.raises(ValueError, match="q must be a torch tensor in GPU memory"):
        mla.mla_prefill(**t, workspace=ws, stream=0)
    with pytest.raises(ValueError, match="q must be a torch tensor in GPU memory"):
        mla.mla_prefill_no_alloc(**t, stream=0)
    with pytest.raises(ValueError, match="GPU memory"):
        mla.prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], t["q_seqlen"], t["kv_seqlen"], 4, 4, 0.1,
                    mla.MASK_CAUSAL)
    g = gather_args()
    g["context_lens"] = np.zeros(2, np.int32)  # host lengths: the gather reads them on the device
    with pytest.raises(ValueError, match="key_cache must be a torch tensor in GPU memory"):
        mla.paged_cache_load(**g, stream=0)
    with pytest.raises(ValueError, match="GPU memory"):
        mla.mla_prolog(**prolog_args(t=0), workspace=None, stream=0)
    with pytest.raises(ValueError, match="GPU memory"):
        mla.mla_prefill_paged(t["q"], t["q_rope"], torch.zeros(1, 64, 4, 128, dtype=torch.bfloat16),
                              torch.zeros(1, 64, 4, 64, dtype=torch.bfloat16),
                              torch.zeros(1, 64, 4, 128, dtype=torch.bfloat16), torch.zeros(2, 1, dtype=torch.int32),
                              t["q_seqlen"], t["kv_seqlen"], None, 4, 0.1, 4, mla.MASK_CAUSAL, t["atten_out"], ws,
                              stream=0)


def test_device_check_names_the_host_argument():
    class FakeCuda:  # stands in for a device tensor in the check's eyes only
        pass
    with pytest.raises(ValueError, match="context_lens must be .* \\(got ndarray\\)"):
        mla._on_device([("context_lens", np.zeros(2, np.int32))])
    with pytest.raises(ValueError, match="got tensor on cpu"):
        mla._on_device([("q", torch.zeros(2))])
    with pytest.raises(ValueError, match="got FakeCuda"):
        mla._on_device([("v", FakeCuda())])
    mla._on_device([("mask", None)])  # absent optional arguments are fine


def gather_args(**kw):
    a = dict(key_cache=torch.zeros(4, 8, 2, 16, dtype=torch.bfloat16),
             value_cache=torch.zeros(4, 8, 2, 16, dtype=torch.bfloat16),
             block_tables=torch.zeros(2, 2, dtype=torch.int32), context_lens=torch.zeros(2, dtype=torch.int32),
             key=torch.zeros(10, 2, 16, dtype=torch.bfloat16), value=torch.zeros(10, 2, 16, dtype=torch.bfloat16),
             seq_starts=None, kv_cache_cfg=mla.KV_CACHE_ND, is_seq_lens_cumsum_type=False, has_seq_starts=False)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(kv_cache_cfg=mla.KV_CACHE_NZ), "MLA_ERR_SHAPE"),   # ND-shaped outputs under NZ
    (dict(kv_cache_cfg=5), "MLA_ERR_VALUE"),
    (dict(value=None), "MLA_ERR_NULL"),
    (dict(key=torch.zeros(10, 2, 8, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),
    (dict(key=torch.zeros(10, 2, 16, dtype=torch.float16)), "MLA_ERR_DTYPE"),
    (dict(block_tables=torch.zeros(2, 2, dtype=torch.int64)), "MLA_ERR_DTYPE"),
    (dict(context_lens=torch.zeros(3, dtype=torch.int32)), "MLA_ERR_SHAPE"),   # [batch+1] needs cumsum
    (dict(has_seq_starts=True), "MLA_ERR_NULL"),
    (dict(has_seq_starts=True, seq_starts=torch.zeros(3, dtype=torch.int32)), "MLA_ERR_SHAPE"),
    (dict(key_cache=torch.zeros(4, 8, 32, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),
    (dict(key_cache=torch.zeros(4, 8, 2, 16, dtype=torch.float32)), "MLA_ERR_DTYPE"),
])
def test_gather_validation_errors(kw, status):
    assert c_paged_cache_load(**gather_args(**kw)) == status


def nz_args(**kw):
    # NZ: caches [num_blocks, chunks, block_size, 32 bytes of elements], outputs [num_tokens, chunks * elems]
    a = dict(key_cache=torch.zeros(4, 16, 8, 16, dtype=torch.bfloat16),
             value_cache=torch.zeros(4, 8, 8, 16, dtype=torch.bfloat16),
             block_tables=torch.zeros(2, 2, dtype=torch.int32), context_lens=torch.zeros(2, dtype=torch.int32),
             key=torch.zeros(10, 256, dtype=torch.bfloat16), value=torch.zeros(10, 128, dtype=torch.bfloat16),
             seq_starts=None, kv_cache_cfg=mla.KV_CACHE_NZ, is_seq_lens_cumsum_type=False, has_seq_starts=False)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(is_seq_lens_cumsum_type=True), "MLA_ERR_UNSUPPORTED"),   # the page: ND only
    (dict(has_seq_starts=True, seq_starts=torch.zeros(2, dtype=torch.int32)), "MLA_ERR_UNSUPPORTED"),
    (dict(key_cache=torch.zeros(4, 16, 8, 32, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),   # 16-bit: 16 per chunk
    (dict(key_cache=torch.zeros(4, 8, 8, 16, dtype=torch.int8), key=torch.zeros(10, 128, dtype=torch.int8),
          value_cache=None, value=None), "MLA_ERR_SHAPE"),                                # int8: 32 per chunk
    (dict(key=torch.zeros(10, 16, 16, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),
    (dict(value=torch.zeros(9, 128, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),
    (dict(value_cache=torch.zeros(4, 8, 4, 16, dtype=torch.bfloat16)), "MLA_ERR_SHAPE"),   # block size differs
])
def test_gather_nz_validation_errors(kw, status):
    assert c_paged_cache_load(**nz_args(**kw)) == status


def test_gather_nz_valid_shapes_pass_validation():
    # zero tokens: validation passes and nothing is launched (no HIP call here)
    assert c_paged_cache_load(**nz_args(key=torch.zeros(0, 256, dtype=torch.bfloat16),
                                        value=torch.zeros(0, 128, dtype=torch.bfloat16))) == "MLA_OK"
    assert c_paged_cache_load(**nz_args(key_cache=torch.zeros(4, 8, 8, 32, dtype=torch.int8),
                                        key=torch.zeros(0, 256, dtype=torch.int8), value_cache=None,
                                        value=None)) == "MLA_OK"


# ------------------------------------------------------------------ planner

def visible_count(mask_type, ql, kl, i):
    """Keys row i can see, from a materialised mask row."""
    p = kl - ql + i
    j = np.arange(kl)
    if mask_type == mla.MASK_UNDEFINED:
        vis = np.ones(kl, bool)
    elif mask_type in (mla.MASK_SPEC, mla.MASK_CAUSAL):
        vis = j <= p
    else:
        vis = (j // 512 <= p // 512) & (p >= 0)
    return int(vis.nonzero()[0].max()) + 1 if vis.any() else 0


def heads_per_task(heads, kv_heads):
    # largest power of two up to 8 dividing the group size
    g, p = heads // kv_heads, 1
    while p < 8 and g % (2 * p) == 0:
        p *= 2
    return p


def split_cap(items, heads, kv_heads):
    """Longest run of key tiles a task may hold: an even share W of the work
    (tiles plus 2 per task) over the 256 compute units, at least 16 tiles;
    unbounded unless the longest item exceeds 1.5 W."""
    pack = heads_per_task(heads, kv_heads)
    total = sum(int(nt) + 2 for _, _, nt, _ in items) * (heads // pack)
    share = -(-total // 256)
    if 2 * max(int(nt) for _, _, nt, _ in items) <= 3 * share:
        return 1 << 40
    return max(16, share)


@pytest.mark.parametrize("mask_type", [0, 1, 2, 3])
@pytest.mark.parametrize("case", [([17, 40], [17, 40], 4, 4), ([300, 1, 0, 129], [1000, 1, 5, 100], 8, 2),
                                  ([2048] * 3, [16384] * 3, 16, 16), ([700], [100], 2, 1),
                                  ([100, 33], [100, 260], 12, 4), ([513, 64], [600, 64], 32, 2),
                                  ([70], [70], 16, 1), ([4096], [4096], 16, 16), ([3000, 5], [5000, 700], 2, 1),
                                  ([1500, 2500], [1500, 9000], 8, 8)])
def test_plan_covers_every_row_once_with_exact_tile_ranges(case, mask_type):
    qs, ks, heads, kv_heads = case
    pack = heads_per_task(heads, kv_heads)
    rows = mla.PLAN_Q_ROWS // pack
    seqs, items, tasks = mla.mla_prefill_plan_host(qs, ks, heads, kv_heads, mask_type)
    # batch records are prefix sums
    assert (seqs[:, 0] == np.concatenate([[0], np.cumsum(qs)[:-1]])).all()
    assert (seqs[:, 1] == np.concatenate([[0], np.cumsum(ks)[:-1]])).all()
    assert (seqs[:, 2] == qs).all() and (seqs[:, 3] == ks).all()
    # every (b, q-tile of PLAN_Q_ROWS / pack rows) is one item
    assert (items[:, 3] == rows).all()
    want = sorted((b, r) for b, n in enumerate(qs) for r in range(0, n, rows))
    assert sorted((int(b), int(r)) for b, r, _, _ in items) == want
    # tile range = tiles holding the furthest visible key of any row in the item
    for b, r, nt, _ in items:
        ql, kl = qs[b], ks[b]
        far = max(visible_count(mask_type, ql, kl, i) for i in range(r, min(ql, r + rows)))
        assert nt == -(-far // mla.PLAN_KV_COLS), (b, r)
    # every (item, head) is covered by its tasks' key-tile runs exactly once:
    # one task over [0, kv_tiles), or consecutive runs of at most the even
    # share of the work (cut at 512-key multiples under MASK_FREE) when the
    # item is longer than that; the heads of a task share one kv head; the
    # rest is padding
    real = tasks[tasks[:, 0] >= 0]
    runs = {}
    for i, h0, k0, k1 in real.tolist():
        for k in range(pack):
            runs.setdefault((i, h0 + k), []).append((k0, k1))
    assert sorted(runs) == sorted((i, h) for i in range(len(items)) for h in range(heads))
    cap = split_cap(items, heads, kv_heads)
    gran = 8 if mask_type == mla.MASK_FREE else 1
    for (i, h), rs in runs.items():
        rs.sort()
        nt = int(items[i][2])
        assert rs[0][0] == 0 and rs[-1][1] == nt and all(a[1] == b[0] for a, b in zip(rs, rs[1:])), (i, h, rs)
        if nt <= cap:
            assert rs == [(0, nt)], (i, h, rs, cap)
        else:
            assert len(rs) >= 2 and all(0 < k1 - k0 <= cap + gran - 1 and k0 % gran == 0 for k0, k1 in rs), rs
    g = heads // kv_heads
    assert all(h0 % pack == 0 and h0 // g == (h0 + pack - 1) // g for _, h0, _, _ in real.tolist())
    assert len(tasks) % 8 == 0
    # the tasks reading one K/V stream (sequence, kv head) sit on one XCD (task
    # index mod 8), unless the stream holds more than 1/32 of all work
    stream_work, xcds = {}, {}
    for i, (it, h, k0, k1) in enumerate(tasks.tolist()):
        if it < 0:
            continue
        key = (int(items[it][0]), h // (heads // kv_heads))
        stream_work[key] = stream_work.get(key, 0) + k1 - k0 + 1
        xcds.setdefault(key, set()).add(i % 8)
    total = sum(stream_work.values())
    for key, w in stream_work.items():
        if 32 * w <= total:
            assert len(xcds[key]) == 1, key


def test_plan_balances_xcds_on_causal_workload():
    """4096-token causal prefill with 128 heads: every XCD gets the same work."""
    seqs, items, tasks = mla.mla_prefill_plan_host([4096], [4096], 128, 128, mla.MASK_CAUSAL)
    work = np.zeros(8)
    for i, (it, h, k0, k1) in enumerate(tasks.tolist()):
        if it >= 0:
            work[i % 8] += k1 - k0 + 1
    assert work.max() == work.min()
    # plenty of work for the CUs: no item is split
    real = tasks[tasks[:, 0] >= 0]
    assert (real[:, 2] == 0).all() and (real[:, 3] == items[real[:, 0], 2]).all()


@pytest.mark.parametrize("kv_heads", [128, 16, 1])
def test_plan_balances_xcds_with_few_kv_heads(kv_heads):
    """4096-token causal prefill, 128 query heads over kv_heads KV heads: a
    K/V stream holding more than 1/32 of the work is spread over XCDs, so
    every XCD's work is within 5% of the mean."""
    seqs, items, tasks = mla.mla_prefill_plan_host([4096], [4096], 128, kv_heads, mla.MASK_CAUSAL)
    work = np.zeros(8)
    for i, (it, h, k0, k1) in enumerate(tasks.tolist()):
        if it >= 0:
            work[i % 8] += k1 - k0 + 1
    assert work.max() <= 1.05 * work.mean(), work


def test_plan_splits_the_longest_items_when_work_is_scarce():
    """4096-token causal prefill at 16 heads: 256 items of 4..64 tiles for 256
    CUs. Items longer than the even share (36 tiles with 2 per task for the
    fixed work) are cut in two, so no task is longer than that share."""
    seqs, items, tasks = mla.mla_prefill_plan_host([4096], [4096], 16, 16, mla.MASK_CAUSAL)
    real = tasks[tasks[:, 0] >= 0]
    cap = split_cap(items, 16, 16)
    assert cap == 36
    assert (real[:, 3] - real[:, 2]).max() <= cap
    long_items = int((items[:, 2] > cap).sum())
    assert long_items == 7  # the items of rows 2304.. see 40, 44, .., 64 tiles
    assert len(real) == 16 * (16 + long_items)


def split_workspace_bytes(items, tasks, head_dim):
    """mla_prefill's workspace for a plan: launch records, merge records
    (one per split (item, head pack)), then per partial slot 256 rows of
    log-sum-exp and of head_dim fp32 values, each array 256-byte aligned."""
    up = lambda x: -(-x // 256) * 256
    real = tasks[tasks[:, 0] >= 0]
    split = real[(real[:, 2] != 0) | (real[:, 3] != items[real[:, 0], 2])]
    parts = len(split)
    merges = len({(int(i), int(h)) for i, h in split[:, :2]})
    if parts == 0:
        return len(tasks) * 32
    return up(len(tasks) * 32) + up(merges * 32) + up(parts * 256 * 4) + parts * 256 * head_dim * 4


def test_plan_does_not_split_when_the_longest_item_is_near_the_share():
    """4096-token causal prefill at 24 heads: the even share is 54 tiles and
    the longest item 64; no item is split (measured slower)."""
    seqs, items, tasks = mla.mla_prefill_plan_host([4096], [4096], 24, 24, mla.MASK_CAUSAL)
    real = tasks[tasks[:, 0] >= 0]
    assert (real[:, 2] == 0).all() and (real[:, 3] == items[real[:, 0], 2]).all()


@pytest.mark.parametrize("case", [((3000, 5), (5000, 700), 2, 1, 128), ((900,), (900,), 1, 1, 64),
                                  ((17, 40), (17, 40), 4, 4, 128)])
def test_workspace_size_of_split_plans(case):
    qs, ks, h, hk, d = case
    seqs, items, tasks = mla.mla_prefill_plan_host(list(qs), list(ks), h, hk, mla.MASK_CAUSAL)
    assert ws_size(tensors(qs=qs, ks=ks, h=h, hk=hk, d=d)) == split_workspace_bytes(items, tasks, d)


def test_plan_padded_offsets():
    seqs, _, _ = mla.mla_prefill_plan_host([3, 4, 5], [7, 8, 9], 2, 2, 2, kv_padded_max_seq=10)
    assert list(seqs[:, 1]) == [0, 10, 20]


# ------------------------------------------------------------------ page contract

def test_page_contract_values():
    g = json.load(open(GOLDEN))
    assert g["paged_cache_load"]["kvCacheCfg"]["value"] == {"K_CACHE_V_CACHE_NZ": mla.KV_CACHE_NZ,
                                                            "K_CACHE_V_CACHE_ND": mla.KV_CACHE_ND}
    assert g["mla_prefill"]["rope_dim"]["value"] == 64
    assert g["mla_prefill"]["mask_shape"]["value"] == [512, 512]
    import inspect
    sig = inspect.signature(mla.prefill)
    assert sig.parameters["qk_scale"].default == g["mla_prefill"]["qkScale_default"]["value"]
    assert sig.parameters["mask_type"].default == mla.MASK_UNDEFINED
    sig = inspect.signature(mla.paged_cache_load)
    assert sig.parameters["is_seq_lens_cumsum_type"].default is g["paged_cache_load"][
        "isSeqLensCumsumType_default"]["value"]
    assert sig.parameters["has_seq_starts"].default is g["paged_cache_load"]["hasSeqStarts_default"]["value"]
    # the page's headNum / kvHeadNum default of 0 is rejected as a value
    t = tensors()
    t["head_num"] = g["mla_prefill"]["headNum_default"]["value"]
    assert status_of(t) == "MLA_ERR_VALUE"


# ------------------------------------------------------------------ paged attention validation

def paged_tensors(qs=(17, 40), ks=(30, 100), h=4, hk=2, bs=64, nb=8, cols=2, dtype=torch.bfloat16):
    nq = sum(qs)
    z = lambda *s, dt=dtype: torch.zeros(s, dtype=dt)
    return dict(q=z(nq, h, 128), q_rope=z(nq, h, 64), key_cache=z(nb, bs, hk, 128),
                krope_cache=z(nb, bs, hk, 64), value_cache=z(nb, bs, hk, 128),
                block_tables=torch.zeros((len(qs), cols), dtype=torch.int32),
                q_seqlen=np.array(qs, np.int32), kv_seqlen=np.array(ks, np.int32), mask=None, head_num=h,
                qk_scale=0.1, kv_head_num=hk, mask_type=mla.MASK_CAUSAL, atten_out=z(nq, h, 128))


def paged_status(t):
    try:
        mla.mla_prefill_paged_get_workspace_size(**t)
        return 0
    except mla.MlaError as e:
        return e.code


def test_paged_valid_problem_plans_like_the_contiguous_one():
    t = paged_tensors()
    size = mla.mla_prefill_paged_get_workspace_size(**t)
    c = tensors(qs=(17, 40), ks=(30, 100), h=4, hk=2)
    assert size == ws_size(c) > 0


@pytest.mark.parametrize("mutate,status", [
    (dict(bs=96), -5),                 # block size not a multiple of 64
    (dict(bs=32, cols=4), -5),
    (dict(cols=1), -2),                # table too narrow for 100 keys at 64 per block
    (dict(ks=(30, 2048 * 64 + 1), cols=2100, nb=2100), -5),  # beyond the fused path's key limit
])
def test_paged_validation_errors(mutate, status):
    assert paged_status(paged_tensors(**mutate)) == status


def test_paged_cache_shape_and_dtype_errors():
    t = paged_tensors()
    t["krope_cache"] = torch.zeros((8, 64, 2, 32), dtype=torch.bfloat16)
    assert paged_status(t) == -2
    t = paged_tensors()
    t["value_cache"] = torch.zeros((8, 64, 2, 128), dtype=torch.float16)
    assert paged_status(t) == -3
    t = paged_tensors()
    t["block_tables"] = torch.zeros((2, 2), dtype=torch.int64)
    assert paged_status(t) == -3
    t = paged_tensors()
    t["block_tables"] = torch.zeros((3, 2), dtype=torch.int32)
    assert paged_status(t) == -2
    t = paged_tensors()
    t["key_cache"] = torch.zeros((8, 128, 2, 128), dtype=torch.bfloat16)  # block size differs between caches
    assert paged_status(t) == -2


# ------------------------------------------------------------------ prolog validation

def prolog_args(t=0, h=128, r=512, heads=2, hd=512, rd=64, **over):
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)
    a = dict(token_x=z(t, h), wq_a=z(h, r), wq_b=z(r, heads * hd), wkv=z(h, hd), rope_cos=z(t, rd),
             rope_sin=z(t, rd), gamma_cq=z(r), gamma_ckv=z(hd), eps=1e-6, q_out=z(t, heads, hd), kv_out=z(t, hd),
             qr_out=z(t, r))
    a.update(over)
    return a


def prolog_status(**kw):
    try:
        mla.mla_prolog_get_workspace_size(**prolog_args(**kw))
        return 0
    except mla.MlaError as e:
        return e.code


def test_prolog_workspace_size_and_empty_call():
    assert mla.mla_prolog_get_workspace_size(**prolog_args(t=0)) == 0
    # the fp32 rows of x . wq_a (256-byte aligned), then wq_a, wkv and wq_b
    # repacked (2 bytes per weight)
    h, r, heads, hd = 128, 512, 2, 512
    assert mla.mla_prolog_get_workspace_size(**prolog_args(t=3)) == \
        256 * -(-3 * r * 4 // 256) + 2 * h * r + 2 * h * hd + 2 * r * heads * hd
    # t = 0: valid, nothing to launch (no HIP call)
    assert c_mla_prolog(prolog_args(t=0), None) == "MLA_OK"


def test_prolog_validation_errors():
    ERR_SHAPE, ERR_DTYPE, ERR_VALUE, ERR_UNSUP = -2, -3, -4, -5
    assert prolog_status(token_x=torch.zeros(0, 64, dtype=torch.float16)) == ERR_DTYPE
    assert prolog_status(eps=0.0) == ERR_VALUE
    assert prolog_status(wq_a=torch.zeros(64, 512, dtype=torch.bfloat16)) == ERR_SHAPE
    assert prolog_status(gamma_ckv=torch.zeros(511, dtype=torch.bfloat16)) == ERR_SHAPE
    assert prolog_status(q_out=torch.zeros(0, 3, 512, dtype=torch.bfloat16)) == ERR_SHAPE
    assert prolog_status(kv_out=torch.zeros(1, 512, dtype=torch.bfloat16)) == ERR_SHAPE
    # the kernels' supported sizes
    assert prolog_status(hd=256) == ERR_UNSUP
    assert prolog_status(rd=32) == ERR_UNSUP
    assert prolog_status(r=1000) == ERR_UNSUP
    assert prolog_status(h=48) == ERR_UNSUP
    assert prolog_status(h=192) == ERR_UNSUP
    # 2-D q_out is accepted
    assert prolog_status(q_out=torch.zeros(0, 1024, dtype=torch.bfloat16)) == 0


def prolog_quant_args(t=0, h=128, r=512, heads=2, hd=512, rd=64, **over):
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)
    a = dict(token_x=z(t, h), wq_a=z(h, r), wq_b=z(r, heads * hd, dt=torch.int8), wkv=z(h, hd), rope_cos=z(t, rd),
             rope_sin=z(t, rd), gamma_cq=z(r), gamma_ckv=z(hd), wq_b_scale=z(heads * hd, 1, dt=torch.float32),
             eps=1e-6, q_out=z(t, heads, hd), kv_out=z(t, hd), qr_out=z(t, r, dt=torch.int8),
             qr_scale_out=z(t, 1, dt=torch.float32))
    a.update(over)
    return a


def prolog_quant_status(**kw):
    try:
        mla.mla_prolog_quant_get_workspace_size(**prolog_quant_args(**kw))
        return 0
    except mla.MlaError as e:
        return e.code


def test_prolog_quant_workspace_size():
    assert mla.mla_prolog_quant_get_workspace_size(**prolog_quant_args(t=0)) == 0
    # the fp32 rows of x . wq_a, then wq_a and wkv repacked (2 bytes per
    # weight) and wq_b repacked (1 byte per weight), each 256-byte aligned
    h, r, heads, hd = 128, 512, 2, 512
    assert mla.mla_prolog_quant_get_workspace_size(**prolog_quant_args(t=3)) == \
        256 * -(-3 * r * 4 // 256) + 2 * h * r + 2 * h * hd + r * heads * hd
    # [n] scales are accepted as well as [n, 1]
    assert prolog_quant_status(t=2, wq_b_scale=torch.zeros(1024, dtype=torch.float32),
                               qr_scale_out=torch.zeros(2, dtype=torch.float32)) == 0


def test_prolog_quant_validation_errors():
    ERR_SHAPE, ERR_DTYPE, ERR_UNSUP = -2, -3, -5
    # wq_b and qr_out must be int8, the scales float32
    assert prolog_quant_status(wq_b=torch.zeros(512, 1024, dtype=torch.bfloat16)) == ERR_DTYPE
    assert prolog_quant_status(qr_out=torch.zeros(0, 512, dtype=torch.bfloat16)) == ERR_DTYPE
    assert prolog_quant_status(wq_b_scale=torch.zeros(1024, 1, dtype=torch.bfloat16)) == ERR_DTYPE
    assert prolog_quant_status(t=2, qr_scale_out=torch.zeros(2, 1, dtype=torch.float16)) == ERR_DTYPE
    # one scale per column of wq_b, one per token
    assert prolog_quant_status(wq_b_scale=torch.zeros(512, 1, dtype=torch.float32)) == ERR_SHAPE
    assert prolog_quant_status(wq_b_scale=torch.zeros(1024, 2, dtype=torch.float32)) == ERR_SHAPE
    assert prolog_quant_status(t=2, qr_scale_out=torch.zeros(3, 1, dtype=torch.float32)) == ERR_SHAPE
    # the plain prolog's checks still apply, and q_lora_rank is at most 2048
    assert prolog_quant_status(hd=256) == ERR_UNSUP
    assert prolog_quant_status(r=2560) == ERR_UNSUP
    assert prolog_status(r=2560) == 0  # the plain prolog has no such limit
    # the plain entry point still wants bf16 wq_b
    assert prolog_status(wq_b=torch.zeros(512, 1024, dtype=torch.int8)) == ERR_DTYPE


def test_gather_batch_limit():
    # the gather kernel keeps the batch's offsets in LDS: 8192 sequences at most
    def args(batch):
        return gather_args(block_tables=torch.zeros(batch, 1, dtype=torch.int32),
                           context_lens=torch.zeros(batch, dtype=torch.int32),
                           key=torch.zeros(0, 2, 16, dtype=torch.bfloat16),
                           value=torch.zeros(0, 2, 16, dtype=torch.bfloat16))
    assert c_paged_cache_load(**args(8192)) == "MLA_OK"  # valid; zero tokens, nothing launched
    assert c_paged_cache_load(**args(8193)) == "MLA_ERR_UNSUPPORTED"


def test_prolog_workspace_with_split_first_product():
    # h 4096: 32 runs of 4 stages; at t = 64 the first product has 3 tiles
    # (q_lora_rank 1024 + the 512-column kv tile), so it is split into all 32
    # runs, whose fp32 sums follow the packed weights
    t, h, r, heads, hd = 64, 4096, 1024, 2, 512
    up = lambda x: -(-x // 256) * 256
    base = up(t * r * 4) + up(2 * h * r) + up(2 * h * hd) + up(2 * r * heads * hd)
    got = mla.mla_prolog_get_workspace_size(**prolog_args(t=t, h=h, r=r, heads=heads))
    assert got == base + up(32 * t * (r + 512) * 4)
    # 9 tiles at 300 rows: 16 runs (the smallest divisor of 32 giving 128 workgroups)
    got = mla.mla_prolog_get_workspace_size(**prolog_args(t=300, h=h, r=r, heads=heads))
    assert got == up(300 * r * 4) + up(2 * h * r) + up(2 * h * hd) + up(2 * r * heads * hd) + up(16 * 300 * (r + 512) * 4)
    # 129 tiles and more: no split
    got = mla.mla_prolog_get_workspace_size(**prolog_args(t=128 * 43, h=h, r=r, heads=heads))
    assert got == up(128 * 43 * r * 4) + up(2 * h * r) + up(2 * h * hd) + up(2 * r * heads * hd)


def test_prolog_packed_weights_and_prepacked_workspace_sizes():
    up = lambda x: -(-x // 256) * 256
    h, r, heads, hd = 4096, 1024, 2, 512
    a = prolog_args(t=64, h=h, r=r, heads=heads)
    # wq_a, wkv and wq_b rearranged, 2 bytes per weight (1 for int8 wq_b)
    assert mla.mla_prolog_weights_size(a["wq_a"], a["wq_b"], a["wkv"]) == up(2 * h * r) + up(2 * h * hd) + \
        up(2 * r * heads * hd)
    q = prolog_quant_args(t=64, h=h, r=r, heads=heads)
    assert mla.mla_prolog_weights_size(q["wq_a"], q["wq_b"], q["wkv"]) == up(2 * h * r) + up(2 * h * hd) + \
        up(r * heads * hd)
    # prepacked workspace: x . wq_a and the split sums (32 runs at 64 rows), no weights
    assert mla.mla_prolog_prepacked_workspace_size(a["token_x"], a["wq_a"]) == up(64 * r * 4) + \
        up(32 * 64 * (r + 512) * 4)
    assert mla.mla_prolog_prepacked_workspace_size(a["token_x"][:0], a["wq_a"]) == 0
    # with the packing operator's workspace: weights + the same
    assert mla.mla_prolog_get_workspace_size(**a) == mla.mla_prolog_prepacked_workspace_size(a["token_x"], a["wq_a"]) \
        + mla.mla_prolog_weights_size(a["wq_a"], a["wq_b"], a["wkv"])


def test_prolog_prepacked_errors_before_any_launch():
    keep = []
    a = prolog_args(t=3)
    need = mla.mla_prolog_weights_size(a["wq_a"], a["wq_b"], a["wkv"])
    small = torch.zeros(need - 256, dtype=torch.uint8)
    ws = torch.zeros(mla.mla_prolog_prepacked_workspace_size(a["token_x"], a["wq_a"]), dtype=torch.uint8)
    lib = mla._load()
    args = mla._prolog_args(**a, keep=keep)
    rc = lib.mla_prolog_prepacked(*args, ctypes.c_void_p(small.data_ptr()), ctypes.c_uint64(small.numel()),
                                  ctypes.c_void_p(ws.data_ptr()), ctypes.c_uint64(ws.numel()), None)
    assert c_status(rc) == "MLA_ERR_WORKSPACE" and "packed weights" in mla.mla_last_error()
    rc = lib.mla_prolog_prepacked(*args, None, ctypes.c_uint64(need), ctypes.c_void_p(ws.data_ptr()),
                                  ctypes.c_uint64(ws.numel()), None)
    assert c_status(rc) == "MLA_ERR_NULL"
    # the weights alone: dtype and shape checks
    with pytest.raises(mla.MlaError) as e:
        mla.mla_prolog_weights_size(a["wq_a"].half(), a["wq_b"], a["wkv"])
    assert e.value.status == "MLA_ERR_DTYPE"
    with pytest.raises(mla.MlaError) as e:
        mla.mla_prolog_weights_size(a["wq_a"], a["wq_b"][:, :1000].contiguous(), a["wkv"])
    assert e.value.status == "MLA_ERR_SHAPE"
    with pytest.raises(mla.MlaError) as e:
        mla.mla_prolog_weights_size(a["wq_a"], a["wq_b"], a["wkv"][:, :256].contiguous())
    assert e.value.status == "MLA_ERR_UNSUPPORTED"


@pytest.mark.parametrize("case", [((17, 40), (17, 40), 4, 4), ((3000, 5), (5000, 700), 2, 1)])
def test_mask_free_workspace_ends_with_the_tile_classes(case):
    # MASK_FREE: after the plan's arrays, 256-byte aligned, one class byte per
    # (tile row, 64-key block): 512 * 8 bytes
    qs, ks, h, hk = case
    up = lambda x: -(-x // 256) * 256
    _, items, tasks = mla.mla_prefill_plan_host(list(qs), list(ks), h, hk, mla.MASK_FREE)
    t = tensors(qs=qs, ks=ks, h=h, hk=hk)
    t.update(mask=torch.zeros(512, 512, dtype=torch.float16), mask_type=mla.MASK_FREE)
    assert ws_size(t) == up(split_workspace_bytes(items, tasks, 128)) + 512 * 8
