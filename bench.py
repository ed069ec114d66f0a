#!/usr/bin/env python3
"""Benchmark of the MLA varlen-prefill hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input:
mla_prefill_get_workspace_size-style validation and planning on the host, the
work-list copy, and the attention kernel (the ``single`` workload: batch 1,
4096 query and key tokens, 128 heads, embeddimV 128 + rope 64, bf16,
causal). Inputs are resident in HBM before timing starts.

Prints ONE JSON line with the throughput in algorithmic TFLOP/s (640 FLOP per
visible (query, key, head) triple), the kernel's roofline position measured
with HIP events on the launch stream, the CPU oracle timed on a bounded sample
of the same workload, and the paged gather's bandwidth on the paged workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mla_varlen_prefill_amd as mla  # noqa: E402
from mla_varlen_prefill_amd import synth  # noqa: E402

METRIC = "MLA prefill attention TFLOP/s at 1 MI355X + % of bf16 MFMA peak"
PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA
FLOP_PER_PAIR = 2 * (128 + 64) + 2 * 128
PMC_FILE = os.path.join(ROOT, "profiles", "mla_fwd_single_pmc.json")
COPY_BYTES = 1 << 30  # plain copy of known size, for scaling the HBM counters


def visible_pairs(qs, ks, mask_type):
    """Visible (query, key) pairs of one head."""
    total = 0
    for ql, kl in zip(qs, ks):
        ql, kl = int(ql), int(kl)
        if mask_type == synth.MASK_UNDEFINED:
            total += ql * kl
            continue
        p = kl - ql + np.arange(ql, dtype=np.int64)  # key position of each row
        total += int(np.clip(p + 1, 0, kl).sum())
    return total


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("mla_fwd.hip", "kernels.h"):
        with open(os.path.join(ROOT, "mla_varlen_prefill_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    try:
        with open(PMC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def calibration_copy():
    """A plain device copy of COPY_BYTES (reads and writes COPY_BYTES of HBM)."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def summarize_pmc(fetch_dir, write_dir, out_json):
    """Turn two rocprofv3 --pmc runs of `bench.py --calibrate-copy` (one with
    FETCH_SIZE, one with WRITE_SIZE) into HBM bytes per attention launch.

    Each counter is scaled by COPY_BYTES over what it read for the plain copy
    kernel in the same run."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        copy = [v for (i, k), v in vals.items() if "copy" in k.lower() and "mla" not in k]
        attn = [v for (i, k), v in vals.items() if "mla_fwd_kernel" in k]
        return max(copy), attn

    fetch_copy, fetch_attn = per_dispatch(fetch_dir, "FETCH_SIZE")
    write_copy, write_attn = per_dispatch(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / (fetch_copy * 1024.0)
    w_scale = COPY_BYTES / (write_copy * 1024.0)
    fetch = float(np.median(fetch_attn)) * 1024.0 * f_scale
    write = float(np.median(write_attn)) * 1024.0 * w_scale
    rec = {"kernel": "mla_fwd_kernel", "workload": "single", "kernel_source_sha256_16": kernel_source_hash(),
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": fetch_copy, "copy_write_kib": write_copy,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "attn_fetch_kib_median": float(np.median(fetch_attn)), "attn_write_kib_median": float(np.median(write_attn)),
           "hbm_fetch_bytes_per_launch": fetch, "hbm_write_bytes_per_launch": write,
           "hbm_bytes_per_launch": fetch + write, "dispatches": len(fetch_attn)}
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


# Counter passes for the attention kernel's utilisation (each within one
# rocprofv3 pass: at most 8 SQ and 2 GRBM counters).
UTIL_PASSES = (
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE",
    "SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS "
    "SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 GRBM_GUI_ACTIVE",
)
SIMDS = 1024          # 256 CUs x 4 SIMDs
MFMA_FLOP_PER_SIMD_CYCLE = 1024  # bf16/fp16 dense: 2.5 PFLOP/s = 1024 SIMDs x 1024 x ~2.4 GHz
XCCS = 8              # GRBM_GUI_ACTIVE is summed over the 8 XCDs


def summarize_util(workload, out_json, dirs):
    """Medians over the timed dispatches of mla_fwd_kernel of the counters of
    the UTIL_PASSES runs in ``dirs`` (``rocprofv3 --kernel-trace --pmc ...
    --output-format csv``; the first two dispatches, warm-up, are dropped),
    with the derived figures:

      cycles          GRBM_GUI_ACTIVE / 8 (per XCD)
      clock_ghz       cycles / dispatch duration
      mfma_busy       SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)
      mfma_flop       SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (FLOP issued to the matrix cores)
      useful          algorithmic FLOP / mfma_flop (masked parts of diagonal tiles are issued but not counted)
      predicted       mfma_busy x 1024 SIMDs x 1024 FLOP/cycle x clock x useful
      valu_busy       SQ_ACTIVE_INST_VALU x 4 / (cycles x 1024 SIMDs)
      lds_conflict    SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS
    """
    import collections
    import csv
    import glob
    import statistics as st

    qs, ks = synth.workload_seqlens(workload)
    heads = synth.WORKLOADS[workload]["heads"]
    alg = FLOP_PER_PAIR * heads * visible_pairs(qs, ks, synth.MASK_CAUSAL)
    merged = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        per = collections.defaultdict(dict)
        for f in files:
            for r in csv.DictReader(open(f)):
                if "mla_fwd_kernel" not in r["Kernel_Name"]:
                    continue
                v = per[int(r["Dispatch_Id"])]
                v[r["Counter_Name"]] = v.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                v["duration_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        rows = [per[k] for k in sorted(per)][2:]
        for name in rows[0]:
            key = name if name not in merged else f"{name}@{os.path.basename(os.path.normpath(d))}"
            merged[key] = st.median(x[name] for x in rows)
        merged.setdefault("dispatches", len(rows))
    cycles = merged["GRBM_GUI_ACTIVE"] / XCCS
    dur = merged["duration_ns"] * 1e-9
    clock = cycles / dur
    busy = merged["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS)
    mfma_flop = merged["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    useful = alg / mfma_flop
    predicted = busy * SIMDS * MFMA_FLOP_PER_SIMD_CYCLE * clock * useful
    rec = {"kernel": "mla_fwd_kernel", "workload": workload, "kernel_source_sha256_16": kernel_source_hash(),
           "counters_median": merged, "algorithmic_flop": alg, "duration_ms": dur * 1e3,
           "cycles": cycles, "clock_ghz": clock / 1e9, "mfma_busy": busy, "mfma_flop": mfma_flop,
           "useful_fraction": useful, "tflops_measured": alg / dur / 1e12,
           "tflops_from_mfma_counter": mfma_flop / dur / 1e12 * useful,
           "tflops_predicted_from_busy": predicted / 1e12,
           "predicted_over_measured": predicted / (alg / dur),
           "valu_busy": merged.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / (cycles * SIMDS),
           "mfma_valu_coexec": merged.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / (cycles * SIMDS),
           "lds_bank_conflict_per_lds_active": (merged.get("SQ_LDS_BANK_CONFLICT", 0.0)
                                                / max(merged.get("SQ_ACTIVE_INST_LDS", 0.0), 1.0))}
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def bench_attention(name, steps, warmup):
    t, qs, ks, params = synth.workload_inputs(name, device="cuda")
    H = params["head_num"]
    out = torch.empty_like(t["q"])
    args = dict(q=t["q"], q_rope=t["q_rope"], k=t["k"], k_rope=t["k_rope"], v=t["v"], q_seqlen=qs,
                kv_seqlen=ks, mask=None, head_num=H, qk_scale=params["qk_scale"],
                kv_head_num=params["kv_head_num"], mask_type=params["mask_type"], cache_mode=0, atten_out=out)
    ws_bytes = mla.mla_prefill_get_workspace_size(**args)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        mla.mla_prefill(**args, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        mla.mla_prefill(**args, workspace=ws, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    flops = FLOP_PER_PAIR * H * visible_pairs(qs, ks, params["mask_type"])
    return dict(tensors=t, qs=qs, ks=ks, params=params, out=out, flops=flops,
                ms_per_step=(t1 - t0) * 1e3 / steps, launch_ms=float(np.mean(launch_ms)),
                launch_ms_min=float(np.min(launch_ms)))


def _attention_tflops(t, qs, ks, heads, kv_heads, mask_type, mask, steps):
    d = t["q"].shape[-1]
    out = torch.empty((t["q"].shape[0], heads, d), dtype=t["q"].dtype, device="cuda")
    args = dict(q=t["q"], q_rope=t["q_rope"], k=t["k"], k_rope=t["k_rope"], v=t["v"], q_seqlen=qs, kv_seqlen=ks,
                mask=mask, head_num=heads, qk_scale=synth.QK_SCALE, kv_head_num=kv_heads, mask_type=mask_type,
                cache_mode=0, atten_out=out)
    ws = torch.empty(max(mla.mla_prefill_get_workspace_size(**args), 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ms = _time(lambda: mla.mla_prefill(**args, workspace=ws, stream=stream), steps, stream)
    # 2 * (D + 64) for the scores and 2 * D for P.V per visible (query, key, head)
    flops = (4 * d + 2 * 64) * heads * visible_pairs(qs, ks, mask_type)
    return {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}


def bench_extras(steps, cpu=True):
    """Secondary configurations: the chunked workload under MASK_FREE with the
    causal fp16 tile (the same visible pairs as causal); one GPU's share of an
    8-way split over heads (16 heads) of the single and chunked shapes; the
    single shape at head dim 64; and the single shape with its 128 query heads
    grouped over 16 and over 1 KV heads."""
    res = {}
    t, qs, ks, p = synth.workload_inputs("chunked", device="cuda")
    res["chunked_causal"] = _attention_tflops(t, qs, ks, 128, 128, synth.MASK_CAUSAL, None, steps)
    tile = synth.causal_mask_tile(torch.float16, "cuda")
    res["chunked_mask_free_causal_tile"] = _attention_tflops(t, qs, ks, 128, 128, synth.MASK_FREE, tile, steps)
    oracle_recs = {}
    if cpu:
        seed = synth.WORKLOADS["chunked"]["seed"]
        oracle_recs["chunked"] = oracle_sampled(t, qs, ks, 128, 128, synth.MASK_CAUSAL, seed)
        oracle_recs["chunked_mask_free_causal_tile"] = oracle_sampled(t, qs, ks, 128, 128, synth.MASK_FREE, seed,
                                                                      tile=tile, tile_edge_rows=True)
    del t
    for name in ("single", "chunked"):
        qs, ks = synth.workload_seqlens(name)
        w = synth.WORKLOADS[name]
        t = synth.attention_inputs(qs, ks, 16, 16, w["dtype"], w["sigma"], w["seed"], "cuda")
        res[f"tp8_share_{name}_16_heads"] = _attention_tflops(t, np.asarray(qs, np.int32), np.asarray(ks, np.int32),
                                                             16, 16, synth.MASK_CAUSAL, None, steps)
        del t
    qs, ks = synth.workload_seqlens("single")
    w = synth.WORKLOADS["single"]
    t = synth.attention_inputs(qs, ks, 128, 128, w["dtype"], w["sigma"], w["seed"], "cuda", d_nope=64)
    res["single_head_dim_64"] = _attention_tflops(t, np.asarray(qs, np.int32), np.asarray(ks, np.int32), 128, 128,
                                                  synth.MASK_CAUSAL, None, steps)
    del t
    for hk in (16, 1):
        t = synth.attention_inputs(qs, ks, 128, hk, w["dtype"], w["sigma"], w["seed"], "cuda")
        res[f"single_128_heads_{hk}_kv_heads"] = _attention_tflops(t, np.asarray(qs, np.int32),
                                                                   np.asarray(ks, np.int32), 128, hk,
                                                                   synth.MASK_CAUSAL, None, steps)
        del t
    torch.cuda.empty_cache()
    return {k: {"ms": round(v["ms"], 4), "tflops": round(v["tflops"], 2)} for k, v in res.items()}, oracle_recs


def cpu_baseline(res, seconds):
    """The oracle as it stands, on whole heads of the same workload until about
    ``seconds`` of CPU time have been spent (at least one head)."""
    import oracle
    t, qs, ks, params = res["tensors"], res["qs"], res["ks"], res["params"]
    oracle.build()
    ql, kl = int(qs[0]), int(ks[0])
    flops = 0
    spent = 0.0
    heads = 0
    for h in range(params["head_num"]):
        hk = oracle.kv_head_of(h, params["head_num"], params["kv_head_num"])
        a = [t["q"][:ql, h], t["q_rope"][:ql, h], t["k"][:kl, hk], t["k_rope"][:kl, hk], t["v"][:kl, hk]]
        a = [x.double().cpu().numpy() for x in a]
        s = time.perf_counter()
        oracle.attention_head(*a, params["qk_scale"], params["mask_type"])
        spent += time.perf_counter() - s
        flops += FLOP_PER_PAIR * visible_pairs([ql], [kl], params["mask_type"])
        heads += 1
        if spent >= seconds:
            break
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{heads} of {params['head_num']} heads, all {ql} query rows each, of the same workload "
                      f"({spent:.1f} s, fp64)"}


def _visible_keys(ql, kl, i, mask_type):
    """Keys query row i of a (ql, kl) sequence sees under a causal-like rule
    (MASK_FREE is only ever timed here with the causal tile)."""
    if mask_type == synth.MASK_UNDEFINED:
        return kl
    return int(min(kl, max(0, kl - ql + i + 1)))


def oracle_sampled(t, qs, ks, heads, kv_heads, mask_type, seed, tile=None, paged=None, tile_edge_rows=False,
                   pairs=256, rows_per_pair=8):
    """The oracle as it stands on a seeded sample of a workload, with the time
    of the whole workload extrapolated from it.

    Sample: ``pairs`` (sequence, head) pairs from default_rng(seed + 1000),
    the sequence drawn with probability proportional to its query rows and the
    head uniformly, ``rows_per_pair`` uniform rows of each (so every query row
    of the workload is equally likely); plus, for every sequence, rows 0, 1
    and qlen - 1 at heads 0 and H - 1; with ``tile_edge_rows``, also the rows
    whose key position is 0, 1 or 511 modulo 512 (edges of the MASK_FREE tile
    blocks) at head 0. Only the (sequence, KV head) slices the sample reads are
    copied to the host. Each row is one oracle call, with the oracle set to
    one thread. Paged inputs (``paged`` = caches + table) go through the
    oracle's gather of the sampled sequence and head first, as its paged path
    does.

    Extrapolation: the oracle scores every key of a sequence for every query
    row, so its time per row is proportional to the sequence's key count;
    full time = sampled time per (row x key) x sum over heads and sequences of
    qlen x kvlen (the paged gather: per (head x key), once per sequence and
    head)."""
    import oracle
    oracle.build()
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        return _oracle_sampled(oracle, threads, t, qs, ks, heads, kv_heads, mask_type, seed, tile, paged,
                               tile_edge_rows, pairs, rows_per_pair)
    finally:
        oracle.set_num_threads(threads)


def _oracle_sampled(oracle, threads, t, qs, ks, heads, kv_heads, mask_type, seed, tile, paged, tile_edge_rows,
                    pairs, rows_per_pair):
    qs, ks = np.asarray(qs, np.int64), np.asarray(ks, np.int64)
    nb = len(qs)
    qoff = np.concatenate([[0], np.cumsum(qs)])
    koff = np.concatenate([[0], np.cumsum(ks)])
    rng = np.random.default_rng(seed + 1000)
    groups = {}
    pb = rng.choice(nb, size=pairs, p=qs / qs.sum())
    ph = rng.integers(0, heads, size=pairs)
    for b, h in zip(pb.tolist(), ph.tolist()):
        groups.setdefault((b, h), set()).update(rng.integers(0, qs[b], size=rows_per_pair).tolist())
    sampled = sum(len(v) for v in groups.values())
    for b in range(nb):
        if qs[b] == 0:
            continue
        for h in (0, heads - 1):
            groups.setdefault((b, h), set()).update({0, min(1, int(qs[b]) - 1), int(qs[b]) - 1})
        if tile_edge_rows:
            pos = ks[b] - qs[b] + np.arange(qs[b])
            edge = np.nonzero(np.isin(pos % synth.MASK_TILE, (0, 1, synth.MASK_TILE - 1)))[0]
            groups.setdefault((b, 0), set()).update(edge.tolist())
    tile64 = tile.double().cpu().numpy() if tile is not None else None
    d = t["q"].shape[-1]
    flop_pair = 4 * d + 2 * 64
    t_attn = t_gather = 0.0
    n_rows = row_keys = gather_keys = 0
    sample_flops = 0
    # fp32 on the device, fp64 in numpy: no torch CPU op (whose worker threads
    # would keep spinning beside the timed oracle calls)
    host = lambda x: x.contiguous().float().cpu().numpy().astype(np.float64)
    for (b, h), rows in sorted(groups.items()):
        hk = oracle.kv_head_of(h, heads, kv_heads)
        ql, kl = int(qs[b]), int(ks[b])
        q = host(t["q"][qoff[b]:qoff[b] + ql, h])
        qr = host(t["q_rope"][qoff[b]:qoff[b] + ql, h])
        if paged is None:
            k = host(t["k"][koff[b]:koff[b] + kl, hk])
            kr = host(t["k_rope"][koff[b]:koff[b] + kl, hk])
            v = host(t["v"][koff[b]:koff[b] + kl, hk])
        else:
            bs = paged["key_cache"].shape[1]
            nblk = -(-kl // bs)
            idx = paged["block_tables"][b, :nblk].long()
            sub = [host(paged[c][:, :, hk][idx]).reshape(nblk, bs, 1, -1)
                   for c in ("key_cache", "rope_cache", "value_cache")]
            row = np.arange(nblk, dtype=np.int64)[None]
            lens = np.array([kl], np.int64)
            s0 = time.perf_counter()
            k, _ = oracle.paged_cache_load(sub[0], None, row, lens)
            kr, _ = oracle.paged_cache_load(sub[1], None, row, lens)
            v, _ = oracle.paged_cache_load(sub[2], None, row, lens)
            t_gather += time.perf_counter() - s0
            gather_keys += kl
            k, kr, v = k[:, 0], kr[:, 0], v[:, 0]
        for i in sorted(rows):
            s0 = time.perf_counter()
            oracle.attention_head(q, qr, k, kr, v, synth.QK_SCALE, mask_type, mask=tile64,
                                  rows=np.array([i], np.int64))
            t_attn += time.perf_counter() - s0
            n_rows += 1
            row_keys += kl
            sample_flops += flop_pair * _visible_keys(ql, kl, i, mask_type)
    full_row_keys = heads * int((qs * ks).sum())
    full_flops = flop_pair * heads * visible_pairs(qs, ks, mask_type)
    est = t_attn / row_keys * full_row_keys
    if paged is not None:
        est += t_gather / gather_keys * heads * int(ks.sum())
    rec = {"value": full_flops / est / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
           "value_is": "extrapolated: the workload's FLOPs over the extrapolated full oracle time",
           "sample": f"{n_rows} query rows in {len(groups)} (sequence, head) pairs ({sampled} seeded rows in "
                     f"{pairs} pairs + boundary rows), one row per oracle call, fp64, one core",
           "sample_seconds": round(t_attn + t_gather, 3), "sample_tflops": sample_flops / (t_attn + t_gather) / 1e12,
           "extrapolated_full_seconds_one_core": round(est, 1),
           "extrapolated_full_seconds_ideal_all_cores": round(est / threads, 1), "host_threads": threads}
    if paged is not None:
        rec["sample_gather_seconds"] = round(t_gather, 3)
    return rec


def bench_configs(steps, cpu=True):
    """The varlen (fp16) and tiny workloads: ms per call (host planning,
    work-list copy and kernel), TFLOP/s and fraction of the bf16/fp16 MFMA
    peak. The tiny workload is timed with the full oracle beside it; varlen
    with the sampled oracle."""
    out = {}
    for name in ("varlen", "tiny"):
        t, qs, ks, p = synth.workload_inputs(name, device="cuda")
        n = steps if name == "varlen" else max(steps, 200)
        r = _attention_tflops(t, qs, ks, p["head_num"], p["kv_head_num"], p["mask_type"], None, n)
        w = synth.WORKLOADS[name]
        rec = {"workload": name, "dtype": "fp16" if w["dtype"] == torch.float16 else "bf16", "batch": len(qs),
               "heads": p["head_num"], "mask": "causal", "tokens": int(np.sum(qs)), "timed_calls": n,
               "ms": round(r["ms"], 4), "tflops": round(r["tflops"], 2), "frac": round(r["tflops"] / PEAK_TFLOPS, 4)}
        if cpu and name == "varlen":
            rec["cpu_baseline"] = oracle_sampled(t, qs, ks, p["head_num"], p["kv_head_num"], p["mask_type"],
                                                 w["seed"])
        elif cpu:
            rec["cpu_baseline"] = oracle_full(t, qs, ks, p)
        out[name] = rec
        del t
    torch.cuda.empty_cache()
    return out


def oracle_full(t, qs, ks, params):
    """The oracle on every row and head of a (small) workload."""
    import oracle
    oracle.build()
    h = {k: v.double().cpu().numpy() for k, v in t.items()}
    s0 = time.perf_counter()
    oracle.attention(h["q"], h["q_rope"], h["k"], h["k_rope"], h["v"], qs, ks, params["head_num"],
                     params["kv_head_num"], params["qk_scale"], params["mask_type"])
    spent = time.perf_counter() - s0
    flops = FLOP_PER_PAIR * params["head_num"] * visible_pairs(qs, ks, params["mask_type"])
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "the whole workload", "seconds": round(spent, 4)}


def _time(fn, steps, stream):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_paged(steps, cpu=True):
    """The paged workload: the gather's bandwidth, then attention over the same
    caches two ways -- fused (mla_prefill_paged reads K/KRope/V through the
    block table) and two-step (gather, then mla_prefill on the gathered
    tensors). Queries: qlen = kvlen = context length, causal, 128 heads, bf16."""
    lens, _ = synth.workload_seqlens("paged")
    caches = synth.paged_inputs(lens, device="cuda", with_rope=True)
    total = int(lens.sum())
    heads = caches["key_cache"].shape[2]
    key = torch.empty((total, heads, 128), dtype=torch.bfloat16, device="cuda")
    value = torch.empty_like(key)
    rope = torch.empty((total, heads, 64), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def gather():
        mla.paged_cache_load(caches["key_cache"], caches["value_cache"], caches["block_tables"],
                             caches["context_lens"], key, value, None, mla.KV_CACHE_ND, False, False, stream)
        mla.paged_cache_load(caches["rope_cache"], None, caches["block_tables"], caches["context_lens"], rope,
                             None, None, mla.KV_CACHE_ND, False, False, stream)

    gather_ms = _time(gather, steps, stream)
    nbytes = 2 * total * (key[0].numel() + value[0].numel() + rope[0].numel()) * 2  # read + write
    gbs = nbytes / (gather_ms * 1e-3) / 1e9
    gather_rec = {"workload": "paged", "tokens": total, "bytes_per_step": nbytes, "ms_per_step": gather_ms,
                  "value": gbs, "unit": "GB/s", "peak": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS}

    qs = ks = np.asarray(lens, np.int32)
    q = synth._randn((total, heads, 128), torch.bfloat16, 1.0, 4 * 100 + 8, "cuda")
    qr = synth._randn((total, heads, 64), torch.bfloat16, 1.0, 4 * 100 + 9, "cuda")
    out = torch.empty((total, heads, 128), dtype=torch.bfloat16, device="cuda")
    mt = synth.MASK_CAUSAL
    ws_c = mla.mla_prefill_get_workspace_size(q, qr, key, rope, value, qs, ks, None, heads, synth.QK_SCALE, heads,
                                              mt, 0, out)
    ws_p = mla.mla_prefill_paged_get_workspace_size(q, qr, caches["key_cache"], caches["rope_cache"],
                                                    caches["value_cache"], caches["block_tables"], qs, ks, None,
                                                    heads, synth.QK_SCALE, heads, mt, out)
    ws = torch.empty(max(ws_c, ws_p, 1), dtype=torch.uint8, device="cuda")
    attn_steps = max(1, min(steps, 2))
    gathered_ms = _time(lambda: mla.mla_prefill(q, qr, key, rope, value, qs, ks, None, heads, synth.QK_SCALE,
                                                heads, mt, 0, out, ws, stream), attn_steps, stream)
    fused_ms = _time(lambda: mla.mla_prefill_paged(q, qr, caches["key_cache"], caches["rope_cache"],
                                                   caches["value_cache"], caches["block_tables"], qs, ks, None,
                                                   heads, synth.QK_SCALE, heads, mt, out, ws, stream),
                     attn_steps, stream)
    flops = FLOP_PER_PAIR * heads * visible_pairs(qs, ks, mt)
    del key, value, rope, out, ws
    oracle_rec = None
    if cpu:
        oracle_rec = oracle_sampled({"q": q, "q_rope": qr}, qs, ks, heads, heads, mt, synth.WORKLOADS["paged"]["seed"],
                                    paged=caches, pairs=128, rows_per_pair=16)
    del caches, q, qr
    torch.cuda.empty_cache()
    attn_rec = {"workload": "paged", "tokens": total, "heads": heads, "mask": "causal", "block_size":
                synth.BLOCK_SIZE, "flops_per_step": flops, "fused_ms": fused_ms,
                "fused_tflops": flops / (fused_ms * 1e-3) / 1e12, "gathered_attention_ms": gathered_ms,
                "two_step_ms": gather_ms + gathered_ms, "fused_speedup_over_two_step":
                (gather_ms + gathered_ms) / fused_ms}
    return gather_rec, attn_rec, oracle_rec


def bench_gather_nz(steps):
    """The paged workload's gather with the caches in the NZ layout (the same
    lengths, table and bytes as the ND leg; contents are random bit patterns,
    which a copy does not look at)."""
    lens, _ = synth.workload_seqlens("paged")
    meta = synth.paged_inputs(lens, heads=1, head_size_k=16, head_size_v=16, with_rope=False, device="cuda")
    table, ctx = meta["block_tables"], meta["context_lens"]
    nb, bs, heads = meta["key_cache"].shape[0], synth.BLOCK_SIZE, 128
    del meta

    def nz_cache(head_size):
        return torch.empty((nb, heads * head_size // 16, bs, 16), dtype=torch.int16,
                           device="cuda").random_().view(torch.bfloat16)

    kc, vc, rc = nz_cache(128), nz_cache(128), nz_cache(64)
    total = int(lens.sum())
    key = torch.empty((total, heads * 128), dtype=torch.bfloat16, device="cuda")
    value = torch.empty_like(key)
    rope = torch.empty((total, heads * 64), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def gather():
        mla.paged_cache_load(kc, vc, table, ctx, key, value, None, mla.KV_CACHE_NZ, False, False, stream)
        mla.paged_cache_load(rc, None, table, ctx, rope, None, None, mla.KV_CACHE_NZ, False, False, stream)

    ms = _time(gather, steps, stream)
    nbytes = 2 * total * (key[0].numel() + value[0].numel() + rope[0].numel()) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    del kc, vc, rc, key, value, rope
    torch.cuda.empty_cache()
    return {"workload": "paged", "layout": "NZ", "tokens": total, "bytes_per_step": nbytes, "ms_per_step": ms,
            "value": gbs, "unit": "GB/s", "peak": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS}


def bench_prolog(steps):
    """The non-quantised MLA prolog (NEXT-4) on its measured workload: 16384
    tokens at the sizes the MlaProlog page's constraints name (h 4096,
    q_lora_rank 1024, 64 heads x 512, rope 64); random-init bf16 weights.
    FLOPs are the three products' 2 * M * N * K; the norms and the rope are
    not counted."""
    t = synth.PROLOG_TOKENS
    d = synth.prolog_inputs(t, seed=1, device="cuda")
    hd, r = d["wkv"].shape[1], d["wq_a"].shape[1]
    heads = d["wq_b"].shape[1] // hd
    q = torch.empty((t, heads, hd), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((t, hd), dtype=torch.bfloat16, device="cuda")
    cq = torch.empty((t, r), dtype=torch.bfloat16, device="cuda")
    eps = synth.PROLOG_EPS
    args = (d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"], d["gamma_cq"],
            d["gamma_ckv"], eps, q, kv, cq)
    ws = torch.empty(max(mla.mla_prolog_get_workspace_size(*args), 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ms = _time(lambda: mla.mla_prolog(*args, ws, stream), steps, stream)
    # the same calls with the weights packed once (mla_prolog_pack_weights,
    # outside the timed region: it depends on the weights only)
    packed = mla.pack_prolog_weights(d["wq_a"], d["wq_b"], d["wkv"])
    wsp = torch.empty(max(mla.mla_prolog_prepacked_workspace_size(d["token_x"], d["wq_a"]), 1), dtype=torch.uint8,
                      device="cuda")
    ms_pp = _time(lambda: mla.mla_prolog_prepacked(*args, packed, wsp, stream), steps, stream)
    flops = synth.PROLOG_FLOP_PER_TOKEN * t
    tf = flops / (ms * 1e-3) / 1e12
    tf_pp = flops / (ms_pp * 1e-3) / 1e12
    del d, q, kv, cq, ws, packed, wsp
    torch.cuda.empty_cache()
    return {"workload": "prolog", "tokens": t, "sizes": dict(synth.PROLOG_SIZES), "flop_per_step": flops,
            "ms_per_step": ms, "value": tf, "unit": "TFLOP/s", "peak": PEAK_TFLOPS, "frac": tf / PEAK_TFLOPS,
            "prepacked": {"ms_per_step": ms_pp, "value": tf_pp, "frac": tf_pp / PEAK_TFLOPS}}


def bench_prolog_quant(steps):
    """The quantised MLA prolog (NEXT-4, mla_prolog_quant) on the same
    16384-token workload: x . [wq_a | wkv] in bf16 and qr . wq_b in int8
    (int8 weights with per-column scales, synth.prolog_quant_inputs). The
    roofline is per precision: the least time is the bf16 FLOPs at the bf16
    peak plus the int8 operations at the int8 peak, and frac is that time over
    the measured one."""
    t = synth.PROLOG_TOKENS
    d = synth.prolog_quant_inputs(t, seed=1, device="cuda")
    hd, r, h = d["wkv"].shape[1], d["wq_a"].shape[1], d["wq_a"].shape[0]
    heads = d["wq_b"].shape[1] // hd
    q = torch.empty((t, heads, hd), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((t, hd), dtype=torch.bfloat16, device="cuda")
    qr = torch.empty((t, r), dtype=torch.int8, device="cuda")
    qs = torch.empty((t, 1), dtype=torch.float32, device="cuda")
    eps = synth.PROLOG_EPS
    args = (d["token_x"], d["wq_a"], d["wq_b"], d["wkv"], d["rope_cos"], d["rope_sin"], d["gamma_cq"],
            d["gamma_ckv"], d["wq_b_scale"], eps, q, kv, qr, qs)
    ws = torch.empty(max(mla.mla_prolog_quant_get_workspace_size(*args), 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ms = _time(lambda: mla.mla_prolog_quant(*args, ws, stream), steps, stream)
    packed = mla.pack_prolog_weights(d["wq_a"], d["wq_b"], d["wkv"])
    wsp = torch.empty(max(mla.mla_prolog_prepacked_workspace_size(d["token_x"], d["wq_a"]), 1), dtype=torch.uint8,
                      device="cuda")
    ms_pp = _time(lambda: mla.mla_prolog_quant_prepacked(*args, packed, wsp, stream), steps, stream)
    bf16_flops = 2 * t * h * (r + hd)
    int8_ops = 2 * t * r * heads * hd
    least_ms = (bf16_flops / (PEAK_TFLOPS * 1e12) + int8_ops / (PEAK_INT8_TOPS * 1e12)) * 1e3
    del d, q, kv, qr, qs, ws, packed, wsp
    torch.cuda.empty_cache()
    return {"workload": "prolog_quant", "tokens": t, "sizes": dict(synth.PROLOG_SIZES), "bf16_flop_per_step":
            bf16_flops, "int8_op_per_step": int8_ops, "ms_per_step": ms,
            "value": (bf16_flops + int8_ops) / (ms * 1e-3) / 1e12, "unit": "TOP/s (bf16 FLOP + int8 OP)",
            "least_ms_at_peaks": least_ms, "frac": least_ms / ms,
            "prepacked": {"ms_per_step": ms_pp, "value": (bf16_flops + int8_ops) / (ms_pp * 1e-3) / 1e12,
                          "frac": least_ms / ms_pp}}


def _progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="single", choices=["single", "varlen", "chunked", "tiny"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain copy of known size first (for scaling rocprofv3 HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                    help="turn FETCH_SIZE / WRITE_SIZE rocprofv3 runs into HBM bytes per launch, then exit")
    ap.add_argument("--summarize-util", nargs="+", metavar="ARG",
                    help="WORKLOAD OUT_JSON DIR [DIR ...]: medians and derived utilisation of mla_fwd_kernel "
                         "from rocprofv3 --pmc runs of the UTIL_PASSES counters, then exit")
    ap.add_argument("--prolog-quant-only", action="store_true",
                    help="time only the quantised MLA prolog leg and print its JSON object")
    ap.add_argument("--prolog-only", action="store_true",
                    help="time only the MLA prolog leg and print its JSON object (for profiling it)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_util:
        summarize_util(args.summarize_util[0], args.summarize_util[1], args.summarize_util[2:])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(the path runs on a single MI355X, without collectives).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.prolog_only:
        print(json.dumps(bench_prolog(args.steps)), flush=True)
        return
    if args.prolog_quant_only:
        print(json.dumps(bench_prolog_quant(args.steps)), flush=True)
        return
    if args.calibrate_copy:
        calibration_copy()
    res = bench_attention(args.workload, args.steps, args.warmup)
    _progress(f"{args.workload}: {res['launch_ms']:.4f} ms per launch")
    flops = res["flops"]
    value = flops / (res["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (res["launch_ms"] * 1e-3) / 1e12
    w = synth.WORKLOADS[args.workload]
    dtype = "bf16" if w["dtype"] == torch.bfloat16 else "fp16"
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": args.workload, "batch": len(res["qs"]),
                   "q_seqlen": [int(x) for x in res["qs"]] if len(res["qs"]) <= 16 else "varlen",
                   "kv_seqlen": [int(x) for x in res["ks"]] if len(res["ks"]) <= 16 else "varlen",
                   "heads": w["heads"], "kv_heads": w["kv_heads"], "embeddim_v": 128, "rope_dim": 64,
                   "mask": "causal", "flops_per_step": flops},
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic_from_profile(),
                     "kernel": "mla_fwd_kernel", "avg_launch_ms": round(res["launch_ms"], 4),
                     "min_launch_ms": round(res["launch_ms_min"], 4)},
    }
    if not args.no_gather and args.workload == "single":
        res_t = res.pop("tensors") if args.no_cpu_baseline else None
        cpu = not args.no_cpu_baseline
        by_config = {}
        line["configs"] = bench_configs(max(5, min(args.steps, 20)), cpu)
        for name, rec in line["configs"].items():
            if "cpu_baseline" in rec:
                by_config[name] = rec.pop("cpu_baseline")
        _progress("varlen and tiny done")
        line["gather"], line["paged_attention"], by_config["paged"] = bench_paged(max(2, min(args.steps, 5)), cpu)
        _progress("paged done")
        line["gather_nz"] = bench_gather_nz(max(2, min(args.steps, 5)))
        line["extras"], extra_cpu = bench_extras(max(3, min(args.steps, 10)), cpu)
        by_config.update(extra_cpu)
        _progress("extras done")
        line["prolog"] = bench_prolog(max(3, min(args.steps, 10)))
        line["prolog_quant"] = bench_prolog_quant(max(3, min(args.steps, 10)))
        _progress("prolog done")
        if cpu:
            line["cpu_baseline_by_config"] = by_config
        del res_t
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(res, args.cpu_seconds)
        _progress("cpu baseline done")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
