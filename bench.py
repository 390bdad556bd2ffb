"""Throughput of one sequence-sharded MLA decode step on one MI355X.

A step is the whole hot path over one batch: the partial decode of every
emulated shard (one launch over all shards) followed by the LSE merge of the
shard partials.  Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line.  `value` is the achieved HBM bandwidth of the step in
GB/s, counting algorithmic bytes only (every attended cache row once, the
query once, each shard partial written once and read once, the final output
once); `kv_tokens_per_s` and `pct_of_peak` ride along.  The `roofline` object
reports the dominant kernel (the partial decode launch) timed with HIP events
on the stream it runs on; `cpu_baseline` times the float64 oracle on a bounded
sample of the same workload on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "dense_bf16_32k"
METRIC = "MLA decode attention: achieved HBM GB/s (% of peak) and KV tokens/s at 32K"
KERNEL_SOURCES = ["decode_valu.hpp", "decode_mfma.hpp", "decode_fp8.hpp", "mfma_common.hpp", "common.hpp",
                  "params.hpp", "api.hip",
                  "reduce.hpp", "plan.hpp", "host.cpp"]
# the sources a decode step's kernels are compiled from, per cache dtype: the
# kernel family of that dtype plus the shared helpers, plan, combine, merge
# and launch code (each family's header includes no other family's)
_DECODE_SHARED = ["mfma_common.hpp", "common.hpp", "params.hpp", "api.hip", "reduce.hpp", "plan.hpp", "host.cpp"]
DECODE_SOURCES = {"bf16": ["decode_mfma.hpp", "sparse_list.hpp"] + _DECODE_SHARED,
                  "fp8_ds": ["decode_fp8.hpp"] + _DECODE_SHARED,
                  "f32": ["decode_valu.hpp"] + _DECODE_SHARED}
WRITE_SOURCES = ["kv_write.hpp", "common.hpp", "api.hip"]
TOPK_SOURCES = ["topk.hpp", "common.hpp", "api.hip"]
TOPK_METRIC = "DCP top-K index selection: achieved HBM GB/s (% of peak) and rows/s, per-shard top-2048 + merge"
VARLEN_METRIC = ("MLA varlen decode attention (1 or 2 query tokens per request): achieved HBM GB/s "
                 "(% of peak) and KV tokens/s")
WRITE_METRIC = "DCP KV cache write: achieved HBM GB/s (% of peak) and tokens/s, 1M tokens over 8 shards"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(sources=KERNEL_SOURCES):
    """Hash of the kernel sources with comments and blank lines removed, so
    that recorded counters stay valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for name in sources:
        p = os.path.join(ROOT, "sequence_sharded_mla_amd", "csrc", name)
        if os.path.exists(p):
            text = open(p).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
            h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(x, out_bytes=2, q_bytes=2):
    """(step bytes, decode-launch bytes, attended KV tokens)."""
    from sequence_sharded_mla_amd.layout import ROW_BYTES
    sp = x.spec
    B, Tq, H, N = sp.batch, sp.q_len, sp.heads, sp.n_shards
    if x.topk_idx is None:
        tokens = int(sum(max(int(L) - Tq + j + 1, 0) for L in x.context_lens for j in range(Tq)))
        idx_bytes = 0
    else:
        tokens = int((x.topk_idx >= 0).sum())
        idx_bytes = x.topk_idx.size * 4
    kv = tokens * ROW_BYTES[sp.kv_dtype]
    q = B * Tq * H * 576 * q_bytes
    part = N * B * Tq * H * (512 * out_bytes + 4)
    final = B * Tq * H * (512 * out_bytes + 4)
    decode_launch = kv + q + idx_bytes + part
    step = decode_launch + part + final
    return step, decode_launch, tokens


def shard_bytes(x, s, out_bytes=2, q_bytes=2):
    """Algorithmic bytes of one shard's decode launch (what one DCP rank's
    call moves): its owned KV rows, the query, the index lists, its partials."""
    from sequence_sharded_mla_amd.layout import ROW_BYTES
    sp = x.spec
    B, Tq, H, N = sp.batch, sp.q_len, sp.heads, sp.n_shards
    if x.topk_idx is None:
        vis = [max(int(L) - Tq + j + 1, 0) for L in x.context_lens for j in range(Tq)]
        tokens = int(sum((v - s + N - 1) // N if v > s else 0 for v in vis))
        idx_bytes = 0
    else:
        g = x.topk_idx
        tokens = int(((g >= 0) & (g % N == s)).sum())
        idx_bytes = g.size * 4
    return tokens * ROW_BYTES[sp.kv_dtype] + B * Tq * H * 576 * q_bytes + idx_bytes + \
        B * Tq * H * (512 * out_bytes + 4), tokens


def copy_rate_gbs(reps=5):
    """Bytes moved (read + write) per second by a plain 1 GiB device copy,
    the median of `reps` copies: a practical HBM reference measured in the
    same run (a copy reaches less than a pure read stream)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    return 2 * n / (float(np.median(ts)) * 1e-3) / 1e9


def stream_read_gbs(reps=7, nbytes=4 << 30, grid=16384):
    """HBM streaming-read reference measured in the same run: bytes per
    second a read-only kernel (libmla_hbm_probe.so: 16-byte non-temporal
    loads, eight in flight per thread, 16384 workgroups) reaches over a 4 GiB
    buffer.  Returns (median, best) GB/s over `reps` launches."""
    import ctypes
    import torch
    from sequence_sharded_mla_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.mla_hbm_read_probe
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        if fn(buf.data_ptr(), nbytes, grid, sink.data_ptr(), stream.cuda_stream) != 0:
            raise RuntimeError("mla_hbm_read_probe failed")
    launch()
    torch.cuda.synchronize()
    ts = time_launches(launch, reps, stream)
    del buf
    return nbytes / (float(np.median(ts)) * 1e-3) / 1e9, nbytes / (float(ts.min()) * 1e-3) / 1e9


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x, budget_s=10.0):
    """Time the float64 oracle (shard partials + merge) on whole requests."""
    from threadpoolctl import threadpool_info
    from oracle import attention, decode as odecode
    sp = x.spec
    q = odecode.query_to_f64(x.q, sp.q_dtype)
    rows = odecode.storage_rows(sp.kv_dtype, x.latent, x.scales, x.rope, x.row_offsets, x.row_pos)
    done, tokens, t0 = 0, 0, time.perf_counter()
    while done < sp.batch and (time.perf_counter() - t0) < budget_s:
        b = done
        r = odecode.mla_decode(q, rows, x.context_lens, sp.q_len, sp.n_shards, sp.scale,
                               topk_idx=x.topk_idx, requests=[b], full=False)
        attention.merge(r["o_shards"], r["lse_shards"])
        if x.topk_idx is None:
            tokens += sum(max(int(x.context_lens[b]) - sp.q_len + j + 1, 0) for j in range(sp.q_len))
        else:
            tokens += int((x.topk_idx[b] >= 0).sum())
        done += 1
    dt = time.perf_counter() - t0
    from sequence_sharded_mla_amd.layout import ROW_BYTES
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    kv_bytes = tokens * ROW_BYTES[sp.kv_dtype]
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s",
            "kv_tokens_per_s": round(tokens / dt, 1), "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{done} of {sp.batch} requests (all {sp.n_shards} shards + merge), "
                      f"{tokens} attended tokens, {dt:.1f} s"}


def profile_record(workload, khash):
    """The committed counter record of a workload (profiles/traffic_*.json),
    or None when the kernel sources have changed since it was taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    return rec if rec.get("kernel_hash") == khash else None


def traffic_for(workload, khash):
    rec = profile_record(workload, khash)
    return None if rec is None else rec.get("bytes_per_launch")


def write_bytes_per_token(src_dtype, kv_dtype):
    """Algorithmic bytes of one written token: source row, request id and
    position (int32 each), cache row."""
    from sequence_sharded_mla_amd.layout import ROW_BYTES
    return (576 * (2 if src_dtype == "bf16" else 4)) + 4 + 4 + ROW_BYTES[kv_dtype]


def write_cpu_baseline(src, tables, w, budget_s=10.0):
    """Time the oracle's slot mapping + row encoding on a prefix of the tokens."""
    from oracle import kv_write as okw
    n_shards = w["n_shards"]
    pool_blocks = int(tables.max()) + 1
    done, chunk, t0 = 0, 256, time.perf_counter()
    while done < src.shape[0] and (time.perf_counter() - t0) < budget_s:
        rows = src[done:done + chunk]
        f = (rows.astype(np.uint32) << 16).view(np.float32) if w["src_dtype"] == "bf16" else rows
        pos = np.arange(done, done + rows.shape[0])
        slots, _ = okw.dcp_slot_mapping(np.zeros(pos.size, np.int64), pos, tables, 0, n_shards,
                                        n_shards, pool_blocks)
        for i in range(rows.shape[0]):
            okw.row_bytes_for(f[i], w["kv_dtype"])
        done += rows.shape[0]
    dt = time.perf_counter() - t0
    per = write_bytes_per_token(w["src_dtype"], w["kv_dtype"])
    return {"value": round(done * per / dt / 1e9, 6), "unit": "GB/s",
            "tokens_per_s": round(done / dt, 1), "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {src.shape[0]} tokens (slot mapping + row encoding), {dt:.1f} s"}


def time_launches(fn, K, stream):
    import torch
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(K)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def topk_cpu_baseline(scores, lens, w, budget_s=10.0):
    """Time the oracle's per-shard selection + merge on whole rows."""
    from oracle import topk as otk
    B, Tq, K, N = w["batch"], w["q_len"], w["topk"], w["n_shards"]
    done, t0 = 0, time.perf_counter()
    while done < B and (time.perf_counter() - t0) < budget_s:
        sl = slice(done, done + 1)
        parts = [otk.local_topk(scores[sl], lens[sl], Tq, K, s, N) for s in range(N)]
        otk.merge_topk(np.stack([p.reshape(Tq, K) for p, _ in parts]),
                       np.stack([c.reshape(Tq, K) for _, c in parts]), K)
        done += 1
    dt = time.perf_counter() - t0
    score_bytes = done * Tq * w["context"] * 4
    return {"value": round(score_bytes / dt / 1e9, 6), "unit": "GB/s",
            "rows_per_s": round(done * Tq / dt, 2), "cores": 1, "kind": "oracle",
            "sample": f"{done} of {B} requests ({done * Tq} rows, all {N} shards + merge), {dt:.1f} s"}


def run_topk(args):
    """Top-K selection for every query token of the sparse workload: each
    shard's local top-K (all shards in one launch), then the merge."""
    import torch
    import workload
    from sequence_sharded_mla_amd import layout, mla_topk_local, mla_topk_merge
    name = "topk_select_262k"
    w = workload.SELECT_SPECS[name]
    B, Tq, L, K, N = w["batch"], w["q_len"], w["context"], w["topk"], w["n_shards"]
    log(f"bench: generating {name}")
    scores = workload.indexer_scores(B, Tq, L, seed=w["seed"])
    lens = np.full(B, L, dtype=np.int32)
    sc_sh = layout.shard_scores(scores, N)
    d_sc = torch.from_numpy(sc_sh).cuda()
    d_lens = torch.from_numpy(lens).cuda()
    rows = B * Tq
    ci = torch.empty((N, B, Tq, K), dtype=torch.int32, device="cuda")
    cs = torch.empty((N, B, Tq, K), dtype=torch.float32, device="cuda")
    out = torch.empty((rows, K), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def local():
        mla_topk_local(d_sc, d_lens, K, 0, N, ci, cs)

    def merge():
        mla_topk_merge(ci.view(N, rows, K), cs.view(N, rows, K), K, out)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        local()
        merge()
    torch.cuda.synchronize()
    K_steps = args.steps
    log(f"bench: timing {K_steps} steps")
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(K_steps)]
    t0 = time.perf_counter()
    for a, b, c in ev:
        a.record(stream)
        local()
        b.record(stream)
        merge()
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_loc = np.array([a.elapsed_time(b) for a, b, _ in ev])
    t_mer = np.array([b.elapsed_time(c) for _, b, c in ev])
    ms_step = wall * 1e3 / K_steps
    # every owned score read once; candidates written once and read once; result written once
    local_bytes = B * Tq * L * 4 + B * 4 + N * rows * K * 8
    merge_bytes = N * rows * K * 8 + rows * K * 4
    step_bytes = local_bytes + merge_bytes
    loc_ms = float(np.mean(t_loc))
    achieved = local_bytes / (loc_ms * 1e-3) / 1e9
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    khash = kernel_hash(TOPK_SOURCES)
    rec = {
        "metric": TOPK_METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) indexer scores)",
        "config": {"workload": name, "batch": B, "q_len": Tq, "context": L, "topk": K, "n_shards": N},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "rows_per_s": round(rows / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kernels_ms": {"local_topk": round(loc_ms, 4), "merge_topk": round(float(np.mean(t_mer)), 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(name, khash),
                     "kernel": "local_topk_kernel (all shards, one launch)",
                     "algorithmic_bytes_per_launch": int(local_bytes)},
        "kernel_hash": khash,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        rec["cpu_baseline"] = topk_cpu_baseline(scores, lens, w, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def run_kv_write(args):
    """Cache write of one request's 1M new tokens, dealt over 8 shards held in
    one pool: the fused owner-slot + quantise-and-store call (one launch)."""
    import torch
    import workload
    from sequence_sharded_mla_amd import (layout, mla_clear_device_error, mla_dcp_kv_write,
                                          mla_dcp_slot_mapping, mla_get_device_error, mla_kv_write)
    name = "kv_write_fp8_1m"
    w = workload.WRITE_SPECS[name]
    T, N, kv = w["tokens"], w["n_shards"], w["kv_dtype"]
    log(f"bench: generating {name}")
    src = workload.new_token_rows(T, seed=w["seed"], dtype=w["src_dtype"])
    tables, blocks = layout.build_block_tables(np.array([T]), N, seed=w["seed"])
    rb = layout.ROW_BYTES[kv]
    d_src = torch.from_numpy(src.view(np.int16)).cuda().view(torch.bfloat16)
    d_req = torch.zeros(T, dtype=torch.int32, device="cuda")
    d_pos = torch.arange(T, dtype=torch.int32, device="cuda")
    d_tab = torch.from_numpy(tables).cuda()
    d_tab0 = torch.from_numpy(np.ascontiguousarray(tables[:1])).cuda()
    d_slots = torch.empty(T, dtype=torch.int64, device="cuda")
    pool = torch.zeros(blocks * 64 * rb, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    mla_clear_device_error(ws)
    stream = torch.cuda.current_stream()

    def step():
        mla_dcp_kv_write(d_src, d_req, d_pos, d_tab, 0, N, pool, kv, blocks, workspace=ws)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    log(f"bench: timing {K} steps")
    t0 = time.perf_counter()
    t_step = time_launches(step, K, stream)
    wall = time.perf_counter() - t0
    # the same write as two calls (slot array, then write) and one rank's call
    extras = not args.no_extras
    nan = np.array([np.nan])
    t_map = time_launches(lambda: mla_dcp_slot_mapping(d_req, d_pos, d_tab, 0, N, blocks, d_slots,
                                                       workspace=ws), K, stream) if extras else nan
    t_two = time_launches(lambda: mla_kv_write(d_src, d_slots, pool, kv, blocks, workspace=ws), K,
                          stream) if extras else nan
    t_rank = time_launches(lambda: mla_dcp_kv_write(d_src, d_req, d_pos, d_tab0, 0, N, pool, kv, blocks,
                                                    workspace=ws), K, stream) if extras else nan
    assert mla_get_device_error(ws) == 0
    ms_step = wall * 1e3 / K
    per = write_bytes_per_token(w["src_dtype"], kv)
    launch_bytes = T * per + tables.size * 4
    wr_ms = float(np.mean(t_step))
    achieved = launch_bytes / (wr_ms * 1e-3) / 1e9
    gbs = launch_bytes / (ms_step * 1e-3) / 1e9
    khash = kernel_hash(WRITE_SOURCES)
    rank_bytes = (T // N) * (per - 8) + T * 8 + tables[:1].size * 4
    rec = {
        "metric": WRITE_METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) bf16 rows, random-permuted paged blocks)",
        "config": {"workload": name, "tokens": T, "n_shards": N, "source": w["src_dtype"],
                   "kv_cache": kv, "block_size": 64},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": int(launch_bytes),
        "kernels_ms": {"dcp_kv_write": round(wr_ms, 4),
                       "dcp_kv_write_p10_p90": [round(float(np.percentile(t_step, 10)), 4),
                                                round(float(np.percentile(t_step, 90)), 4)],
                       "two_calls": {"slot_mapping": round(float(np.mean(t_map)), 4),
                                     "kv_write": round(float(np.mean(t_two)), 4)} if extras else None,
                       "one_rank_of_8": round(float(np.mean(t_rank)), 4) if extras else None,
                       "one_rank_of_8_gbs": round(rank_bytes / (float(np.mean(t_rank)) * 1e-3) / 1e9, 1)
                       if extras else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(name, khash),
                     "kernel": "kv_write_kernel<bf16, fp8_ds, fused> (all shards, one launch)",
                     "algorithmic_bytes_per_launch": int(launch_bytes)},
        "kernel_hash": khash,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        rec["cpu_baseline"] = write_cpu_baseline(src, tables, w, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def varlen_cpu_baseline(x, q, qsl, budget_s=10.0):
    """Time the float64 oracle's varlen step (shard partials + merge) on
    whole requests, one request's tokens per call."""
    from threadpoolctl import threadpool_info
    from oracle import decode as odecode
    sp = x.spec
    qf = odecode.query_to_f64(q, sp.q_dtype)
    rows = odecode.storage_rows(sp.kv_dtype, x.latent, x.scales, x.rope, x.row_offsets, x.row_pos)
    done, tokens, t0 = 0, 0, time.perf_counter()
    while done < sp.batch and (time.perf_counter() - t0) < budget_s:
        b = done
        toks = list(range(int(qsl[b]), int(qsl[b + 1])))
        if toks:
            odecode.mla_decode_varlen(qf, rows, x.context_lens, qsl, sp.n_shards, sp.scale,
                                      tokens=toks)
        c = len(toks)
        tokens += sum(max(int(x.context_lens[b]) - c + t + 1, 0) for t in range(c))
        done += 1
    dt = time.perf_counter() - t0
    from sequence_sharded_mla_amd.layout import ROW_BYTES
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(tokens * ROW_BYTES[sp.kv_dtype] / dt / 1e9, 4), "unit": "GB/s",
            "kv_tokens_per_s": round(tokens / dt, 1), "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {sp.batch} requests ({int(qsl[done])} query tokens, all "
                      f"{sp.n_shards} shards + merge), {tokens} attended tokens, {dt:.1f} s"}


def run_varlen(args):
    """Varlen decode step: requests of the fp8 mixed-length cache carry one
    or two query tokens (multi-token-prediction drafts) in one call."""
    import torch
    import workload
    from sequence_sharded_mla_amd import layout, mla_get_device_error
    from sequence_sharded_mla_amd.layout import ROW_BYTES
    from sequence_sharded_mla_amd.step import VarlenDecodeStep
    name = "varlen_fp8_mtp2"
    w = workload.VARLEN_SPECS[name]
    sp = workload.SPECS[w["base"]].with_(q_len=w["q_len"])
    log(f"bench: generating {name} ({sp.name} with {sp.q_len} query tokens per request)")
    x = workload.generate(sp)
    counts = workload.varlen_counts(sp.batch, sp.q_len, w["seed"])
    sel = [(b, j) for b, c in enumerate(counts) for j in range(sp.q_len - int(c), sp.q_len)]
    q = np.stack([x.q[b, j] for b, j in sel])
    qsl = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n_q = int(qsl[-1])
    cache = layout.pack(x, device="cuda")
    dq = torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).cuda().view(torch.bfloat16)
    step = VarlenDecodeStep(cache, sp.out_dtype, dq, torch.from_numpy(qsl).cuda())
    stream = torch.cuda.current_stream()

    H, N = sp.heads, sp.n_shards
    tokens = int(sum(max(int(L) - int(c) + t + 1, 0)
                     for L, c in zip(x.context_lens, counts) for t in range(int(c))))
    part = N * n_q * H * (512 * 2 + 4)
    launch_bytes = tokens * ROW_BYTES[sp.kv_dtype] + n_q * H * 576 * 2 + qsl.size * 4 + part
    step_bytes = launch_bytes + part + n_q * H * (512 * 2 + 4)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert mla_get_device_error(step.workspace) == 0
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    log(f"bench: timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        a, b, c = ev[i]
        a.record(stream)
        step.partials()
        b.record(stream)
        step.merge()
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_part = np.array([e[0].elapsed_time(e[1]) for e in ev])
    t_merge = np.array([e[1].elapsed_time(e[2]) for e in ev])
    assert mla_get_device_error(step.workspace) == 0
    ms_step = wall * 1e3 / K
    part_ms = float(np.mean(t_part))
    achieved = launch_bytes / (part_ms * 1e-3) / 1e9
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    khash = kernel_hash(DECODE_SOURCES[sp.kv_dtype])
    rec = {
        "metric": VARLEN_METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) query/latent/rope, random-permuted paged blocks, "
                "seeded query counts)",
        "config": {"workload": name, "batch": sp.batch, "q_len_max": sp.q_len,
                   "query_tokens": n_q, "heads": H, "context": list(sp.ctx_range),
                   "n_shards": N, "kv_cache": sp.kv_dtype, "block_size": 64},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "kv_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kernels_ms": {"decode_partials": round(part_ms, 4),
                       "decode_partials_median": round(float(np.median(t_part)), 4),
                       "lse_merge": round(float(np.mean(t_merge)), 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(name, khash),
                     "kernel": "varlen decode partials (all shards, one launch)",
                     "algorithmic_bytes_per_launch": int(launch_bytes)},
        "kernel_hash": khash,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        rec["cpu_baseline"] = varlen_cpu_baseline(x, q, qsl, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--kv-write", action="store_true",
                    help="time the cache write (owner slot mapping + quantise-and-store) instead "
                         "of the decode step")
    ap.add_argument("--topk", action="store_true",
                    help="time the top-K index selection (per-shard local top-K + merge)")
    ap.add_argument("--varlen", action="store_true",
                    help="time the varlen decode step (1 or 2 query tokens per request)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the timed region's launches (for profiling): with --kv-write the "
                         "fused all-shard call; for the decode step no cold-cache, single-shard or "
                         "copy series")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy three times (HBM counter calibration)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only run the 4 GiB streaming-read probe three times (counter reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sharded step is emulated on a single device)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return
    if args.stream_probe:
        med, best = stream_read_gbs(reps=3)
        print(json.dumps({"stream_probe_bytes": 4 << 30, "launches": 5, "median_gbs": round(med, 1),
                          "best_gbs": round(best, 1)}), flush=True)
        return
    if args.kv_write:
        run_kv_write(args)
        return
    if args.topk:
        run_topk(args)
        return
    if args.varlen:
        run_varlen(args)
        return
    import workload
    from sequence_sharded_mla_amd import layout, mla_get_device_error
    from sequence_sharded_mla_amd.step import ShardedDecodeStep

    sp = workload.SPECS[args.workload]
    log(f"bench: generating {sp.name}")
    t0 = time.perf_counter()
    x = workload.generate(sp)
    log(f"bench: generated {x.total_rows} rows in {time.perf_counter() - t0:.1f} s; packing")
    cache = layout.pack(x, device="cuda")
    step = ShardedDecodeStep(cache, sp.out_dtype)
    stream = torch.cuda.current_stream()
    out_b = 2 if sp.out_dtype == "bf16" else 4
    q_b = 2 if sp.q_dtype == "bf16" else 4
    step_bytes, launch_bytes, tokens = algorithmic_bytes(x, out_b, q_b)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert mla_get_device_error(step.workspace) == 0

    # Timed region: K steps, each after a 1 GiB write (outside its events) that
    # evicts the 256 MB last-level cache, so no cache row of the previous step
    # is served from it, then a 512 MiB read of a clean buffer (also outside
    # the events) that pushes the write's dirty lines out of the cache: left
    # there, their write-back to HBM would run during the step and compete
    # with its reads.  The step's time is its own events (partials, then
    # merge); the flush kernels run on the same stream between them.  The same
    # K steps after the write alone are reported beside it.
    K = args.steps
    evict = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    clean = torch.ones(1 << 27, dtype=torch.int32, device="cuda")  # 512 MiB

    def timed_series(clean_read):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            evict.fill_(i & 0xff)
            if clean_read:
                clean.sum()
            a, b, c = ev[i]
            a.record(stream)
            step.partials()
            b.record(stream)
            step.merge()
            c.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        t_part = np.array([e[0].elapsed_time(e[1]) for e in ev])
        t_merge = np.array([e[1].elapsed_time(e[2]) for e in ev])
        return t_part, t_merge, wall

    log(f"bench: timing {K} steps (cache flushed before each)")
    t_part, t_merge, wall = timed_series(True)
    t_step = t_part + t_merge
    ms_per_step = float(np.mean(t_step))
    assert mla_get_device_error(step.workspace) == 0
    flush_w = None
    if not args.no_extras:
        tw_part, tw_merge, _ = timed_series(False)
        flush_w = {"note": "the same steps after the 1 GiB write alone (its dirty lines written back "
                           "during the step)",
                   "ms_per_step": round(float(np.mean(tw_part + tw_merge)), 4),
                   "decode_partials_mean_ms": round(float(np.mean(tw_part)), 4),
                   "decode_frac": round(launch_bytes / (float(np.mean(tw_part)) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        assert mla_get_device_error(step.workspace) == 0
    del evict, clean

    extras = not args.no_extras
    # Warm series (secondary): K steps back to back, no flush.
    warm = None
    if extras:
        ev_w = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                 torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        tw0 = time.perf_counter()
        for a, b, c in ev_w:
            a.record(stream)
            step.partials()
            b.record(stream)
            step.merge()
            c.record(stream)
        torch.cuda.synchronize()
        wall_w = time.perf_counter() - tw0
        tw_part = np.array([e[0].elapsed_time(e[1]) for e in ev_w])
        tw_merge = np.array([e[1].elapsed_time(e[2]) for e in ev_w])
        warm = {"note": "back-to-back steps, no flush; wall-clock per step includes launch gaps",
                "ms_per_step_wall": round(wall_w * 1e3 / K, 4),
                "decode_partials_mean_ms": round(float(np.mean(tw_part)), 4),
                "decode_partials_median_ms": round(float(np.median(tw_part)), 4),
                "lse_merge_mean_ms": round(float(np.mean(tw_merge)), 4),
                "decode_frac": round(launch_bytes / (float(np.mean(tw_part)) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        assert mla_get_device_error(step.workspace) == 0

    # One shard's call, the launch one DCP rank makes for its share of the
    # cache (shard 0, its own block table and workspace).
    from sequence_sharded_mla_amd import alloc_workspace, mla_decode_partial
    d = cache.desc
    rows = d.batch * d.q_len
    o1 = torch.empty((rows, d.num_heads, 512), dtype=step.o_partials.dtype, device="cuda")
    l1 = torch.empty((rows, d.num_heads), dtype=torch.float32, device="cuda")
    ws1 = alloc_workspace(d, 1)
    bt0 = cache.block_tables[0].contiguous()

    def one_shard():
        mla_decode_partial(d, cache.q, cache.pool, bt0, cache.context_lens, cache.topk_idx, 0,
                           cache.n_shards, o1, l1, ws1)
    for _ in range(3 if extras else 0):
        one_shard()
    torch.cuda.synchronize()
    t_one = time_launches(one_shard, K, stream) if extras else np.array([np.nan])
    assert mla_get_device_error(ws1) == 0
    one_bytes, one_tokens = shard_bytes(x, 0, out_b, q_b)

    from sequence_sharded_mla_amd.layout import ROW_BYTES
    kv_bytes = tokens * ROW_BYTES[sp.kv_dtype]
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    part_ms = float(np.mean(t_part))
    achieved = launch_bytes / (part_ms * 1e-3) / 1e9
    khash = kernel_hash(DECODE_SOURCES[sp.kv_dtype])
    prof = profile_record(sp.name, khash)
    stream_med = stream_best = None
    if extras:
        stream_med, stream_best = stream_read_gbs()
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None if prof is None else prof.get("bytes_per_launch"),
                "kernel": "decode partials (all shards, one launch), flushed-cache steps, HIP events",
                "algorithmic_bytes_per_launch": int(launch_bytes),
                "decode_launch_mean_ms": round(part_ms, 4),
                "decode_launch_median_ms": round(float(np.median(t_part)), 4),
                "decode_launch_p10_p90_ms": [round(float(np.percentile(t_part, 10)), 4),
                                             round(float(np.percentile(t_part, 90)), 4)]}
    if stream_med:
        roofline["stream_read_gbs"] = round(stream_med, 1)
        roofline["frac_of_stream_read"] = round(achieved / stream_med, 4)
    if prof is not None and prof.get("kernel_avg_ns"):
        # the decode kernel alone, from the committed rocprofv3 trace of the
        # same kernel sources (kernel_hash)
        k_gbs = prof["kernel_bytes_per_launch"] / (prof["kernel_avg_ns"] * 1e-9) / 1e9
        roofline["profile_kernel"] = {"kernel": prof.get("kernel"), "avg_us": round(prof["kernel_avg_ns"] / 1e3, 1),
                                      "achieved_gbs": round(k_gbs, 1), "frac": round(k_gbs / PEAK_HBM_GBS, 4),
                                      "source": prof.get("source")}
    rec = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sp.q_dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) query/latent/rope, random-permuted paged blocks)",
        "config": {"workload": sp.name, "batch": sp.batch, "q_len": sp.q_len, "heads": sp.heads,
                   "context": sp.context or list(sp.ctx_range), "n_shards": sp.n_shards,
                   "kv_cache": sp.kv_dtype, "topk": sp.topk, "block_size": 64},
        "timing": "each step after a 1 GiB write and a 512 MiB clean read (cache evicted, no dirty "
                  "lines left), both outside the events; ms_per_step = mean of the steps' HIP-event "
                  "times (partials + merge)",
        "write_flush_only": flush_w,
        "wall_ms_per_step_incl_flush": round(wall * 1e3 / K, 4),
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "kv_tokens_per_s": round(tokens / (ms_per_step * 1e-3), 1),
        "kv_only_gbs": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kernels_ms": {"decode_partials": round(part_ms, 4),
                       "decode_partials_median": round(float(np.median(t_part)), 4),
                       "decode_partials_p10_p90": [round(float(np.percentile(t_part, 10)), 4),
                                                   round(float(np.percentile(t_part, 90)), 4)],
                       "lse_merge": round(float(np.mean(t_merge)), 4),
                       "step_median": round(float(np.median(t_step)), 4)},
        "warm": warm,
        "single_shard": None if not extras else {
            "note": "mla_decode_partial for shard 0 of the same cache (one rank's call), back to back",
            "median_ms": round(float(np.median(t_one)), 4),
            "algorithmic_bytes": int(one_bytes), "kv_tokens": one_tokens,
            "achieved_gbs": round(one_bytes / (float(np.median(t_one)) * 1e-3) / 1e9, 2),
            "frac": round(one_bytes / (float(np.median(t_one)) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "roofline": roofline,
        "kernel_hash": khash,
    }
    if extras:
        copy_gbs = copy_rate_gbs()
        rec["hbm_reference"] = {"copy_gbs": round(copy_gbs, 1),
                                "stream_read_gbs": round(stream_med, 1),
                                "stream_read_best_gbs": round(stream_best, 1),
                                "note": "same run: a 1 GiB device copy (read + write bytes) and the "
                                        "streaming-read probe over 4 GiB (read bytes)"}
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
