"""Benchmark: SPICY-KV compressed-KV decode on one MI355X.

One step = one pass of the whole hot path over one batch: spicy_coarsen of the
batch's fresh chunk into the paged cache (plan + segmented moments + RoPE +
pack), then the decode of one query token per sequence over the whole
compressed cache (split-K decode with the log-sum-exp combine in the same
launch).

Default workload: the shared-prefix batch (32 sequences sharing one
65536-token prefix compressed 28.6x, a private exact suffix of U[512, 2048]
tokens each, and a fresh 8192-token chunk per sequence coarsened every step
with equal-variation segments), Qwen2-7B head shape (28 query / 4 KV heads,
d = 128), bf16.  Other workloads: --workload qwen2_7b_layer | long_ragged |
qwen2_1.5b_layer | tiny_fp32 (those have no per-step coarsen; a step is their
whole coarsen + decode).

Prints ONE JSON line.  `value` = query tokens per second of K whole steps.
Per-call durations come from HIP events on the launch stream, with the calls
queued behind a sleep kernel so that no call waits for the host: `roofline`
describes the step's dominant call (largest median duration), and
`roofline_decode` the decode call, beside the streaming-read ceiling at its
byte count.  `decode_configs` adds the decode alone on the 7B layer and the
long ragged batch, over rotated cache copies.  `achieved` = algorithmic bytes
per call / mean call duration.  Inputs are resident in HBM before the timed
region.

The K timed steps replay one captured HIP graph of the step (`launch` in the
line; --eager issues every call from the host instead): the same kernels on
the same buffers, with one launch per step, so that a slow or loaded host does
not starve the GPU.  `step_us` and the per-call figures come from eagerly
issued steps.

Other modes: --decode-only (the decode call alone), --copy-calibration (the
known-size copy that scales rocprofv3's byte counters), --cu-probe (how fast
a few workgroups can read, against the whole chip), --summarize-profile DIR
(writes profiles/<name>.txt from rocprofv3 CSV output).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
DECODE_TARGET_FRAC = 0.70      # the target on compressed-cache decode: 70% of peak HBM bandwidth
DECODE_CONFIGS = ("qwen2_7b_layer", "long_ragged")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="shared_prefix")
    ap.add_argument("--splits", type=int, default=0, help="decode split count (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-decode-configs", action="store_true",
                    help="skip the decode-alone lines of the 7B layer and the long ragged batch")
    ap.add_argument("--decode-only", action="store_true",
                    help="diagnostic: time the decode call alone over rotated copies of the cache")
    ap.add_argument("--rotate-bytes", type=float, default=1.5e9,
                    help="decode-alone timing: total bytes of distinct cache copies rotated through")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device copy (torch.neg, fp32) 5 times: the known-size "
                         "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    ap.add_argument("--cu-probe", action="store_true",
                    help="streaming-read rate of N workgroups (one per CU up to 256), each reading about "
                         "600 KB, for N from 8 to 512: what one CU can pull against the whole chip")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="summarize rocprofv3 CSV output under DIR (trace/, FETCH_SIZE/, WRITE_SIZE/, "
                         "copy_FETCH_SIZE/, copy_WRITE_SIZE/, pmc_<counters>/) into profiles/<--profile-name>.txt")
    ap.add_argument("--profile-name", default=None, help="name of the summary file under profiles/")
    ap.add_argument("--profile-commands", default="",
                    help="the commands that produced DIR, recorded in the summary (one per ';')")
    ap.add_argument("--profile-last", type=int, default=0,
                    help="summary: also give the statistics of each kernel's last N dispatches (0 = 2 x steps)")
    ap.add_argument("--device-policy", action="store_true",
                    help="every step also runs spicy_policy on the chunk (equal-variation segments and "
                         "key-norm landmarks on the GPU) and coarsens with its output")
    ap.add_argument("--query-tokens", type=int, default=1,
                    help="query tokens per sequence in every decode call (spicy_decode_attn_multi when > 1, "
                         "as for speculative verification against the compressed cache)")
    ap.add_argument("--weighted", action="store_true",
                    help="with --device-policy: spicy_coarsen_weighted, the macro-nodes' keys and values weighted "
                         "by the policy's per-token variation")
    ap.add_argument("--merge", action="store_true",
                    help="every step also merges one dyadic level over the entries its coarsening wrote "
                         "(spicy_merge_level; the cache keeps its metadata), then gives the freed entries "
                         "back (spicy_compact_range): the decode reads the compacted cache")
    ap.add_argument("--no-compact", action="store_true",
                    help="with --merge: leave the merged range's nulls in place (the decode reads them)")
    ap.add_argument("--diag-closure", action="store_true",
                    help="the cache carries per-dimension variances (diagonal closure): coarsen writes them, "
                         "decode reads them in place of the scalar beta")
    ap.add_argument("--eager", action="store_true",
                    help="issue every call of each timed step from the host (default: one step captured "
                         "once as a HIP graph and replayed per step)")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="decode a shared-prefix batch with spicy_decode_attn (every page per sequence)")
    return ap.parse_args(argv)


def elem_bytes(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


def policy_alg_bytes(call, spec) -> int:
    """Bytes the policy must move: read K and V of every token of the chunk;
    write the protection mask and the segment offsets."""
    T, H, d = call.total_tokens, call.H_kv, call.d
    return 2 * T * H * d * elem_bytes(call.dtype) + T * H + 4 * (call.B * spec.n_segments + 1) + 4 * (call.B + 1)


def coarsen_alg_bytes(call, lengths: np.ndarray, diag: bool = False, weighted: bool = False,
                      meta: bool = False) -> int:
    """Bytes the coarsening must move: read K and V of every token and the
    mask (and with `weighted` one int64 weight per token); write every entry
    it produces (key row, value column, alpha, beta, with `diag` the variance
    row, with `meta` the 16-byte metadata record), null padding included."""
    eb = elem_bytes(call.dtype)
    T, H, d = call.total_tokens, call.H_kv, call.d
    read = T * H * d * 2 * eb + T * H + (8 * T if weighted else 0)
    written_entries = 0
    for b in range(call.B):
        end = -(-int(lengths[b]) // 16) * 16
        written_entries += H * (end - int(call.entry_start[b]))
    write = written_entries * (((3 if diag else 2) * d + 2) * eb + (16 if meta else 0)) + call.B * 4
    return read + write


def merge_pair_count(meta: np.ndarray, table: np.ndarray, entry_start, lengths) -> int:
    """Pairs one merge level forms: per sequence and KV head, half the
    macro-nodes (metadata kind 2) among entries [entry_start[b], lengths[b]),
    rounded down.  meta [pages, H, 16, 4] int32 records, table [B, max_pages]."""
    total = 0
    for b in range(table.shape[0]):
        e = np.arange(int(entry_start[b]), int(lengths[b]))
        kinds = meta[table[b, e // 16], :, e % 16, 0]            # [entries, H]
        total += int((np.count_nonzero(kinds == 2, axis=0) // 2).sum())
    return total


def merge_alg_bytes(call, lengths: np.ndarray, pairs: int) -> int:
    """Bytes one merge level must move: the 16-byte metadata record of every
    entry in the range (its kind), then per merged pair both entries read
    (key and value rows, alpha and beta, metadata) and both written."""
    eb = elem_bytes(call.dtype)
    H, d = call.H_kv, call.d
    ranged = int(sum(int(lengths[b]) - int(call.entry_start[b]) for b in range(call.B))) * H
    per_entry = (2 * d + 2) * eb + 16
    return 16 * ranged + 4 * per_entry * pairs


def compact_alg_bytes(call, page_table: np.ndarray, alpha_null: np.ndarray, lengths: np.ndarray,
                      new_lengths: np.ndarray, meta: bool = True) -> int:
    """Bytes one spicy_compact_range must move.  alpha_null: bool
    [pages, H, 16], the cache's nulls before the call.  Per sequence: the
    alpha of every entry of the range and head once (the null test), the
    range's page ids; per head, every entry that moves (a non-null one after
    the range's first null) read and written whole (key and value rows,
    alpha and beta, metadata), and the nulls written from its last entry to
    the end of the new last page; entry_begin, lengths and lengths_out."""
    eb = elem_bytes(call.dtype)
    H, d = call.H_kv, call.d
    entry = (2 * d + 2) * eb + (16 if meta else 0)
    total = 12 * call.B
    for b in range(call.B):
        e0, L = int(call.entry_start[b]), int(lengths[b])
        es = np.arange(e0, L)
        total += H * (L - e0) * eb + 4 * (-(-L // 16) - e0 // 16)
        pad_end = -(-int(new_lengths[b]) // 16) * 16
        for h in range(H):
            nul = alpha_null[page_table[b, es // 16], h, es % 16]
            first = int(np.argmax(nul)) if nul.any() else len(nul)
            moved = int((~nul[first:]).sum())
            live = int((~nul).sum())
            total += 2 * entry * moved + entry * (pad_end - (e0 + live))
    return total


def decode_alg_bytes(wl, lengths: np.ndarray, q_tokens: int = 1, diag: bool = False) -> int:
    """Bytes the decode must move: every cache entry it attends to (key,
    value, alpha, beta, and with `diag` the variance row), once per physical
    slot (the shared prefix is read from HBM once), plus Q, O, LSE of every
    query token."""
    eb = elem_bytes(wl.dtype)
    used = {}
    for b in range(wl.B):
        L = int(lengths[b])
        for lp in range(-(-L // 16)):
            p = int(wl.page_table[b, lp])
            used[p] = max(used.get(p, 0), min(16, L - 16 * lp))
    entries = sum(used.values()) * wl.H_kv
    per_entry = ((3 if diag else 2) * wl.d + 2) * eb
    qol = wl.B * q_tokens * wl.H_q * (wl.d * eb + wl.d * 4 + 4)
    return entries * per_entry + qol


COPY_BYTES = 512 << 20


def copy_calibration():
    import torch
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy-calibration", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "kernel": "torch.neg fp32", "launches": 5}), flush=True)



CU_PROBE_BYTES_PER_WG = 600 * 1024       # about one private page group of the benchmark's decode (72 pages)


def cu_probe(rotate_bytes: float = 1.5e9, reps: int = 10) -> list:
    """The plain streaming read (libspicy_probe.so) with N workgroups of 256
    threads, N x 600 KB per call over rotated buffers: per-workgroup and total
    GB/s.  Up to 256 workgroups the dispatcher gives each its own CU, so the
    per-workgroup rate at small N is what one CU can pull; at 256 and 512 the
    whole chip reads."""
    import torch
    lib = _probe_lib()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for n in (8, 32, 64, 128, 256, 512):
        nb = n * CU_PROBE_BYTES_PER_WG
        L = max(2, int(np.ceil(rotate_bytes / nb)))
        bufs = [torch.ones(nb // 4, dtype=torch.float32, device="cuda") for _ in range(L)]
        for unroll in (1, 8):
            def issue(u=unroll):
                for x in bufs:
                    rc = lib.spicy_probe_stream_read(x.data_ptr(), nb, n, u, sink.data_ptr(), stream)
                    assert rc == 0, rc
            us = statistics.median(_queued_per_call_us(issue, L, reps))
            line = {"mode": "cu-probe", "workgroups": n, "threads_per_workgroup": 256, "loads_in_flight": unroll,
                    "bytes_per_workgroup": CU_PROBE_BYTES_PER_WG, "us": round(us, 3),
                    "GBps_per_workgroup": round(CU_PROBE_BYTES_PER_WG / (us * 1e-6) / 1e9, 1),
                    "GBps_total": round(nb / (us * 1e-6) / 1e9, 1)}
            print(json.dumps(line), flush=True)
            out.append(line)
        del bufs
    return out


# the source file that defines each kernel; its digest also covers the
# headers every kernel includes
KERNEL_SOURCE = {
    "coarsen_main_kernel": "coarsen.hip", "coarsen_cpoint_kernel": "coarsen.hip",
    "decode_mfma_kernel": "decode.hip", "decode_f32_kernel": "decode.hip",
    "policy_token_kernel": "policy.hip", "policy_seq_kernel": "policy.hip",
    "merge_level_kernel": "merge.hip",
    "compact_count_kernel": "compact.hip", "compact_move_kernel": "compact.hip",
}
# the kernels of each call, for its traffic
CALL_KERNELS = {
    "coarsen": ["coarsen_main_kernel", "coarsen_cpoint_kernel"],
    "decode": ["decode_mfma_kernel"],
    "policy": ["policy_token_kernel", "policy_seq_kernel"],
    "merge": ["merge_level_kernel"],
    "compact": ["compact_count_kernel", "compact_move_kernel"],
}


def kernel_digest(kernel: str) -> str:
    """sha256 over the file defining `kernel` and the shared headers: a
    traffic figure measured on other sources is not reported."""
    import hashlib
    from coarse_grained_decode_amd import build as B
    h = hashlib.sha256()
    for f in [KERNEL_SOURCE[kernel]] + sorted(B.HEADERS):
        h.update(f.encode())
        with open(os.path.join(B.CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "spicy.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from profiles/traffic_<workload>.txt (rocprofv3
    FETCH_SIZE and WRITE_SIZE passes, scaled by the copy calibration), keyed
    by kernel name; a kernel whose sources changed since its counters were
    taken is left out.  None when the file is missing."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    table = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) >= 4 and parts[0] == "traffic_bytes" and parts[1] in KERNEL_SOURCE:
                if parts[3] == kernel_digest(parts[1]):
                    table[parts[1]] = float(parts[2])
    return table


# ------------------------------------------------------------------ host cores

def host_description() -> dict:
    """The host the oracle runs on: its CPU model, the logical CPUs of the
    machine and of this process's affinity set, and the thread count the
    oracle uses (the affinity set, capped by OMP_NUM_THREADS when the
    environment sets it, as the GPU machines do for each process's share)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    threads = min(aff, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else aff
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": aff, "threads": threads}


def cpu_baseline(wl, reps: int, policy: bool = False, q_tokens: int = 1, diag: bool = False,
                 weighted: bool = False, merge: bool = False, compact: bool = False):
    """The oracle (plain C, double precision) on the host cores: one whole
    step for every sequence of the batch (with `policy`, the oracle's policy
    on the chunk first; then the per-step coarsen and the decode), setup calls
    untimed.  Coarsening runs one sequence per work item, decoding one
    (sequence, KV head) per work item, over all the threads host_description
    gives.  Returns query tokens/s and details."""
    import dataclasses
    import oracle
    host = host_description()
    threads = host["threads"]
    cache = oracle.Cache(wl.dtype, wl.num_pages, wl.H_kv, wl.d, fill=False, diag=diag)
    lengths = None
    for call in wl.setup:
        lengths = oracle.coarsen(call, cache, threads=threads)
    qm = None
    if q_tokens > 1:
        from coarse_grained_decode_amd import workloads as W
        qm = W.query_tokens(wl, q_tokens)
    times = []
    for r in range(reps + 1):
        t0 = time.perf_counter()
        step = wl.step
        if policy:
            sp, c = wl.policy, wl.step
            pr = oracle.policy(c.k, c.v, c.seq_offsets, sp.proj_ptr, sp.proj_idx, sp.n_segments, sp.n_landmarks,
                               sp.sink, sp.recent)
            step = dataclasses.replace(c, seg_offsets=pr.seg_offsets, seq_seg_ptr=pr.seq_seg_ptr, mask=pr.mask)
        if step is not None:
            lengths = oracle.coarsen(step, cache, threads=threads,
                                     token_weight=pr.variation if (policy and weighted) else None)
            if merge:
                oracle.merge_level(cache, wl.page_table, step.entry_start, lengths, step.rope_base, threads=threads)
            if merge and compact:
                lengths = oracle.compact_range(cache, wl.page_table, step.entry_start, lengths, threads=threads)
        if q_tokens > 1:
            oracle.decode_multi(qm, wl.dtype, cache, wl.page_table, lengths, threads=threads)
        else:
            oracle.decode(wl.q, wl.dtype, cache, wl.H_q, wl.page_table, lengths, threads=threads)
        dt = time.perf_counter() - t0
        if r > 0:
            times.append(dt)
        print(f"[bench] cpu oracle step {r}: {dt:.3f} s", file=sys.stderr, flush=True)
    med = statistics.median(times)
    out = dict(value=wl.B * q_tokens / med, unit="query-tokens/s", cores=threads, kind="oracle",
               sample=f"one whole step of the same workload ({wl.B} sequences: "
                      f"{'policy (single thread) + ' if policy else ''}"
                      f"{'per-step coarsen + ' if wl.step is not None else ''}decode"
                      f"{f' of {q_tokens} query tokens per sequence' if q_tokens > 1 else ''}"
                      f"{', diagonal closure' if diag else ''}"
                      f"{', variation-weighted representatives' if weighted else ''}"
                      f"{', one merge level over the chunk' if merge else ''}"
                      f"{' and its compaction' if merge and compact else ''}), "
                      f"median of {reps} after 1 warm-up, {med:.3f} s per step")
    out.update(host)
    return out


def _loadavg():
    try:
        return float(open("/proc/loadavg").read().split()[0])
    except (OSError, ValueError, IndexError):
        return None


# --------------------------------------------------------------- GPU timing

_SLEEP = {}


def _sleep_cycles_for(us: float) -> int:
    """Cycles for torch.cuda._sleep to keep the GPU busy about `us` microseconds
    (calibrated once per process)."""
    import torch
    if "per_cycle_us" not in _SLEEP:
        n = 1 << 22
        torch.cuda._sleep(n)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        e1.synchronize()
        _SLEEP["per_cycle_us"] = e0.elapsed_time(e1) * 1e3 / n
    return max(1, int(us / _SLEEP["per_cycle_us"]))


def _hold_stream(host_us: float) -> None:
    """Queue a sleep kernel long enough (3x the host time of what follows, +2
    ms) that the host enqueues everything behind it before the GPU gets there."""
    import torch
    torch.cuda._sleep(_sleep_cycles_for(3 * host_us + 2000))


def _queued_per_call_us(issue, n_calls: int, reps: int, warmup: int = 2):
    """Per-call microseconds of `issue()` (n_calls calls on the current
    stream), measured with the calls back to back on the GPU: a sleep kernel
    holds the stream while the host enqueues them, and the events bracket only
    the calls."""
    import torch
    t0 = time.perf_counter()
    issue()
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - t0) * 1e6
    out = []
    for r in range(warmup + reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _hold_stream(host_us)
        e0.record()
        issue()
        e1.record()
        e1.synchronize()
        if r >= warmup:
            out.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    return out


def _stats(xs):
    xs = sorted(xs)
    q = lambda f: xs[min(len(xs) - 1, max(0, int(round(f * (len(xs) - 1)))))]
    return {"median": round(statistics.median(xs), 3), "p10": round(q(0.1), 3), "p90": round(q(0.9), 3),
            "mean": round(statistics.mean(xs), 3), "n": len(xs)}


def _rotating_copies(dw, rotate_bytes: float):
    """L distinct copies of the compressed cache (L x cache bytes >= rotate_bytes,
    well above the 256 MB Infinity Cache), so that calls rotating through them
    stream their cache from HBM."""
    from coarse_grained_decode_amd import PagedCache
    parts = (dw.cache.k, dw.cache.v, dw.cache.ab) + ((dw.cache.s2,) if dw.cache.s2 is not None else ())
    cache_bytes = sum(t.numel() * t.element_size() for t in parts)
    L = max(1, int(np.ceil(rotate_bytes / cache_bytes)))
    copies = [PagedCache(dw.cache.k.clone(), dw.cache.v.clone(), dw.cache.ab.clone(), None,
                         dw.cache.s2.clone() if dw.cache.s2 is not None else None) for _ in range(L)]
    return copies, cache_bytes


# ------------------------------------------------------------ read ceilings

_PROBE = {}


def _probe_lib():
    """libspicy_probe.so: the plain streaming-read kernel (not part of the
    SPICY-KV library; built beside it)."""
    import ctypes
    if "lib" not in _PROBE:
        from coarse_grained_decode_amd import build as B
        if not os.path.exists(B.PROBE_LIB):
            raise RuntimeError(f"{B.PROBE_LIB} is missing: build with python -m coarse_grained_decode_amd.build")
        L = ctypes.CDLL(B.PROBE_LIB)
        L.spicy_probe_stream_read.restype = ctypes.c_int
        L.spicy_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p]
        _PROBE["lib"] = L
    return _PROBE["lib"]


def read_ceiling(nbytes: int, rotate_bytes: float, reps: int = 10) -> dict:
    """Plain streaming-read ceiling at `nbytes`, over distinct buffers rotated
    through (L x nbytes >= rotate_bytes), calls back to back on the GPU:
      probe: the fastest of a few launch shapes of a grid-stride read of
             16-byte loads (libspicy_probe.so);
      torch: the fastest torch read-only reduction of the same bytes (rows
             of 4096 fp32 reduced along the row)."""
    import torch
    lib = _probe_lib()
    nb = max(16, nbytes // 16 * 16)
    L = max(1, int(np.ceil(rotate_bytes / nb)))
    bufs = [torch.ones(nb // 4, dtype=torch.float32, device="cuda") for _ in range(L)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for blocks_per_cu, unroll in ((8, 1), (16, 1), (8, 8), (4, 2)):
        def issue(bpc=blocks_per_cu, u=unroll):
            for x in bufs:
                rc = lib.spicy_probe_stream_read(x.data_ptr(), nb, 256 * bpc, u, sink.data_ptr(), stream)
                assert rc == 0, rc
        us = statistics.median(_queued_per_call_us(issue, L, reps))
        if best is None or us < best[0]:
            best = (us, f"grid-stride 16-byte loads, {256 * blocks_per_cu} workgroups x 256, {unroll} in flight")
    cols = 4096
    rows = max(1, nb // (4 * cols))
    views = [x[:rows * cols].view(rows, cols) for x in bufs]
    outs = [torch.empty(rows, dtype=torch.float32, device="cuda") for _ in range(L)]
    tbest = None
    for name, op in (("sum", torch.sum), ("amax", torch.amax)):
        def issue(op=op):
            for x, o in zip(views, outs):
                op(x, dim=1, out=o)
        us = statistics.median(_queued_per_call_us(issue, L, reps))
        if tbest is None or us < tbest[0]:
            tbest = (us, f"torch.{name}(dim=1) over fp32 rows of 4096")
    del bufs, views, outs
    gbs = lambda us: nb / (us * 1e-6) / 1e9
    return {"us": round(best[0], 3), "GBps": round(gbs(best[0]), 1), "frac": round(gbs(best[0]) / HBM_PEAK_GBS, 4),
            "op": best[1], "bytes": int(nb),
            "torch": {"us": round(tbest[0], 3), "GBps": round(gbs(tbest[0]), 1), "op": tbest[1]}}


# ------------------------------------------------------------ decode alone

def decode_config_line(wl, dw, rotate_bytes: float, reps: int, ceiling: bool = True) -> dict:
    """The decode call alone, back to back over rotated cache copies:
    per-call time (median, p10, p90), algorithmic bytes and rate, and the
    streaming-read ceiling at that byte count."""
    lengths = dw.lengths.cpu().numpy()
    copies, cache_bytes = _rotating_copies(dw, rotate_bytes)
    L = len(copies)

    def issue():
        for c in copies:
            dw.decode(c)
    per_call = _queued_per_call_us(issue, L, reps)
    assert int(dw.dws[0].item()) == 0, "device error word set (decode)"
    db = decode_alg_bytes(wl, lengths, dw.q_tokens, dw.cache.s2 is not None)
    st = _stats(per_call)
    gbs = db / (st["mean"] * 1e-6) / 1e9
    out = {"workload": wl.name, "description": wl.description, "calls_per_rep": L, "cache_bytes": int(cache_bytes),
           "bound": "hbm", "call": "decode", "alg_bytes_per_call": int(db), "call_us": st, "achieved": round(gbs, 1),
           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "target_frac": DECODE_TARGET_FRAC,
           "query_tokens_per_s": round(wl.B * dw.q_tokens / (st["mean"] * 1e-6), 1),
           "query_tokens_per_seq": dw.q_tokens, "plan": dw.plan, "shared_prefix_pages": dw.shared_prefix_pages}
    # HBM bytes per launch from the workload's rocprofv3 counters, while the sources match
    t = measured_traffic(wl.name)
    out["traffic"] = int(t["decode_mfma_kernel"]) if t and "decode_mfma_kernel" in t else None
    del copies
    if ceiling:
        c = read_ceiling(db, rotate_bytes)
        out["ceiling"] = c
        out["frac_of_ceiling"] = round(c["us"] / st["mean"], 4)
    return out


def decode_only(args, wl, dw):
    """Diagnostic mode: the decode call alone, back to back over rotated
    copies of the cache, next to the streaming-read ceiling of the same byte
    count."""
    import torch
    if dw.step is not None:
        dw.step.run(dw.cache)
        dw.lengths = dw.step.lengths
    torch.cuda.synchronize()
    line = decode_config_line(wl, dw, args.rotate_bytes, max(args.steps, 10))
    line["mode"] = "decode-only"
    print(json.dumps(line), flush=True)


def decode_configs(args, dev) -> list:
    """The decode alone on the 7B layer and the long ragged batch (their
    coarsening once, untimed), one line each."""
    import torch
    from coarse_grained_decode_amd import workloads as W
    from coarse_grained_decode_amd.runner import DeviceWorkload
    out = []
    for name in DECODE_CONFIGS:
        t0 = time.perf_counter()
        wl = W.WORKLOADS[name]()
        dw = DeviceWorkload.of(wl, dev, meta=False, fill=None)
        dw.run_setup()
        torch.cuda.synchronize()
        print(f"[bench] decode config {name}: generated and coarsened in {time.perf_counter() - t0:.1f} s",
              file=sys.stderr, flush=True)
        out.append(decode_config_line(wl, dw, args.rotate_bytes, max(10, args.steps // 2)))
        del dw, wl
        torch.cuda.empty_cache()
    return out


# --------------------------------------------------------- profile summary

def _base_kernel_name(name: str) -> str:
    """'void spicy::decode_mfma_kernel<128, 3, ...>(spicy::DecodeArgs)' ->
    'decode_mfma_kernel' (and torch's kernels to their template name)."""
    n = name.replace("(anonymous namespace)::", "")
    n = n.split("(")[0]
    n = re.sub(r"<.*", "", n)
    return n.split("::")[-1].replace("void ", "").strip()


def _read_csvs(pattern):
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _dispatches(d):
    """Kernel dispatches of a rocprofv3 --kernel-trace CSV dir, in start order:
    (base name, duration us)."""
    rows = _read_csvs(os.path.join(d, "**", "*kernel_trace.csv"))
    out = [(_base_kernel_name(r["Kernel_Name"]), int(r["Start_Timestamp"]),
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]
    out.sort(key=lambda x: x[1])
    return [(n, du) for n, _, du in out]


def _counters(d):
    """Per dispatch counter values of a rocprofv3 --pmc CSV dir, in dispatch
    order: {base kernel name: [{counter: value}, ...]}."""
    rows = _read_csvs(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in rows:
        key = (int(r.get("Dispatch_Id", 0)), _base_kernel_name(r["Kernel_Name"]))
        per.setdefault(key, {})
        name = r["Counter_Name"]
        per[key][name] = per[key].get(name, 0.0) + float(r["Counter_Value"])
    out = {}
    for (did, k), v in sorted(per.items()):
        out.setdefault(k, []).append(v)
    return out


def summarize_profile(args) -> None:
    """Write profiles/<name>.txt from the rocprofv3 CSV output under DIR:
    per-kernel durations (all dispatches and the last N), HBM traffic per
    launch (FETCH_SIZE and WRITE_SIZE scaled by the copy calibration), any
    other counter passes, and the machine-read traffic lines with the
    kernels' source digests."""
    d = args.summarize_profile
    name = args.profile_name or "profile"
    last = args.profile_last or 2 * args.steps
    lines = [f"# rocprofv3 summary: SPICY-KV kernels, {name}", ""]
    if args.profile_commands:
        lines.append("Commands (run from /tmp with TMPDIR=/tmp; R = repository root, OUT = output dir):")
        lines += [f"  {c.strip()}" for c in args.profile_commands.split(";") if c.strip()]
        lines.append("")
    disp = _dispatches(os.path.join(d, "trace"))
    if disp:
        lines.append(f"## Kernel durations (kernel trace; 'last' = each kernel's last {last} dispatches)")
        lines.append("")
        lines.append(f"{'kernel':34s} {'calls':>6s} {'mean us':>9s} {'median':>8s} {'min':>8s} {'max':>8s}   "
                     f"{'last mean':>9s} {'last med':>9s} {'last p10':>9s} {'last p90':>9s}")
        by = {}
        for n, du in disp:
            by.setdefault(n, []).append(du)
        for n, xs in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            tl = sorted(xs[-last:])
            q = lambda f: tl[min(len(tl) - 1, int(round(f * (len(tl) - 1))))]
            lines.append(f"{n[:34]:34s} {len(xs):6d} {statistics.mean(xs):9.2f} {statistics.median(xs):8.2f} "
                         f"{min(xs):8.2f} {max(xs):8.2f}   {statistics.mean(tl):9.2f} {statistics.median(tl):9.2f} "
                         f"{q(0.1):9.2f} {q(0.9):9.2f}")
        lines.append("")
    fetch = _counters(os.path.join(d, "FETCH_SIZE"))
    write = _counters(os.path.join(d, "WRITE_SIZE"))
    cf = _counters(os.path.join(d, "copy_FETCH_SIZE"))
    cw = _counters(os.path.join(d, "copy_WRITE_SIZE"))
    digest_lines = []
    measured = {}
    if fetch and write and cf and cw:
        def copy_kib(c, ctr):
            vals = [v[ctr] for k, vs in c.items() if "neg" in k or "elementwise" in k for v in vs if ctr in v]
            return statistics.median(vals)
        fk = copy_kib(cf, "FETCH_SIZE")
        wk = copy_kib(cw, "WRITE_SIZE")
        ff = COPY_BYTES / (fk * 1024.0)
        wf = COPY_BYTES / (wk * 1024.0)
        lines.append("## HBM traffic per launch (FETCH_SIZE / WRITE_SIZE, KiB per dispatch, median of each "
                     "kernel's last 3 dispatches)")
        lines.append("")
        lines.append(f"Calibration: a plain fp32 copy of {COPY_BYTES} bytes (torch.neg) reads FETCH_SIZE {fk:.0f} KiB "
                     f"and WRITE_SIZE {wk:.0f} KiB per dispatch: bytes = KiB x 1024 x {ff:.4f} (fetch), "
                     f"x {wf:.4f} (write).")
        lines.append("")
        lines.append(f"{'kernel':34s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} {'bytes/launch':>14s}")
        for k in sorted(set(fetch) & set(write)):
            fv = statistics.median([v["FETCH_SIZE"] for v in fetch[k][-3:] if "FETCH_SIZE" in v])
            wv = statistics.median([v["WRITE_SIZE"] for v in write[k][-3:] if "WRITE_SIZE" in v])
            b = fv * 1024 * ff + wv * 1024 * wf
            lines.append(f"{k[:34]:34s} {fv:12.0f} {wv:12.0f} {b:14.0f}")
            measured[k] = b
            if k in KERNEL_SOURCE:
                digest_lines.append(f"traffic_bytes {k} {b:.0f} {kernel_digest(k)}")
        lines.append("")
    for pdir in sorted(glob.glob(os.path.join(d, "pmc_*"))):
        ctr = _counters(pdir)
        if not ctr:
            continue
        names = sorted({c for vs in ctr.values() for v in vs for c in v})
        lines.append(f"## Counters {', '.join(names)} (per dispatch, median of each kernel's last 3 dispatches)")
        lines.append("")
        lines.append(f"{'kernel':34s} " + " ".join(f"{n:>24s}" for n in names))
        for k, vs in sorted(ctr.items()):
            row = []
            for n in names:
                xs = [v[n] for v in vs[-3:] if n in v]
                row.append(f"{statistics.median(xs):24.6g}" if xs else f"{'-':>24s}")
            lines.append(f"{k[:34]:34s} " + " ".join(row))
        lines.append("")
    if digest_lines:
        lines.append("Machine-read lines (bench.py reports a kernel's `traffic` only while its sources hash to the "
                     "value given):")
        lines.append("(each line: kernel, bytes per launch, sha256 of the kernel's source file and the shared headers)")
        lines += digest_lines
        lines.append("")
    bench_line = os.path.join(d, "bench_line.json")
    if os.path.exists(bench_line):
        with open(bench_line) as fh:
            raw = fh.read().strip().splitlines()[-1]
        if measured:
            # measured HBM bytes of each call's kernels over the call's algorithmic bytes
            rec = json.loads(raw)
            if rec.get("mode") == "decode-only":        # the line is the decode call itself
                rec = {"roofline": dict(rec, call="decode")}
            rows = []
            for key, r in sorted(rec.items()):
                if not (key.startswith("roofline") and isinstance(r, dict) and r.get("call") in CALL_KERNELS):
                    continue
                ks = CALL_KERNELS[r["call"]]
                if all(k in measured for k in ks) and r.get("alg_bytes_per_call"):
                    tb = sum(measured[k] for k in ks)
                    rows.append(f"{r['call']:10s} {r['alg_bytes_per_call']:14d} {tb:14.0f} {tb / r['alg_bytes_per_call']:8.3f}")
            if rows:
                lines.append("## Measured traffic over algorithmic bytes, per call")
                lines.append("")
                lines.append(f"{'call':10s} {'algorithmic':>14s} {'measured':>14s} {'ratio':>8s}")
                lines += rows
                lines.append("")
        lines.append("## bench.py line of the same tree")
        lines.append("")
        lines.append(raw)
        lines.append("")
    out = os.path.join(ROOT, "profiles", f"{name}.txt")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {out}", flush=True)


# ---------------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize_profile:
        return summarize_profile(args)
    if args.copy_calibration:
        return copy_calibration()
    if args.cu_probe:
        cu_probe(args.rotate_bytes)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path, and every number it reports is one GPU's", file=sys.stderr)
        sys.exit(2)

    import torch
    from coarse_grained_decode_amd import workloads as W
    from coarse_grained_decode_amd.runner import DeviceWorkload

    if args.workload not in W.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(W.WORKLOADS)}")
    t_gen = time.perf_counter()
    wl = W.WORKLOADS[args.workload]()
    print(f"[bench] generated {wl.name} in {time.perf_counter() - t_gen:.1f} s: {wl.description}",
          file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dw = DeviceWorkload.of(wl, dev, meta=args.merge, num_splits=args.splits, fill=None,
                           use_shared_prefix=not args.no_shared_prefix, q_tokens=args.query_tokens,
                           diag=args.diag_closure)
    dw.run_setup()
    torch.cuda.synchronize()
    # a step: the per-step coarsen call if the workload has one, else its whole
    # coarsen (setup) again, then the decode
    step_calls = [dw.step] if dw.step is not None else dw.setup
    policy = None
    if args.device_policy:
        from coarse_grained_decode_amd.runner import DevicePolicy
        if wl.policy is None or dw.step is None:
            sys.exit(f"--device-policy: workload {wl.name} has no per-step chunk with a policy")
        policy = DevicePolicy.of(wl.policy, dw.step.call, dev)
        step_calls = [policy.feed(dw.step, dev, weighted=args.weighted)]
    elif args.weighted:
        sys.exit("--weighted needs --device-policy (the weights are the policy's per-token variation)")
    run_merge, mws = None, None
    if args.merge and args.diag_closure:
        sys.exit("--merge does not combine with --diag-closure (the diagonal variances do not merge)")
    if args.merge:
        from coarse_grained_decode_amd import spicy_merge_level, spicy_merge_workspace_bytes, workspace
        if dw.step is None:
            sys.exit(f"--merge: workload {wl.name} has no per-step chunk to merge")
        mc = step_calls[-1]
        seg_per_seq = wl.policy.n_segments if policy is not None else int(np.diff(mc.call.seq_seg_ptr).max())
        max_range = int(np.diff(mc.call.seq_offsets).max()) + seg_per_seq + 16
        mws = workspace(spicy_merge_workspace_bytes(mc.call.B, mc.call.H_kv, max_range), dev)

        def run_merge():
            spicy_merge_level(dw.cache, mc.call.rope_base, mc.page_table, mc.entry_start, mc.lengths, max_range,
                              mws, max_pages_per_seq=mc.call.max_pages)
    elif args.no_compact:
        sys.exit("--no-compact needs --merge")
    run_compact, clen, cerr = None, None, None
    if args.merge and not args.no_compact:
        from coarse_grained_decode_amd import spicy_compact_range
        clen = torch.empty_like(mc.lengths)
        cerr = torch.zeros(1, dtype=torch.int32, device=dev)

        def run_compact():
            spicy_compact_range(dw.cache, mc.page_table, mc.entry_start, mc.lengths, clen, cerr,
                                max_pages_per_seq=mc.call.max_pages)

    def step(ev=None, until=None):
        """One step; with ev (6 events) each call is bracketed:
        ev[3] policy ev[0] coarsen ev[1] merge ev[5] compact ev[4] decode ev[2].
        until="merge": stop after the merge."""
        if ev is not None:
            ev[3].record()
        if policy is not None:
            policy.run(dw.step)
        if ev is not None:
            ev[0].record()
        for c in step_calls:
            c.run(dw.cache)
        if ev is not None:
            ev[1].record()
        if run_merge is not None:
            run_merge()
        if until == "merge":
            return
        if ev is not None:
            ev[5].record()
        if run_compact is not None:
            run_compact()
        if ev is not None:
            ev[4].record()
        dw.lengths = clen if run_compact is not None else step_calls[-1].lengths
        dw.decode()
        if ev is not None:
            ev[2].record()

    if args.decode_only:
        return decode_only(args, wl, dw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for c in dw.setup + step_calls:
        assert int(c.ws[0].item()) == 0, "device error word set"
    if policy is not None:
        assert int(policy.ws[0].item()) == 0, "device error word set (policy)"

    # the step as one HIP graph (the same kernels on the same buffers; the
    # library neither allocates nor synchronises inside a call), so that each
    # timed step is one launch from the host instead of a few marshalled
    # calls; eager issue on request or if the capture fails
    launch = "eager"
    run_step = step
    if not args.eager:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            for c in dw.setup + step_calls:
                assert int(c.ws[0].item()) == 0, "device error word set (graph replay)"
            run_step = graph.replay
            launch = "hip graph (one step captured, one replay per timed step)"
        except Exception as e:               # noqa: BLE001 - report and time the eager path instead
            launch = f"eager (graph capture failed: {type(e).__name__}: {e})"
            print(f"[bench] {launch}", file=sys.stderr, flush=True)
            torch.cuda.synchronize()

    # throughput: exactly K whole steps with nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    t_issue = time.perf_counter() - t0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert int(dw.dws[0].item()) == 0, "device error word set (decode)"

    # per-call durations: K more whole steps queued behind a sleep kernel (so
    # that no call waits for the host), each call bracketed by HIP events on
    # the launch stream
    # (two more steps go first, untimed: the first queued steps behind the
    # sleep have shown host-side stalls of up to milliseconds)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps + 2)]
    _hold_stream(elapsed * 1e6 * 1.5)
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    evs = evs[2:]
    per = {
        "coarsen": [e[0].elapsed_time(e[1]) * 1e3 for e in evs],
        "decode": [e[4].elapsed_time(e[2]) * 1e3 for e in evs],
    }
    if run_merge is not None:
        per["merge"] = [e[1].elapsed_time(e[5]) * 1e3 for e in evs]
    if run_compact is not None:
        per["compact"] = [e[5].elapsed_time(e[4]) * 1e3 for e in evs]
    if policy is not None:
        per["policy"] = [e[3].elapsed_time(e[0]) * 1e3 for e in evs]
    step_us = [e[3].elapsed_time(e[2]) * 1e3 for e in evs]

    lengths = dw.lengths.cpu().numpy()
    alg = {
        "coarsen": sum(coarsen_alg_bytes(c.call, c.lengths.cpu().numpy(), args.diag_closure, args.weighted, args.merge)
                       for c in step_calls),
        "decode": decode_alg_bytes(wl, lengths, args.query_tokens, args.diag_closure),
    }
    names = {
        "coarsen": "spicy_coarsen (coarsen_main: plan + streaming, then coarsen_cpoint: entries)",
        "decode": ("spicy_decode_attn_multi" if args.query_tokens > 1 else
                   "spicy_decode_attn_shared" if dw.shared_prefix_pages else "spicy_decode_attn") +
                  " (decode_mfma: split-K pages, log-sum-exp combine in the same launch)",
        "policy": "spicy_policy (policy_token: fixed point, projection, variation, key norms; "
                  "then policy_seq: scan, boundaries, landmark radix select)",
        "merge": "spicy_merge_level (merge_level: each workgroup lists its sequence and head's pairs, merges "
                 "its share by the law of total variance; the last one writes the records)",
        "compact": "spicy_compact_range (compact_count: new lengths; compact_move: live entries moved to the "
                   "front of the merged range, nulls to the end of the new last page)",
    }
    pairs = None
    if policy is not None:
        alg["policy"] = policy_alg_bytes(dw.step.call, wl.policy)
    if run_merge is not None:
        mc = step_calls[-1]
        assert int(mws[0].item()) == 0, "device error word set (merge)"
        for c in step_calls:                      # the chunk as the merge finds it
            c.run(dw.cache)
        torch.cuda.synchronize()
        pairs = merge_pair_count(dw.cache.meta.cpu().numpy(), mc.page_table.cpu().numpy(),
                                 mc.entry_start.cpu().numpy(), mc.lengths.cpu().numpy())
        alg["merge"] = merge_alg_bytes(mc.call, mc.lengths.cpu().numpy(), pairs)
    compaction = None
    if run_compact is not None:
        assert int(cerr.item()) == 0, "device error word set (compact)"
        # the nulls the compaction sees: one more step up to the merge
        step(until="merge")
        torch.cuda.synchronize()
        ab = dw.cache.ab[..., 0]
        bits = ab.view(torch.int16) if ab.dtype == torch.bfloat16 else ab.view(torch.int32)
        neg_inf = -128 if ab.dtype == torch.bfloat16 else -8388608          # 0xFF80, 0xFF800000
        alpha_null = (bits == neg_inf).cpu().numpy()
        full = mc.lengths.cpu().numpy()
        run_compact()
        torch.cuda.synchronize()
        new = clen.cpu().numpy()
        alg["compact"] = compact_alg_bytes(mc.call, mc.call.page_table, alpha_null, full, new)
        compaction = {"entries_before": int((full - mc.call.entry_start).sum()),
                      "entries_after": int((new - mc.call.entry_start).sum()),
                      "lengths_max_before": int(full.max()), "lengths_max_after": int(new.max())}

    traffic = measured_traffic(wl.name + ("_policy" if policy is not None else "") +
                               (f"_q{args.query_tokens}" if args.query_tokens > 1 else "") +
                               ("_weighted" if args.weighted else "") + ("_diag" if args.diag_closure else "") +
                               ("_merge" if args.merge else "") + ("_nocompact" if args.no_compact else ""))

    def roof(call):
        st = _stats(per[call])
        gbs = alg[call] / (st["mean"] * 1e-6) / 1e9
        ks = CALL_KERNELS[call]
        t = None
        if traffic is not None and all(k in traffic for k in ks):
            t = int(sum(traffic[k] for k in ks))
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": t, "alg_bytes_per_call": int(alg[call]),
                "mean_call_us": st["mean"], "call_us": st, "call": call, "kernel": names[call]}

    rooflines = {c: roof(c) for c in per}
    dominant = max(rooflines, key=lambda c: rooflines[c]["call_us"]["median"])
    r_decode = dict(rooflines["decode"])
    r_decode["target_frac"] = DECODE_TARGET_FRAC
    r_decode["ceiling"] = read_ceiling(alg["decode"], args.rotate_bytes)
    r_decode["frac_of_ceiling"] = round(r_decode["ceiling"]["us"] / r_decode["call_us"]["mean"], 4)

    ms_per_step = elapsed * 1e3 / args.steps
    out = {
        "metric": "compressed-KV decode query-tokens/s and achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(wl.B * args.query_tokens * args.steps / elapsed, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded clustered-Gaussian keys, Gaussian values/queries)",
        "config": {"workload": wl.name, "description": wl.description, "batch": wl.B,
                   "num_q_heads": wl.H_q, "num_kv_heads": wl.H_kv, "head_dim": wl.d,
                   "decode_plan": dw.plan, "shared_prefix_pages": dw.shared_prefix_pages,
                   "cache_entries_per_seq_mean": float(lengths.mean()),
                   "device_policy": policy is not None, "query_tokens_per_seq": args.query_tokens,
                   "diag_closure": args.diag_closure, "weighted_representatives": args.weighted,
                   "merge_level": args.merge, "compacted": args.merge and not args.no_compact},
        "step_us": _stats(step_us),
        "launch": launch,
        # host time to enqueue the K steps (the loop is host-bound when it nears ms_per_step)
        "host_issue_us_per_step": round(t_issue / args.steps * 1e6, 1),
        "host_loadavg": _loadavg(),
        "roofline": rooflines[dominant],
        "roofline_decode": r_decode,
        "decode_query_tokens_per_s": round(wl.B * args.query_tokens / (r_decode["call_us"]["mean"] * 1e-6), 1),
    }
    for c in ("coarsen", "policy", "merge", "compact"):
        if c in rooflines and c != dominant:
            out[f"roofline_{c}"] = rooflines[c]
    if pairs is not None:
        out["roofline_merge" if dominant != "merge" else "roofline"]["pairs_per_call"] = pairs
    if compaction is not None:
        out["roofline_compact" if dominant != "compact" else "roofline"]["entries"] = compaction
    if not args.no_decode_configs:
        del dw
        torch.cuda.empty_cache()
        out["decode_configs"] = decode_configs(args, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_reps, policy=policy is not None,
                                           q_tokens=args.query_tokens, diag=args.diag_closure,
                                           weighted=args.weighted, merge=args.merge,
                                           compact=args.merge and not args.no_compact)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
