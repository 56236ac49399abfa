"""Benchmark: SPICY-KV compressed-KV decode on one MI355X.

One step = one pass of the whole hot path over one batch: spicy_coarsen of the
batch's fresh chunk into the paged cache (plan + segmented moments + RoPE +
pack), then spicy_decode_attn of one query token per sequence over the whole
compressed cache (split-K decode + log-sum-exp combine).

Default workload: the shared-prefix batch (32 sequences sharing one
65536-token prefix compressed 28.6x, a private exact suffix of U[512, 2048]
tokens each, and a fresh 8192-token chunk per sequence coarsened every step
with equal-variation segments), Qwen2-7B head shape (28 query / 4 KV heads,
d = 128), bf16.  Other workloads: --workload qwen2_7b_layer | long_ragged |
qwen2_1.5b_layer | tiny_fp32 (those have no per-step coarsen; a step is their
whole coarsen + decode).

Prints ONE JSON line.  `value` = query tokens per second of whole steps.
`roofline` describes the step's dominant launch (largest share of the step
time), `roofline_decode` the decode call; `achieved` = algorithmic bytes per
call / mean call duration from HIP events recorded on the stream the
kernels run on.  Inputs are resident in HBM before the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
ENTRY_EXTRA_META = 16          # bytes of optional metadata per entry-head (not used here)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="shared_prefix")
    ap.add_argument("--splits", type=int, default=0, help="decode split count (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--decode-only", action="store_true",
                    help="diagnostic: time spicy_decode_attn alone over rotated copies of the cache")
    ap.add_argument("--rotate-bytes", type=float, default=1.5e9,
                    help="decode-only: total bytes of distinct cache copies rotated through")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device copy (torch.neg, fp32) 5 times: the known-size "
                         "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
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
                         "(spicy_merge_level; the cache keeps its metadata)")
    ap.add_argument("--diag-closure", action="store_true",
                    help="the cache carries per-dimension variances (diagonal closure): coarsen writes them, "
                         "decode reads them in place of the scalar beta")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="decode a shared-prefix batch with spicy_decode_attn (every page per sequence)")
    return ap.parse_args()


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


def merge_alg_bytes(call, lengths: np.ndarray, pairs: int) -> int:
    """Bytes one merge level must move: the 16-byte metadata record of every
    entry in the range (its kind), then per merged pair both entries read
    (key and value rows, alpha and beta, metadata) and both written."""
    eb = elem_bytes(call.dtype)
    H, d = call.H_kv, call.d
    ranged = int(sum(int(lengths[b]) - int(call.entry_start[b]) for b in range(call.B))) * H
    per_entry = (2 * d + 2) * eb + 16
    return 16 * ranged + 4 * per_entry * pairs


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


# the source file that defines each kernel; its digest also covers the
# headers every kernel includes
KERNEL_SOURCE = {
    "coarsen_main_kernel": "coarsen.hip", "coarsen_cpoint_kernel": "coarsen.hip",
    "decode_mfma_kernel": "decode.hip", "combine_kernel": "decode.hip", "decode_f32_kernel": "decode.hip",
    "policy_token_kernel": "policy.hip", "policy_seq_kernel": "policy.hip",
    "merge_list_kernel": "merge.hip", "merge_pair_kernel": "merge.hip",
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


def cpu_baseline(wl, reps: int, policy: bool = False, q_tokens: int = 1, diag: bool = False,
                 weighted: bool = False, merge: bool = False):
    """The oracle (plain C, double precision) on the host cores: one whole
    step for every sequence of the batch (with `policy`, the oracle's policy
    on the chunk first; then the per-step coarsen and the decode), setup calls
    untimed.  Returns query tokens/s and details."""
    import dataclasses
    import oracle
    threads = oracle.default_threads()
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
        if q_tokens > 1:
            oracle.decode_multi(qm, wl.dtype, cache, wl.page_table, lengths, threads=threads)
        else:
            oracle.decode(wl.q, wl.dtype, cache, wl.H_q, wl.page_table, lengths, threads=threads)
        dt = time.perf_counter() - t0
        if r > 0:
            times.append(dt)
        print(f"[bench] cpu oracle step {r}: {dt:.3f} s", file=sys.stderr, flush=True)
    med = statistics.median(times)
    return dict(value=wl.B * q_tokens / med, unit="query-tokens/s", cores=threads, kind="oracle",
                sample=f"one whole step of the same workload ({wl.B} sequences: "
                       f"{'policy (single thread) + ' if policy else ''}"
                       f"{'per-step coarsen + ' if wl.step is not None else ''}decode"
                       f"{f' of {q_tokens} query tokens per sequence' if q_tokens > 1 else ''}"
                       f"{', diagonal closure' if diag else ''}"
                       f"{', variation-weighted representatives' if weighted else ''}"
                       f"{', one merge level over the chunk' if merge else ''}), "
                       f"median of {reps} after 1 warm-up, {med:.3f} s per step")


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


def _queued_per_call_us(issue, n_calls: int, reps: int, warmup: int = 2):
    """Per-call microseconds of `issue()` (n_calls calls on the current
    stream), measured with the calls back to back on the GPU: a sleep kernel
    holds the stream while the host enqueues them, and the events bracket only
    the calls.  The sleep is sized from the host's enqueue time, so no call
    waits for the host."""
    import torch
    t0 = time.perf_counter()
    issue()
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - t0) * 1e6
    cycles = _sleep_cycles_for(3 * host_us + 2000)
    out = []
    for r in range(warmup + reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(cycles)
        e0.record()
        t0 = time.perf_counter()
        issue()
        host = (time.perf_counter() - t0) * 1e6
        e1.record()
        e1.synchronize()
        gpu = e0.elapsed_time(e1) * 1e3
        if host > 0.9 * _SLEEP["per_cycle_us"] * cycles:
            print(f"[bench] warning: enqueueing took {host:.0f} us, longer than the sleep", file=sys.stderr)
        if r >= warmup:
            out.append(gpu / n_calls)
    return out


def _stats(xs):
    xs = sorted(xs)
    q = lambda f: xs[min(len(xs) - 1, max(0, int(round(f * (len(xs) - 1)))))]
    return {"median": round(statistics.median(xs), 3), "p10": round(q(0.1), 3), "p90": round(q(0.9), 3)}


def read_ceiling_us(nbytes: int, rotate_bytes: float, replays: int = 20):
    """Plain streaming-read ceiling at `nbytes`: the fastest of a few torch
    read-only reductions over a tensor of that size, rotating through distinct
    tensors (L x nbytes >= rotate_bytes), back to back on the GPU.  Returns
    (microseconds per read, the op that gave it)."""
    import torch
    # rows of 4096 floats reduced along the row: each output depends on one
    # row only, so the reduction needs no cross-workgroup staging; the
    # output is 1/4096 of the bytes read
    cols = 4096
    rows = max(1, nbytes // (4 * cols))
    L = max(1, int(np.ceil(rotate_bytes / (4 * rows * cols))))
    bufs = [torch.ones(rows, cols, dtype=torch.float32, device="cuda") for _ in range(L)]
    outs = [torch.empty(rows, dtype=torch.float32, device="cuda") for _ in range(L)]
    ops = {"sum": lambda x, o: torch.sum(x, dim=1, out=o), "amax": lambda x, o: torch.amax(x, dim=1, out=o)}
    best = None
    for name, op in ops.items():
        def issue(op=op):
            for x, o in zip(bufs, outs):
                op(x, o)
        us = statistics.median(_queued_per_call_us(issue, L, replays))
        if best is None or us < best[0]:
            best = (us, name)
    del bufs
    return best


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


def decode_config_line(wl, dw, rotate_bytes: float, replays: int, ceiling: bool = True):
    """Per-call decode time (median, p10, p90 over repetitions of L rotated
    calls run back to back), algorithmic bytes and rate, and the read ceiling
    at that size."""
    import torch
    lengths = dw.lengths.cpu().numpy()
    copies, cache_bytes = _rotating_copies(dw, rotate_bytes)
    L = len(copies)

    def issue():
        for c in copies:
            dw.decode(c)
    per_call = _queued_per_call_us(issue, L, replays)
    assert int(dw.dws[0].item()) == 0, "device error word set (decode)"
    db = decode_alg_bytes(wl, lengths, dw.q_tokens, dw.cache.s2 is not None)
    st = _stats(per_call)
    us = st["median"]
    gbs = db / (us * 1e-6) / 1e9
    out = {"workload": wl.name, "calls_per_replay": L, "replays": replays, "cache_bytes": int(cache_bytes),
           "alg_bytes_per_call": int(db), "call_us": st, "achieved_GBps": round(gbs, 1),
           "frac": round(gbs / HBM_PEAK_GBS, 4),
           "query_tokens_per_s": round(wl.B * dw.q_tokens / (us * 1e-6), 1),
           "query_tokens_per_seq": dw.q_tokens, "plan": dw.plan, "shared_prefix_pages": dw.shared_prefix_pages}
    del copies
    if ceiling:
        cus, op = read_ceiling_us(db, rotate_bytes)
        cg = db / (cus * 1e-6) / 1e9
        out["ceiling"] = {"us": round(cus, 3), "GBps": round(cg, 1), "frac": round(cg / HBM_PEAK_GBS, 4),
                          "op": f"torch.{op}(dim=1) over fp32 rows of 4096, same byte count, rotated, "
                                "back to back"}
        out["frac_of_ceiling"] = round(gbs / cg, 4)
    return out


def main():
    args = parse()
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
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

    def step():
        if policy is not None:
            policy.run(dw.step)
        for c in step_calls:
            c.run(dw.cache)
        if run_merge is not None:
            run_merge()
        dw.lengths = step_calls[-1].lengths
        dw.decode()

    if args.decode_only:
        return decode_only(args, wl, dw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for c in dw.setup + step_calls:
        assert int(c.ws[0].item()) == 0, "device error word set"
    if policy is not None:
        assert int(policy.ws[0].item()) == 0, "device error word set (policy)"

    # throughput: exactly K whole steps with nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert int(dw.dws[0].item()) == 0, "device error word set (decode)"

    # per-call durations for the rooflines: K more whole steps, each call
    # bracketed by HIP events on the launch stream.  They run after the
    # throughput loop because an event recorded between two calls leaves the
    # GPU idle for a few microseconds; part of that idle time lands inside the
    # bracketed durations, so these err on the slow side.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in evs:
        e[3].record()
        if policy is not None:
            policy.run(dw.step)
        e[0].record()
        for c in step_calls:
            c.run(dw.cache)
        e[1].record()
        if run_merge is not None:
            run_merge()
        e[4].record()
        dw.decode()
        e[2].record()
    torch.cuda.synchronize()
    coarsen_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    decode_ms = statistics.mean(e[4].elapsed_time(e[2]) for e in evs)
    merge_ms = statistics.mean(e[1].elapsed_time(e[4]) for e in evs) if run_merge is not None else None
    policy_ms = statistics.mean(e[3].elapsed_time(e[0]) for e in evs) if policy is not None else None
    lengths = dw.lengths.cpu().numpy()
    cb = sum(coarsen_alg_bytes(c.call, c.lengths.cpu().numpy(), args.diag_closure, args.weighted, args.merge)
             for c in step_calls)
    db = decode_alg_bytes(wl, lengths, args.query_tokens, args.diag_closure)

    traffic = measured_traffic(wl.name + ("_policy" if policy is not None else "") +
                               (f"_q{args.query_tokens}" if args.query_tokens > 1 else "") +
                               ("_weighted" if args.weighted else "") + ("_diag" if args.diag_closure else "") +
                               ("_merge" if args.merge else ""))

    def roof(nbytes, ms, kernels):
        gbs = nbytes / (ms * 1e-3) / 1e9
        t = None
        if traffic is not None and all(k in traffic for k in kernels):
            t = int(sum(traffic[k] for k in kernels))
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": t,
                "alg_bytes_per_call": int(nbytes), "mean_call_us": round(ms * 1e3, 2)}

    r_coarsen = roof(cb, coarsen_ms, ["coarsen_main_kernel", "coarsen_cpoint_kernel"])
    r_decode = roof(db, decode_ms, ["decode_mfma_kernel", "combine_kernel"])
    r_coarsen["kernel"] = "spicy_coarsen (coarsen_main: plan + streaming, then coarsen_cpoint: entries)"
    r_decode["kernel"] = ("spicy_decode_attn_shared" if dw.shared_prefix_pages else "spicy_decode_attn") + \
        " (decode_mfma + combine)"
    calls = [(coarsen_ms, r_coarsen), (decode_ms, r_decode)]
    if policy is not None:
        c = dw.step.call
        pb = policy_alg_bytes(c, wl.policy)
        r_policy = roof(pb, policy_ms, ["policy_token_kernel", "policy_seq_kernel"])
        r_policy["kernel"] = "spicy_policy (policy_token: fixed point, projection, variation, key norms; " \
                             "then policy_seq: scan, boundaries, landmark radix select)"
        calls.append((policy_ms, r_policy))
    if run_merge is not None:
        mc = step_calls[-1]
        units = mc.call.B * mc.call.H_kv
        pairs = int(mws.view(torch.uint8)[256:256 + 4 * units].view(torch.int32).sum().item())
        assert int(mws[0].item()) == 0, "device error word set (merge)"
        mb = merge_alg_bytes(mc.call, mc.lengths.cpu().numpy(), pairs)
        r_merge = roof(mb, merge_ms, ["merge_list_kernel", "merge_pair_kernel"])
        r_merge["kernel"] = "spicy_merge_level (merge_list: pairs per sequence and head; merge_pair: law of " \
                            "total variance per pair)"
        r_merge["pairs_per_call"] = pairs
        calls.append((merge_ms, r_merge))
    calls.sort(key=lambda x: -x[0])
    dominant, other = calls[0][1], calls[1][1]

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
                   "decode_splits": dw.splits, "decode_plan": dw.plan,
                   "shared_prefix_pages": dw.shared_prefix_pages,
                   "cache_entries_per_seq_mean": float(lengths.mean()),
                   "device_policy": policy is not None, "query_tokens_per_seq": args.query_tokens,
                   "diag_closure": args.diag_closure, "weighted_representatives": args.weighted,
                   "merge_level": args.merge},
        "roofline": dominant,
        "roofline_other": other,
        "decode_query_tokens_per_s": round(wl.B * args.query_tokens / (decode_ms * 1e-3), 1),
    }
    if policy is not None:
        out["roofline_policy"] = r_policy
    if run_merge is not None:
        out["roofline_merge"] = r_merge
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_reps, policy=policy is not None,
                                           q_tokens=args.query_tokens, diag=args.diag_closure,
                                           weighted=args.weighted, merge=args.merge)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
