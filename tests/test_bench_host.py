"""bench.py's host-side accounting, on the CPU: the algorithmic bytes each
roofline divides by, recomputed here from their definitions on small
hand-made inputs, and the traffic table's digest check."""
import types

import numpy as np

import bench


def small_call(dtype="bf16"):
    # 2 sequences of 5 and 3 tokens, H = 2, d = 64; sequence 1 appends at entry 32
    return types.SimpleNamespace(dtype=dtype, total_tokens=8, H_kv=2, d=64, B=2,
                                 entry_start=np.array([0, 32], np.int32))


def test_coarsen_bytes():
    c = small_call()
    lengths = np.array([3, 35], np.int32)              # entries written: pages up to 16 and 48
    read = 8 * 2 * 64 * 2 * 2 + 8 * 2                  # k and v of every token, the mask
    written = 2 * (16 - 0) + 2 * (48 - 32)             # per head, to the end of the last page
    assert bench.coarsen_alg_bytes(c, lengths) == read + written * (2 * 64 + 2) * 2 + 2 * 4
    assert bench.coarsen_alg_bytes(c, lengths, diag=True) == read + written * (3 * 64 + 2) * 2 + 2 * 4
    assert bench.coarsen_alg_bytes(c, lengths, weighted=True) == read + 8 * 8 + written * (2 * 64 + 2) * 2 + 8
    assert bench.coarsen_alg_bytes(c, lengths, meta=True) == read + written * ((2 * 64 + 2) * 2 + 16) + 8


def test_decode_bytes_count_shared_pages_once():
    wl = types.SimpleNamespace(dtype="bf16", B=2, H_q=8, H_kv=2, d=64,
                               page_table=np.array([[0, 1, 2], [0, 1, 3]], np.int32))
    lengths = np.array([40, 20], np.int32)             # pages 0, 1, 2 (8 used) and 0, 1 (4 used)
    entries = (16 + 16 + 8) * 2                        # page 1 counts its 16 slots once
    qol = 2 * 8 * (64 * 2 + 64 * 4 + 4)
    assert bench.decode_alg_bytes(wl, lengths) == entries * (2 * 64 + 2) * 2 + qol
    assert bench.decode_alg_bytes(wl, lengths, q_tokens=3) == entries * (2 * 64 + 2) * 2 + 3 * qol
    assert bench.decode_alg_bytes(wl, lengths, diag=True) == entries * (3 * 64 + 2) * 2 + qol


def test_merge_and_policy_bytes():
    c = small_call()
    lengths = np.array([10, 40], np.int32)
    ranged = (10 + 8) * 2                              # entries in [entry_start, length) per head
    assert bench.merge_alg_bytes(c, lengths, 5) == 16 * ranged + 4 * ((2 * 64 + 2) * 2 + 16) * 5
    spec = types.SimpleNamespace(n_segments=4)
    assert bench.policy_alg_bytes(c, spec) == 2 * 8 * 2 * 64 * 2 + 8 * 2 + 4 * (2 * 4 + 1) + 4 * 3


def test_merge_pair_count_halves_the_macro_nodes_of_each_range():
    """Per (sequence, head): macro-nodes in [entry_start, length), halved and
    rounded down; C-points (kind 1), nulls and entries outside the range do
    not count."""
    meta = np.zeros((4, 2, 16, 4), np.int32)
    table = np.array([[2, 0], [1, 3]], np.int32)
    meta[2, 0, 3:8, 0] = 2                     # sequence 0, head 0: 5 macro-nodes in range
    meta[2, 0, 5, 0] = 1                       # one of them a C-point: 4 left -> 2 pairs
    meta[0, 1, 0:3, 0] = 2                     # sequence 0, head 1: entries 16..18 -> 1 pair
    meta[2, 1, 0:2, 0] = 2                     # before entry_start: not counted
    meta[1, 0, 14:16, 0] = 2                   # sequence 1, head 0: entries 14, 15
    meta[3, 0, 0, 0] = 2                       # entry 16 -> 3 nodes -> 1 pair
    meta[3, 1, 5, 0] = 2                       # entry 21: past length 20, not counted
    assert bench.merge_pair_count(meta, table, [3, 10], [19, 20]) == 2 + 1 + 1


def test_traffic_table_follows_the_sources(tmp_path, monkeypatch):
    """A traffic line counts only while its digest matches the kernel's
    sources; a missing file gives None."""
    assert bench.measured_traffic("no_such_workload") is None
    prof = tmp_path / "profiles"
    prof.mkdir()
    dig = bench.kernel_digest("decode_mfma_kernel")
    (prof / "traffic_w.txt").write_text(
        f"traffic_bytes decode_mfma_kernel 123 {dig}\n"
        f"traffic_bytes merge_level_kernel 456 {'0' * 64}\n")
    digests = {k: bench.kernel_digest(k) for k in bench.KERNEL_SOURCE}   # of the real sources
    monkeypatch.setattr(bench, "kernel_digest", lambda k: digests[k])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    t = bench.measured_traffic("w")
    assert t == {"decode_mfma_kernel": 123.0}


def test_host_description_reports_threads_within_affinity(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    h = bench.host_description()
    assert h["nproc"] >= h["affinity"] >= 1
    assert h["threads"] == min(3, h["affinity"])
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_description()["threads"] == h["affinity"]


def _write_csv(path, header, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summary_from_rocprof_csv(tmp_path, monkeypatch):
    """The summary's durations, calibrated traffic and digest lines, from
    hand-made rocprofv3 CSV files (kernel trace and counter collection)."""
    out = tmp_path / "out"
    th = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    name = "void spicy::decode_mfma_kernel<128, 3, false, 1, 4>(spicy::DecodeArgs)"
    _write_csv(out / "trace" / "run_kernel_trace.csv", th,
               [["KERNEL_DISPATCH", name, 1000 * i, 1000 * i + 10000 + 1000 * (i % 2)] for i in range(4)])
    ch = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(out / "FETCH_SIZE" / "run_counter_collection.csv", ch,
               [[i, name, "FETCH_SIZE", 100.0] for i in range(3)])
    _write_csv(out / "WRITE_SIZE" / "run_counter_collection.csv", ch,
               [[i, name, "WRITE_SIZE", 10.0] for i in range(3)])
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
    _write_csv(out / "copy_FETCH_SIZE" / "run_counter_collection.csv", ch, [[0, neg, "FETCH_SIZE", 262144.0]])
    _write_csv(out / "copy_WRITE_SIZE" / "run_counter_collection.csv", ch, [[0, neg, "WRITE_SIZE", 524288.0]])
    _write_csv(out / "pmc_occupancy" / "run_counter_collection.csv", ch,
               [[i, name, "SQ_WAVES", 2048.0] for i in range(3)])
    (tmp_path / "profiles").mkdir()
    digests = {k: bench.kernel_digest(k) for k in bench.KERNEL_SOURCE}   # of the real sources
    monkeypatch.setattr(bench, "kernel_digest", lambda k: digests[k])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    args = bench.parse(["--summarize-profile", str(out), "--profile-name", "t", "--profile-commands", "a; b",
                        "--profile-last", "2"])
    bench.summarize_profile(args)
    text = (tmp_path / "profiles" / "t.txt").read_text()
    assert "  a" in text and "  b" in text
    row = [l for l in text.splitlines() if l.startswith("decode_mfma_kernel")][0].split()
    assert row[1] == "4" and abs(float(row[2]) - 10.5) < 1e-9       # 4 dispatches of 10 or 11 us
    # 512 MiB copy: FETCH 256 MiB -> factor 2, WRITE 512 MiB -> factor 1
    b = 100 * 1024 * 2 + 10 * 1024 * 1
    assert f"traffic_bytes decode_mfma_kernel {b} {digests['decode_mfma_kernel']}" in text
    assert "SQ_WAVES" in text and "2048" in text


def test_compact_bytes():
    """Two sequences, H = 2, d = 64 bf16 with metadata: every alpha of the
    range read once, moved entries read and written whole, nulls written to
    the end of the new last page, the range's page ids and three int32 per
    sequence."""
    c = types.SimpleNamespace(dtype="bf16", H_kv=2, d=64, B=2, entry_start=np.array([3, 16], np.int32))
    table = np.array([[0, 1], [2, 3]], np.int32)
    null = np.zeros((4, 2, 16), bool)
    # sequence 0, range [3, 20): head 0 nulls at 5 and 17, head 1 none
    null[0, 0, 5] = True
    null[1, 0, 1] = True
    # sequence 1, range [16, 24): head 0 all null, head 1 null at 16 only
    null[3, 0, :8] = True
    null[3, 1, 0] = True
    lengths = np.array([20, 24], np.int32)
    new = np.array([20, 23], np.int32)           # head 1 keeps all 17 / head 1 keeps 7
    entry = (2 * 64 + 2) * 2 + 16
    # seq 0: head 0 moves 6..16 (11 entries) and 18, 19 (2): 13 moves; live 15, pad 3+15..32 -> 14 nulls
    #        head 1: nothing moves, pad 20..32 -> 12 nulls
    s0 = 2 * 17 * 2 + 4 * 2 + 2 * entry * 13 + entry * (32 - 18) + entry * (32 - 20)
    # seq 1: head 0: no live entries, pad 16..32 -> 16 nulls; head 1: 7 moves, pad 23..32 -> 9 nulls
    s1 = 2 * 8 * 2 + 4 * 1 + entry * 16 + 2 * entry * 7 + entry * 9
    assert bench.compact_alg_bytes(c, table, null, lengths, new) == s0 + s1 + 12 * 2


def test_kernel_names_from_rocprof():
    """Template arguments, namespaces and anonymous namespaces removed."""
    assert bench._base_kernel_name("void spicy::decode_mfma_kernel<128, 3, false, 1, 4>(spicy::DecodeArgs)") == \
        "decode_mfma_kernel"
    assert bench._base_kernel_name("void spicy::(anonymous namespace)::merge_level_kernel<unsigned short, 128>"
                                   "(spicy::MergeArgs)") == "merge_level_kernel"
    assert bench._base_kernel_name("void spicy::(anonymous namespace)::compact_move_kernel<2>(spicy::CompactArgs)") \
        == "compact_move_kernel"
    assert bench._base_kernel_name("void (anonymous namespace)::stream_read_kernel<1>(HIP_vector_type<unsigned "
                                   "int, 4u> const*, unsigned long, unsigned int*)") == "stream_read_kernel"
