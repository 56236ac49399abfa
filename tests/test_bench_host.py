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


def test_traffic_table_follows_the_sources(tmp_path, monkeypatch):
    """A traffic line counts only while its digest matches the kernel's
    sources; a missing file gives None."""
    assert bench.measured_traffic("no_such_workload") is None
    prof = tmp_path / "profiles"
    prof.mkdir()
    dig = bench.kernel_digest("decode_mfma_kernel")
    (prof / "traffic_w.txt").write_text(
        f"traffic_bytes decode_mfma_kernel 123 {dig}\n"
        f"traffic_bytes combine_kernel 456 {'0' * 64}\n")
    digests = {k: bench.kernel_digest(k) for k in bench.KERNEL_SOURCE}   # of the real sources
    monkeypatch.setattr(bench, "kernel_digest", lambda k: digests[k])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    t = bench.measured_traffic("w")
    assert t == {"decode_mfma_kernel": 123.0}
