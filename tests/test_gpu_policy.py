"""GPU parity of spicy_policy (through the C ABI) against the CPU oracle.

The policy is integer arithmetic on both sides, so the bar is bit-exact for
every output: the segment offsets, seq_seg_ptr, the protection mask, and (from
the workspace) the per-token variation d_t and the squared fixed-point key
norms.
"""
import numpy as np
import pytest
import torch

import coarse_grained_decode_amd as cgd
import oracle
from coarse_grained_decode_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def run_gpu(k, v, so, ptr, idx, N, L, sink, recent):
    T, H, d = k.shape
    B = len(so) - 1
    kt, vt = bf16_tensor(k), bf16_tensor(v)
    so_t = torch.from_numpy(np.asarray(so, np.int32)).to(DEV)
    pp = torch.from_numpy(np.asarray(ptr, np.int32)).to(DEV)
    pi = torch.from_numpy(np.asarray(idx, np.int32) if len(idx) else np.zeros(1, np.int32)).to(DEV)
    if not len(idx):
        pi = pi[:0]
    seg = torch.full((B * N + 1,), -7, dtype=torch.int32, device=DEV)
    ssp = torch.full((B + 1,), -7, dtype=torch.int32, device=DEV)
    mask = torch.full((T, H), 9, dtype=torch.uint8, device=DEV)
    ws = cgd.workspace(cgd.spicy_policy_workspace_bytes(T, H), DEV)
    cgd.spicy_policy(kt, vt, so_t, pp, pi, N, L, sink, recent, seg, ssp, mask, ws)
    torch.cuda.synchronize()
    err = int(ws[0].item())
    wsb = ws.cpu().numpy().view(np.uint8)
    var = wsb[256:256 + 8 * T].view(np.int64)
    off = 256 + (8 * T + 255) // 256 * 256
    n2 = wsb[off:off + 8 * T * H].view(np.uint64).reshape(T, H)
    return seg.cpu().numpy(), ssp.cpu().numpy(), mask.cpu().numpy(), var, n2, err


def check(case_name, k, v, so, ptr, idx, N, L, sink, recent):
    print(f"[policy] {case_name}: tokens={k.shape[0]} H={k.shape[1]} d={k.shape[2]} B={len(so) - 1} "
          f"N={N} L={L} sink={sink} recent={recent}", flush=True)
    ref = oracle.policy(k, v, so, ptr, idx, N, L, sink, recent)
    seg, ssp, mask, var, n2, err = run_gpu(k, v, so, ptr, idx, N, L, sink, recent)
    assert err == 0, f"device error word {err:#x}"
    assert np.array_equal(var, ref.variation), "variation d_t differs"
    assert np.array_equal(n2, ref.norm2), "key norms differ"
    assert np.array_equal(ssp, ref.seq_seg_ptr), "seq_seg_ptr differs"
    assert np.array_equal(seg, ref.seg_offsets), "segment offsets differ"
    assert np.array_equal(mask, ref.mask), "protection mask differs"
    return ref


RANDOM = [
    # (seed, B, T range, H, d, N, L, sink, recent)
    (1, 3, (1, 300), 2, 64, 9, 4, 2, 3),
    (2, 5, (40, 700), 4, 128, 17, 7, 0, 0),
    (3, 2, (90, 200), 16, 128, 11, 5, 1, 1),       # 4 row chunks per lane
    (4, 3, (33, 160), 12, 128, 6, 9, 0, 2),        # 3 chunks per lane (padded template)
    (5, 4, (1, 64), 8, 64, 40, 3, 0, 0),           # N above most lengths: empty slots
    (6, 2, (500, 1500), 1, 64, 50, 20, 8, 48),
    (7, 6, (0, 40), 3, 64, 4, 100, 0, 0),          # empty sequences; every candidate a landmark
    (8, 2, (64, 64), 4, 128, 1, 0, 0, 0),          # one slot, no landmarks
]


@pytest.mark.parametrize("case", RANDOM)
def test_policy_random_cases(case):
    _need_gpu()
    seed, B, Tr, H, d, N, L, sink, recent = case
    c = W.random_policy_case(seed, B=B, T_range=Tr, H=H, d=d, n_segments=N, n_landmarks=L, sink=sink,
                             recent=recent)
    check(f"random seed {seed}", c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, N, L, sink, recent)


def test_policy_constant_and_short_sequences():
    _need_gpu()
    H, d = 2, 64
    c = W.random_policy_case(20, B=4, T_range=(1, 3), H=H, d=d, n_segments=5, n_landmarks=1)
    check("one to three tokens", c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, 5, 1, 1, 1)
    T = 100
    k = np.tile(W.f32_to_bf16_bits(np.linspace(-2, 2, H * d, dtype=np.float32)).reshape(1, H, d), (T, 1, 1))
    so = np.array([0, 37, T], dtype=np.int32)
    check("constant tokens", k, k.copy(), so, c.spec.proj_ptr, c.spec.proj_idx, 7, 3, 0, 0)


def test_policy_every_bf16_pattern():
    """Token t's key row holds bit pattern t in one dimension (zeros
    elsewhere) and its value row the pattern t ^ 0x8000: every fixed-point
    conversion shows in the norms and the variation."""
    _need_gpu()
    T, H, d = 1 << 16, 1, 64
    k = np.zeros((T, H, d), dtype=np.uint16)
    v = np.zeros((T, H, d), dtype=np.uint16)
    k[:, 0, 5] = np.arange(T, dtype=np.uint32).astype(np.uint16)
    v[:, 0, 9] = (np.arange(T, dtype=np.uint32) ^ 0x8000).astype(np.uint16)
    ptr, idx = np.array([0, 2, 3], np.int32), np.array([6, -(64 + 10), 6], np.int32)
    so = np.array([0, 1000, 40000, T], dtype=np.int32)
    ref = check("all bf16 patterns", k, v, so, ptr, idx, 64, 10, 0, 0)
    want = np.array([oracle.fix16(b) ** 2 for b in range(T)], dtype=np.uint64)
    assert np.array_equal(ref.norm2[:, 0], want)


def test_policy_full_chunk():
    """The benchmark's per-step chunk: 32 sequences of 8192 tokens, 4 KV
    heads, d = 128, N = 204 slots, 82 landmarks per head."""
    _need_gpu()
    wl = W.shared_prefix()
    st, pol = wl.step, wl.policy
    check("shared_prefix chunk", st.k, st.v, st.seq_offsets, pol.proj_ptr, pol.proj_idx, pol.n_segments,
          pol.n_landmarks, pol.sink, pol.recent)


def test_policy_feeds_coarsen():
    """Policy output straight into spicy_coarsen: no device error, and the
    lengths match the oracle's coarsening of the oracle's policy output."""
    _need_gpu()
    from coarse_grained_decode_amd.runner import _tensor
    c = W.random_policy_case(31, B=3, T_range=(200, 600), H=2, d=128, n_segments=12, n_landmarks=6, sink=2,
                             recent=4)
    N, L = 12, 6
    ref = oracle.policy(c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, N, L, 2, 4)
    B, T, H, d = 3, c.k.shape[0], 2, 128
    lens = np.diff(c.seq_offsets)
    max_pages = int(-(-(lens.max() + 16) // 16)) + 1
    table = np.arange(B * max_pages, dtype=np.int32).reshape(B, max_pages)
    call = W.CoarsenCall("bf16", H, d, 1e6, c.k, c.v, c.seq_offsets.astype(np.int32),
                         np.zeros(B, np.int32), ref.seg_offsets, ref.seq_seg_ptr, ref.mask, table,
                         np.zeros(B, np.int32))
    rcache = oracle.Cache("bf16", B * max_pages, H, d)
    rlen = oracle.coarsen(call, rcache)

    seg, ssp, mask, _, _, err = run_gpu(c.k, c.v, c.seq_offsets, c.spec.proj_ptr, c.spec.proj_idx, N, L, 2, 4)
    assert err == 0
    cache = cgd.PagedCache.empty(B * max_pages, H, d, torch.bfloat16, DEV, meta=True)
    so_t = torch.from_numpy(c.seq_offsets.astype(np.int32)).to(DEV)
    lengths = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = cgd.workspace(cgd.spicy_coarsen_workspace_bytes(B, B * N, T, H, d, cgd.SPICY_BF16), DEV)
    cgd.spicy_coarsen(cache, bf16_tensor(c.k), bf16_tensor(c.v), so_t, torch.zeros(B, dtype=torch.int32, device=DEV),
                      torch.from_numpy(seg).to(DEV), torch.from_numpy(ssp).to(DEV), torch.from_numpy(mask).to(DEV),
                      1e6, torch.from_numpy(table).to(DEV), torch.zeros(B, dtype=torch.int32, device=DEV), lengths, ws)
    torch.cuda.synchronize()
    assert int(ws[0].item()) == 0
    assert np.array_equal(lengths.cpu().numpy(), rlen)
