"""spicy_decode_attn_multi_noalloc (the decode for callers that cannot
allocate: no workspace, the library's own per-device scratch array) against
spicy_decode_attn_multi on the same inputs, through the C ABI: two calls in
a row, the second with a smaller batch, each bit for bit equal to the
workspace decode (same plan, same kernels, same order of operations)."""
import numpy as np
import pytest
import torch

import coarse_grained_decode_amd as cgd
from coarse_grained_decode_amd import workloads as W
from coarse_grained_decode_amd.runner import _tensor

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed, B, n_q, prefix_pages, dtype):
    c = W.random_decode_case(seed, B=B, H_q=14, H_kv=2, d=128 if dtype == "bf16" else 64, dtype=dtype,
                             prefix_pages=prefix_pages, private_pages=(0, 9), q_tokens=n_q)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = cgd.PagedCache(_tensor(c.k, dtype, DEV), _tensor(c.v, dtype, DEV), _tensor(c.ab, dtype, DEV), None)
    q = _tensor(c.q, dtype, DEV).view(B, n_q, 14, c.d)
    assert q.dtype == tdt
    table = torch.from_numpy(np.ascontiguousarray(c.page_table, dtype=np.int32)).to(DEV)
    lengths = torch.from_numpy(np.ascontiguousarray(c.lengths, dtype=np.int32)).to(DEV)
    return c, cache, q, table, lengths


def _both(c, cache, q, table, lengths, P):
    B, n_q, H_q, d = q.shape
    o1 = torch.full((B, n_q, H_q, d), float("nan"), device=DEV)
    l1 = torch.full((B, n_q, H_q), float("nan"), device=DEV)
    ws = cgd.workspace(cgd.spicy_decode_multi_workspace_bytes(B, n_q, H_q, 2, d, table.shape[1], P), DEV)
    cgd.spicy_decode_attn_multi(cache, q, table, lengths, P, o1, l1, ws)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    cgd.spicy_decode_attn_multi_noalloc(cache, q, table, lengths, P, o2, l2, err)
    torch.cuda.synchronize()
    assert cgd.device_error(ws) == 0 and int(err.item()) == 0
    return o1.cpu(), l1.cpu(), o2.cpu(), l2.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_equals_workspace_decode(dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: 6 sequences x 3 tokens with a shared prefix; second: 2 x 1
    for seed, B, n_q, P in ((5, 6, 3, 2), (6, 2, 1, 0)):
        c, cache, q, table, lengths = _case(seed, B, n_q, P, dtype)
        o1, l1, o2, l2 = _both(c, cache, q, table, lengths, P)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call B={B} n_q={n_q}: outputs differ"
        assert torch.isfinite(o1).all()


def test_noalloc_rejects_calls_beyond_its_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c, cache, q, table, lengths = _case(7, 2, 1, 0, "bf16")
    big_q = torch.zeros(4700, 1, 14, 128, dtype=torch.bfloat16, device=DEV)    # 65800 query rows > 65536
    o = torch.zeros(4700, 1, 14, 128, device=DEV)
    lse = torch.zeros(4700, 1, 14, device=DEV)
    tb = torch.zeros(4700, table.shape[1], dtype=torch.int32, device=DEV)
    ln = torch.zeros(4700, dtype=torch.int32, device=DEV)
    with pytest.raises(cgd.SpicyError, match="workspace too small"):
        cgd.spicy_decode_attn_multi_noalloc(cache, big_q, tb, ln, 0, o, lse)
    assert cgd.spicy_decode_noalloc_max_bytes() == 32 << 20
