"""GPU parity of spicy_decode_attn_multi (several query tokens per sequence)
against the CPU oracle, through the C ABI.

Same bars as the single-query decode: bf16 storage O max-abs <= 1e-2 and LSE
relative <= 1e-3, fp32 storage 2e-5 / 1e-5.  Two exact invariants on top:
one token is bit-identical to spicy_decode_attn_shared, and permuting the
tokens permutes the outputs bit for bit (each row's result depends only on its
own query).
"""
import numpy as np
import pytest
import torch

import oracle
from coarse_grained_decode_amd import workloads as W
from test_gpu_parity import DEV, _need_gpu, compare_decode, gpu_decode_shared, upload_case

pytestmark = pytest.mark.gpu


def oracle_multi(c):
    cache = oracle.Cache(c.dtype, c.k.shape[0], c.H_kv, c.d, fill=False)
    cache.k[:] = c.k; cache.v[:] = c.v; cache.ab[:] = c.ab
    return oracle.decode_multi(c.q, c.dtype, cache, c.page_table, c.lengths)


def gpu_multi(cache, q, table, lengths, P, H_kv, num_splits=0):
    import coarse_grained_decode_amd as cgd
    B, n_q, H_q, d = q.shape
    tb = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(DEV)
    ln = torch.from_numpy(np.ascontiguousarray(lengths, dtype=np.int32)).to(DEV)
    o = torch.empty(B, n_q, H_q, d, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, n_q, H_q, dtype=torch.float32, device=DEV)
    ws = cgd.workspace(cgd.spicy_decode_multi_workspace_bytes(B, n_q, H_q, H_kv, d, tb.shape[1], P, num_splits), DEV)
    cgd.spicy_decode_attn_multi(cache, q, tb, ln, P, o, lse, ws, num_splits)
    torch.cuda.synchronize()
    assert cgd.device_error(ws) == 0
    return o, lse


MULTI_CASES = [
    # (seed, B, H_q, H_kv, d, dtype, prefix pages, private pages, query tokens)
    (21, 5, 28, 4, 128, "bf16", 0, (1, 6), 2),      # 14 rows per KV head: one tile
    (22, 3, 28, 4, 128, "bf16", 6, (2, 5), 3),      # 21 rows: two tiles, shared prefix
    (23, 4, 16, 2, 64, "bf16", 3, (1, 4), 4),       # 32 rows: exactly two tiles
    (24, 2, 8, 8, 128, "bf16", 0, (3, 3), 16),      # G = 1: sixteen tokens fill one tile
    (25, 6, 12, 2, 64, "bf16", 5, (0, 2), 5),       # 30 rows; some sequences prefix only
    (26, 3, 4, 2, 64, "f32", 2, (1, 3), 3),         # fp32 path
]


@pytest.mark.parametrize("case", MULTI_CASES)
def test_multi_token_decode_matches_oracle(case):
    _need_gpu()
    seed, B, H_q, H_kv, d, dtype, P, priv, n_q = case
    print(f"[multi] seed {seed}: B={B} H_q={H_q} H_kv={H_kv} d={d} {dtype} P={P} n_q={n_q}", flush=True)
    c = W.random_decode_case(seed, B=B, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, prefix_pages=P,
                             private_pages=priv, q_tokens=n_q)
    ro, rlse = oracle_multi(c)
    cache, q = upload_case(c)
    for ns in (0, 1, 3):
        o, lse = gpu_multi(cache, q, c.page_table, c.lengths, P, H_kv, num_splits=ns)
        compare_decode(o.reshape(B * n_q, H_q, d), lse.reshape(B * n_q, H_q),
                       ro.reshape(B * n_q, H_q, d), rlse.reshape(B * n_q, H_q), dtype)


def test_one_token_is_the_shared_decode_and_tokens_permute():
    _need_gpu()
    B, H_q, H_kv, d, P, n_q = 6, 28, 4, 128, 4, 3
    c = W.random_decode_case(31, B=B, H_q=H_q, H_kv=H_kv, d=d, prefix_pages=P, private_pages=(1, 5), q_tokens=n_q)
    cache, q = upload_case(c)
    o1, l1 = gpu_multi(cache, q[:, :1].contiguous(), c.page_table, c.lengths, P, H_kv)
    os_, ls_ = gpu_decode_shared(cache, q[:, 0].contiguous(), c.page_table, c.lengths, P, H_kv)
    assert torch.equal(o1[:, 0], os_) and torch.equal(l1[:, 0], ls_)
    o, lse = gpu_multi(cache, q, c.page_table, c.lengths, P, H_kv)
    perm = [2, 0, 1]
    op, lp = gpu_multi(cache, q[:, perm].contiguous(), c.page_table, c.lengths, P, H_kv)
    assert torch.equal(op, o[:, perm]) and torch.equal(lp, lse[:, perm])
