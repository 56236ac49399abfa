"""The Python binding rejects tensors the kernels would misread before anything
reaches the C ABI: wrong dtype (a bf16 output where the kernel writes fp32, a
query in another dtype than the cache), non-contiguous tables, wrong shapes,
sizes beyond a tensor, tensors on another device than the cache.  Host only:
every call here raises before the library is entered."""
import os

import pytest
import torch

import coarse_grained_decode_amd as cgd


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cgd.library_path()):
        from coarse_grained_decode_amd import build
        build.build(verbose=False)
    return cgd.load_library()


B, H, G, D, P = 2, 2, 3, 64, 8


def cache(dtype=torch.bfloat16):
    return cgd.PagedCache.empty(P, H, D, dtype, "cpu", meta=True)


def decode_args(dtype=torch.bfloat16):
    return dict(q=torch.zeros(B, H * G, D, dtype=dtype), page_table=torch.zeros(B, 4, dtype=torch.int32),
                lengths=torch.zeros(B, dtype=torch.int32), o=torch.zeros(B, H * G, D, dtype=torch.float32),
                lse=torch.zeros(B, H * G, dtype=torch.float32), workspace=torch.zeros(64, dtype=torch.int32))


@pytest.mark.parametrize("change,match", [
    (dict(o=torch.zeros(B, H * G, D, dtype=torch.bfloat16)), "o: dtype"),
    (dict(q=torch.zeros(B, H * G, D, dtype=torch.float32)), "q: dtype"),
    (dict(lse=torch.zeros(B, H * G + 1, dtype=torch.float32)), "lse: shape"),
    (dict(q=torch.zeros(B, H * G, 2 * D, dtype=torch.bfloat16)), "q: shape"),
    (dict(page_table=torch.zeros(4, B, dtype=torch.int32).t()), "page_table: must be contiguous"),
    (dict(page_table=torch.zeros(B, 4, dtype=torch.int64)), "page_table: dtype"),
    (dict(lengths=torch.zeros(B, dtype=torch.int64)), "lengths: dtype"),
    (dict(lengths=torch.zeros(B - 1, dtype=torch.int32)), "fewer rows"),
])
def test_decode_rejects(lib, change, match):
    a = decode_args()
    a.update(change)
    with pytest.raises(ValueError, match=match):
        cgd.spicy_decode_attn(cache(), a["q"], a["page_table"], a["lengths"], a["o"], a["lse"], a["workspace"])


def test_decode_rejects_sizes_beyond_the_tensors(lib):
    a = decode_args()
    with pytest.raises(ValueError, match="max_pages_per_seq"):
        cgd.spicy_decode_attn(cache(), a["q"], a["page_table"], a["lengths"], a["o"], a["lse"], a["workspace"],
                              max_pages_per_seq=5)
    with pytest.raises(ValueError, match="B:"):
        cgd.spicy_decode_attn_shared(cache(), a["q"], a["page_table"], a["lengths"], 0, a["o"], a["lse"],
                                     a["workspace"], B=3)


def test_multi_decode_rejects(lib):
    a = decode_args()
    q4 = torch.zeros(B, 2, H * G, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="o: shape"):
        cgd.spicy_decode_attn_multi(cache(), q4, a["page_table"], a["lengths"], 0, a["o"], a["lse"], a["workspace"])
    with pytest.raises(ValueError, match=r"\[B, n_q, H_q, d\]"):
        cgd.spicy_decode_attn_multi(cache(), a["q"], a["page_table"], a["lengths"], 0, a["o"], a["lse"],
                                    a["workspace"])


def test_cache_pool_shapes_are_checked(lib):
    c = cache()
    c.ab = torch.zeros(P, H, 16, 3, dtype=torch.bfloat16)
    a = decode_args()
    with pytest.raises(ValueError, match="cache.ab"):
        cgd.spicy_decode_attn(c, a["q"], a["page_table"], a["lengths"], a["o"], a["lse"], a["workspace"])


def coarsen_args(T=10, dtype=torch.bfloat16):
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    return dict(k_pre=torch.zeros(T, H, D, dtype=dtype), v=torch.zeros(T, H, D, dtype=dtype),
                seq_offsets=i32(B + 1), pos_base=None, seg_offsets=i32(4), seq_seg_ptr=i32(B + 1),
                protected_mask=torch.zeros(T, H, dtype=torch.uint8), rope_base=1e4, page_table=i32(B, 4),
                entry_start=None, lengths_out=i32(B), workspace=i32(64))


@pytest.mark.parametrize("change,match", [
    (dict(k_pre=torch.zeros(10, H, D, dtype=torch.float32)), "k_pre: dtype"),
    (dict(v=torch.zeros(11, H, D, dtype=torch.bfloat16)), "v: shape"),
    (dict(protected_mask=torch.zeros(10, H, dtype=torch.int32)), "protected_mask: dtype"),
    (dict(seq_offsets=torch.zeros(B + 1, dtype=torch.int64)), "seq_offsets: dtype"),
    (dict(lengths_out=torch.zeros(B - 1, dtype=torch.int32)), "lengths_out"),
    (dict(k_pre=torch.zeros(10, H + 1, D, dtype=torch.bfloat16)), "k_pre: shape"),
])
def test_coarsen_rejects(lib, change, match):
    a = coarsen_args()
    a.update(change)
    with pytest.raises(ValueError, match=match):
        cgd.spicy_coarsen(cache(), **a)


def test_coarsen_rejects_counts_beyond_the_tensors(lib):
    with pytest.raises(ValueError, match="total_tokens"):
        cgd.spicy_coarsen(cache(), **coarsen_args(), total_tokens=11)
    with pytest.raises(ValueError, match="n_seg"):
        cgd.spicy_coarsen(cache(), **coarsen_args(), n_seg=4)
    a = coarsen_args()
    with pytest.raises(ValueError, match="token_weight"):
        cgd.spicy_coarsen_weighted(cache(), a["k_pre"], a["v"], a["seq_offsets"], None, a["seg_offsets"],
                                   a["seq_seg_ptr"], a["protected_mask"], torch.zeros(9, dtype=torch.int64), 1e4,
                                   a["page_table"], None, a["lengths_out"], a["workspace"])


def test_merge_and_policy_reject(lib):
    c = cache()
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    with pytest.raises(ValueError, match="entry_end"):
        cgd.spicy_merge_level(c, 1e4, i32(B, 4), i32(B), i32(B + 1), 10, i32(64))
    k = torch.zeros(10, H, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="seg_offsets"):
        cgd.spicy_policy(k, k, i32(B + 1), i32(3), i32(4), 5, 1, 0, 0, i32(B * 5), i32(B + 1),
                         torch.zeros(10, H, dtype=torch.uint8), i32(64))
    with pytest.raises(ValueError, match="k_pre: dtype"):
        cgd.spicy_policy(k.float(), k, i32(B + 1), i32(3), i32(4), 5, 1, 0, 0, i32(B * 5 + 1), i32(B + 1),
                         torch.zeros(10, H, dtype=torch.uint8), i32(64))


def test_compact_rejects(lib):
    c = cache()
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    ln = i32(B)
    with pytest.raises(ValueError, match="lengths_out: must be a tensor of its own"):
        cgd.spicy_compact_range(c, i32(B, 4), i32(B), ln, ln, i32(1))
    with pytest.raises(ValueError, match="lengths: shape"):
        cgd.spicy_compact_range(c, i32(B, 4), i32(B), i32(B + 1), i32(B), i32(1))
    with pytest.raises(ValueError, match="device_error: dtype"):
        cgd.spicy_compact_range(c, i32(B, 4), i32(B), i32(B), i32(B), torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError, match="page_table"):
        cgd.spicy_compact_range(c, i32(B - 1, 4), i32(B), i32(B), i32(B), i32(1))
