"""Put a synthetic workload on the GPU and drive it through the C ABI.

Plumbing only: copies the host arrays of a workload to device memory once,
allocates the paged cache pool and the workspaces, and issues
spicy_policy / spicy_coarsen / spicy_decode_attn calls on the current stream.  Used by the
tests, the smoke check and the benchmark.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import (PagedCache, spicy_coarsen, spicy_coarsen_weighted, spicy_coarsen_workspace_bytes, spicy_decode_attn,
               spicy_decode_attn_shared, spicy_decode_num_splits, spicy_decode_plan, spicy_decode_shared_workspace_bytes,
               spicy_decode_attn_multi, spicy_decode_multi_workspace_bytes, spicy_policy,
               spicy_policy_workspace_bytes, spicy_merge_level, spicy_merge_workspace_bytes, workspace,
               spicy_compact_range)
from .workloads import CoarsenCall, PolicySpec, Workload, query_tokens


def _tensor(a: np.ndarray, dtype: str | None, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


@dataclass
class DeviceCall:
    call: CoarsenCall
    k: torch.Tensor
    v: torch.Tensor
    seq_offsets: torch.Tensor
    pos_base: torch.Tensor
    seg_offsets: torch.Tensor
    seq_seg_ptr: torch.Tensor
    mask: torch.Tensor
    page_table: torch.Tensor
    entry_start: torch.Tensor
    lengths: torch.Tensor
    ws: torch.Tensor
    token_weight: Optional[torch.Tensor] = None   # int64 [total_tokens]: spicy_coarsen_weighted

    @staticmethod
    def of(call: CoarsenCall, device) -> "DeviceCall":
        return DeviceCall(
            call=call,
            k=_tensor(call.k, call.dtype, device), v=_tensor(call.v, call.dtype, device),
            seq_offsets=_tensor(call.seq_offsets, None, device), pos_base=_tensor(call.pos_base, None, device),
            seg_offsets=_tensor(call.seg_offsets, None, device), seq_seg_ptr=_tensor(call.seq_seg_ptr, None, device),
            mask=_tensor(call.mask, None, device), page_table=_tensor(call.page_table, None, device),
            entry_start=_tensor(call.entry_start, None, device),
            lengths=torch.zeros(call.B, dtype=torch.int32, device=device),
            ws=workspace(spicy_coarsen_workspace_bytes(call.B, call.n_seg, call.total_tokens, call.H_kv, call.d,
                                                       1 if call.dtype == "bf16" else 0), device),
        )

    def run(self, cache: PagedCache, stream=None) -> None:
        c = self.call
        kw = dict(total_tokens=c.total_tokens, n_seg=c.n_seg, B=c.B, max_pages_per_seq=c.max_pages)
        if self.token_weight is None:
            spicy_coarsen(cache, self.k, self.v, self.seq_offsets, self.pos_base, self.seg_offsets,
                          self.seq_seg_ptr, self.mask, c.rope_base, self.page_table, self.entry_start,
                          self.lengths, self.ws, stream, **kw)
        else:
            spicy_coarsen_weighted(cache, self.k, self.v, self.seq_offsets, self.pos_base, self.seg_offsets,
                                   self.seq_seg_ptr, self.mask, self.token_weight, c.rope_base, self.page_table,
                                   self.entry_start, self.lengths, self.ws, stream, **kw)

    @property
    def input_bytes(self) -> int:
        return self.k.numel() * self.k.element_size() * 2


@dataclass
class DevicePolicy:
    """spicy_policy for a workload's per-step chunk: its inputs (the chunk's
    k, v and sequence offsets come from the step call) and its outputs, which
    the step's coarsening then reads instead of the generator's segments and
    mask."""
    spec: PolicySpec
    proj_ptr: torch.Tensor
    proj_idx: torch.Tensor
    seg_offsets: torch.Tensor      # [B*N + 1]
    seq_seg_ptr: torch.Tensor      # [B+1]
    mask: torch.Tensor             # [total_tokens, H] uint8
    ws: torch.Tensor

    @staticmethod
    def of(spec: PolicySpec, call: CoarsenCall, device) -> "DevicePolicy":
        B, N = call.B, spec.n_segments
        return DevicePolicy(
            spec=spec,
            proj_ptr=_tensor(spec.proj_ptr, None, device), proj_idx=_tensor(spec.proj_idx, None, device),
            seg_offsets=torch.zeros(B * N + 1, dtype=torch.int32, device=device),
            seq_seg_ptr=torch.zeros(B + 1, dtype=torch.int32, device=device),
            mask=torch.zeros((call.total_tokens, call.H_kv), dtype=torch.uint8, device=device),
            ws=workspace(spicy_policy_workspace_bytes(call.total_tokens, call.H_kv), device),
        )

    def run(self, step: "DeviceCall", stream=None) -> None:
        sp = self.spec
        spicy_policy(step.k, step.v, step.seq_offsets, self.proj_ptr, self.proj_idx, sp.n_segments,
                     sp.n_landmarks, sp.sink, sp.recent, self.seg_offsets, self.seq_seg_ptr, self.mask, self.ws,
                     stream, B=step.call.B, total_tokens=step.call.total_tokens)

    @property
    def variation(self) -> torch.Tensor:
        """d_t (int64 [total_tokens]) as spicy_policy leaves it in its workspace."""
        T = self.mask.shape[0]
        return self.ws.view(torch.uint8)[256:256 + 8 * T].view(torch.int64)

    def feed(self, step: "DeviceCall", device, weighted: bool = False) -> "DeviceCall":
        """The step call reading this policy's outputs (N slots per sequence);
        weighted: spicy_coarsen_weighted with the policy's variation d_t as
        the token weights."""
        c = step.call
        B, N = c.B, self.spec.n_segments
        shaped = dataclasses.replace(c, seg_offsets=np.zeros(B * N + 1, dtype=np.int32),
                                     seq_seg_ptr=np.zeros(B + 1, dtype=np.int32))
        return dataclasses.replace(
            step, call=shaped, seg_offsets=self.seg_offsets, seq_seg_ptr=self.seq_seg_ptr, mask=self.mask,
            lengths=torch.zeros(B, dtype=torch.int32, device=device),
            ws=workspace(spicy_coarsen_workspace_bytes(B, B * N, c.total_tokens, c.H_kv, c.d,
                                                       1 if c.dtype == "bf16" else 0), device),
            token_weight=self.variation if weighted else None)


class DyadicPyramid:
    """Host-side schedule of the cascaded dyadic merge for a batch whose
    sequences append chunks in lockstep (SPICY-KV demo page, Claim 12: the
    cascaded dyadic ring-buffer pyramid; Claim 10: the law of total variance
    across cascades).  The blocks of entries form a binary counter: an
    appended chunk is a level-0 block; while the two newest blocks have the
    same level they merge into one block a level up, with one
    spicy_merge_level call over their union (each macro-node pairs with its
    neighbour, so the nodes of a level-l block cover 2^l of the chunk's
    segments).  With compaction (cascade), each merge is followed by
    spicy_compact_range, so a level-l block holds one entry per 2^l base
    segments plus its C-points and the freed pages take the next chunk.  The
    schedule is the host's: the pages give no rule for it.
    """

    def __init__(self, B: int):
        self.B = B
        self.blocks: List[tuple] = []          # (begin int32[B], end int32[B], level)

    def push(self, begin, end) -> None:
        """Record a chunk coarsened into entries [begin[b], end[b]) as a
        level-0 block."""
        self.blocks.append((np.asarray(begin, np.int32).copy(), np.asarray(end, np.int32).copy(), 0))

    def next_merge(self) -> Optional[tuple]:
        """(begin, end) int32 arrays of the merge the two newest blocks are
        due for (they have the same level), or None."""
        if len(self.blocks) >= 2 and self.blocks[-1][2] == self.blocks[-2][2]:
            return self.blocks[-2][0], self.blocks[-1][1]
        return None

    def merged(self, end=None) -> None:
        """Replace the two newest blocks by their union one level up.  end:
        the union's end after spicy_compact_range gave back its freed
        entries (default: the newer block's end, nothing compacted)."""
        b2 = self.blocks.pop()
        b1 = self.blocks.pop()
        e = b2[1] if end is None else np.asarray(end, np.int32).copy()
        self.blocks.append((b1[0], e, b1[2] + 1))

    def append(self, begin, end) -> List[tuple]:
        """Record a chunk coarsened into entries [begin[b], end[b]) and return
        the merges it triggers, in order, as (begin, end) int32 arrays (no
        compaction between them)."""
        self.push(begin, end)
        merges = []
        while (m := self.next_merge()) is not None:
            merges.append(m)
            self.merged()
        return merges

    @property
    def levels(self) -> List[int]:
        return [blk[2] for blk in self.blocks]

    @staticmethod
    def run(cache: PagedCache, merges, rope_base: float, page_table: torch.Tensor, device, stream=None) -> None:
        """Issue spicy_merge_level for each (begin, end) merge on the GPU."""
        for begin, end in merges:
            rng = int((end - begin).max()) if len(begin) else 0
            ws = workspace(spicy_merge_workspace_bytes(len(begin), cache.k.shape[1], rng), device)
            spicy_merge_level(cache, rope_base, page_table, _tensor(begin, None, device), _tensor(end, None, device),
                              rng, ws, stream)

    def cascade(self, cache: PagedCache, lengths: np.ndarray, rope_base: float, page_table: torch.Tensor, device,
                stream=None) -> np.ndarray:
        """Run, on the GPU, every merge the newest block is due for, each
        followed by spicy_compact_range over the merged union, so the pyramid
        keeps only live entries; lengths: the sequences' lengths now (the end
        of the newest block).  Returns the lengths after the last compaction
        (read back after each one: the next merge's range ends there)."""
        lengths = np.asarray(lengths, np.int32).copy()
        err = torch.zeros(1, dtype=torch.int32, device=device)
        while (m := self.next_merge()) is not None:
            begin, _ = m
            rng = int((lengths - begin).max()) if len(begin) else 0
            ws = workspace(spicy_merge_workspace_bytes(len(begin), cache.k.shape[1], rng), device)
            tb, tl = _tensor(begin, None, device), _tensor(lengths, None, device)
            spicy_merge_level(cache, rope_base, page_table, tb, tl, rng, ws, stream)
            out = torch.empty_like(tl)
            spicy_compact_range(cache, page_table, tb, tl, out, err, stream)
            if stream is not None:                      # the readback below orders after torch's stream only
                torch.cuda.synchronize(device)
            lengths = out.cpu().numpy()
            if int(ws[0].item()) or int(err.item()):
                raise RuntimeError(f"pyramid cascade: device error {int(ws[0].item()) | int(err.item()):#x}")
            self.merged(lengths)
        return lengths


@dataclass
class DeviceWorkload:
    wl: Workload
    device: torch.device
    cache: PagedCache
    setup: List[DeviceCall]
    step: Optional[DeviceCall]
    q: torch.Tensor
    page_table: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    num_splits: int
    dws: torch.Tensor
    shared_prefix_pages: int = 0
    lengths: torch.Tensor = field(default=None)
    q_tokens: int = 1

    @staticmethod
    def of(wl: Workload, device="cuda", meta: bool = True, num_splits: int = 0,
           fill: float | None = float("nan"), use_shared_prefix: bool = True,
           q_tokens: int = 1, diag: bool = False) -> "DeviceWorkload":
        """q_tokens > 1: every decode call is spicy_decode_attn_multi with that
        many query tokens per sequence (workloads.query_tokens).  diag: the
        cache carries the diagonal closure's per-dimension variances."""
        device = torch.device(device)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        cache = PagedCache.empty(wl.num_pages, wl.H_kv, wl.d, tdt, device, meta=meta, fill=fill, diag=diag)
        setup = [DeviceCall.of(c, device) for c in wl.setup]
        step = DeviceCall.of(wl.step, device) if wl.step is not None else None
        table = _tensor(wl.page_table, None, device)
        P = wl.shared_prefix_pages if use_shared_prefix else 0
        if q_tokens == 1:
            q = _tensor(wl.q, wl.dtype, device)
            o = torch.empty(wl.B, wl.H_q, wl.d, dtype=torch.float32, device=device)
            lse = torch.empty(wl.B, wl.H_q, dtype=torch.float32, device=device)
        else:
            q = _tensor(query_tokens(wl, q_tokens), wl.dtype, device)
            o = torch.empty(wl.B, q_tokens, wl.H_q, wl.d, dtype=torch.float32, device=device)
            lse = torch.empty(wl.B, q_tokens, wl.H_q, dtype=torch.float32, device=device)
        dws = workspace(spicy_decode_multi_workspace_bytes(wl.B, q_tokens, wl.H_q, wl.H_kv, wl.d, wl.max_pages, P,
                                                           num_splits), device)
        return DeviceWorkload(wl, device, cache, setup, step, q, table, o, lse, num_splits, dws, P,
                              q_tokens=q_tokens)

    def run_setup(self) -> None:
        for c in self.setup:
            c.run(self.cache)
        self.lengths = self.setup[-1].lengths if self.step is None else None

    def run_step_coarsen(self) -> None:
        if self.step is not None:
            self.step.run(self.cache)
            self.lengths = self.step.lengths

    def decode(self, cache: PagedCache | None = None) -> None:
        """spicy_decode_attn, or spicy_decode_attn_shared when the batch
        declares a shared prefix, or spicy_decode_attn_multi with several
        query tokens."""
        cache = self.cache if cache is None else cache
        if self.q_tokens > 1:
            spicy_decode_attn_multi(cache, self.q, self.page_table, self.lengths, self.shared_prefix_pages,
                                    self.o, self.lse, self.dws, self.num_splits)
        elif self.shared_prefix_pages > 0:
            spicy_decode_attn_shared(cache, self.q, self.page_table, self.lengths, self.shared_prefix_pages,
                                     self.o, self.lse, self.dws, self.num_splits)
        else:
            spicy_decode_attn(cache, self.q, self.page_table, self.lengths, self.o, self.lse, self.dws,
                              self.num_splits)

    def step_once(self) -> None:
        """One pass of the hot path: coarsen the per-step chunk (if any), then decode."""
        self.run_step_coarsen()
        self.decode()

    @property
    def splits(self) -> int:
        """Private splits per (sequence, KV head) of this workload's decode call."""
        return self.plan["private_splits"]

    @property
    def plan(self) -> dict:
        """The decode call's split-K plan (spicy_decode_plan)."""
        return spicy_decode_plan(self.wl.B, self.wl.H_q, self.wl.H_kv, self.wl.max_pages,
                                 self.shared_prefix_pages, self.num_splits, self.q_tokens)
