"""Device buffers of a paged three-segment cache (allocation only).

Holds the BF16 window, the INT2 (and INT4) page pool, the page tables and the per-request
lengths that the C ABI takes, with the byte sizes the library reports.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import ops
from ._lib import Layout


@dataclasses.dataclass
class CacheBuffers:
    layout: Layout
    batch: int
    max_seq_len: int
    window: torch.Tensor
    pool: torch.Tensor
    page_table: torch.Tensor
    page_table4: Optional[torch.Tensor]
    seq_len: torch.Tensor
    n_int4: Optional[torch.Tensor]

    @property
    def mixed(self) -> bool:
        return bool(self.layout.mixed)


def allocate_cache(num_q_heads: int, num_kv_heads: int, head_dim: int, batch: int, max_seq_len: int, *,
                   sink_len: int = 64, recent_len: int = 256, mixed: bool = False,
                   pages4_per_request: int = 0, pages2_per_request: Optional[int] = None,
                   page_order2: Optional[np.ndarray] = None, page_order4: Optional[np.ndarray] = None,
                   clip_k: float = 0.96, clip_v: float = 0.92, clip_k4: float = 1.0, clip_v4: float = 1.0,
                   codebook: Optional[torch.Tensor] = None, device: str = "cuda") -> CacheBuffers:
    """Allocate buffers for ``batch`` requests of up to ``max_seq_len`` tokens.

    INT2 page ids are [0, P2) and INT4 page ids [P2, P2 + P4) (the INT4 region starts at the
    pool offset). ``page_order2``/``page_order4`` are permutations giving which pool page each
    table entry points at (a shuffled shared pool); identity when omitted. ``codebook``: optional
    INT2 codebook table [Hkv, 2, 4] int16 (device) that the layout points at."""
    hist = max(0, max_seq_len - sink_len - recent_len)
    hp = (hist + 15) // 16
    pp2 = hp if pages2_per_request is None else pages2_per_request
    pp4 = pages4_per_request if mixed else 0
    p2, p4 = batch * pp2, batch * pp4
    layout = ops.make_layout(num_q_heads, num_kv_heads, head_dim, sink_len=sink_len, recent_len=recent_len,
                             mixed=mixed, int4_page_offset=p2 if mixed else 0, pool_pages=p2 + p4, clip_k=clip_k,
                             clip_v=clip_v, clip_k4=clip_k4, clip_v4=clip_v4, codebook=codebook)
    stride = max(pp2, pp4, 1)
    o2 = np.arange(p2, dtype=np.int64) if page_order2 is None else np.asarray(page_order2, np.int64)
    pt2 = np.zeros((batch, stride), np.int32)
    for b in range(batch):
        pt2[b, :pp2] = o2[b * pp2:(b + 1) * pp2]
    pt4 = None
    if mixed:
        o4 = np.arange(p4, dtype=np.int64) if page_order4 is None else np.asarray(page_order4, np.int64)
        pt4 = np.zeros((batch, stride), np.int32)
        for b in range(batch):
            pt4[b, :pp4] = p2 + o4[b * pp4:(b + 1) * pp4]
    dev = torch.device(device)
    return CacheBuffers(
        layout=layout, batch=batch, max_seq_len=max_seq_len,
        window=torch.zeros(max(ops.window_bytes(layout, batch), 1), dtype=torch.uint8, device=dev),
        pool=torch.zeros(max(ops.pool_bytes(layout), 1), dtype=torch.uint8, device=dev),
        page_table=torch.from_numpy(pt2).to(dev),
        page_table4=None if pt4 is None else torch.from_numpy(pt4).to(dev),
        seq_len=torch.zeros(batch, dtype=torch.int32, device=dev),
        n_int4=torch.zeros(batch, dtype=torch.int32, device=dev) if mixed else None)
