"""The selective-sparse-attention hot path of one workload, on the GPU.

Orchestration only: it moves the seeded inputs to the device, owns the output
and workspace buffers, and calls the libspattn entry points in order
(indexer scores -> certified top-K -> sparse attention; indexer scores ->
certified page selection -> attention over the pages of a paged KV cache;
per-page key bounds -> Quest page selection -> attention over the chosen pages;
block keys -> two-level block-then-token selection -> sparse attention;
block keys -> top blocks per GQA group -> block-sparse attention;
block selection -> block-sparse attention; block selection -> three-branch
NSA attention; or a fixed window + global pattern).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import spattn as S
from .inputs import Workload


def to_device(arr: np.ndarray, fmt: str, device="cuda") -> torch.Tensor:
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if fmt == "fp8":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)          # uint8 storage = E4M3FN
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


class HotPath:
    """Buffers and calls for one workload; ``step()`` runs the whole path once."""

    def __init__(self, wl: Workload, inp: Dict[str, np.ndarray], device="cuda", fused: bool = False):
        self.wl = wl
        self.device = device
        self.fused = fused
        dt = wl.dtype
        self.q = to_device(inp["q"], dt, device)
        self.pages = None
        if wl.page_size:
            # paged KV cache: pools of pages and the page table (the logical K/V are not uploaded)
            self.k = to_device(inp["k_pages"], dt, device)
            self.v = to_device(inp["v_pages"], dt, device)
            self.page_table = torch.from_numpy(inp["page_table"].astype(np.int32)).to(device)
            self.pages = S.kv_pages(self.page_table, wl.page_size)
        else:
            self.k = to_device(inp["k"], dt, device)
            self.v = to_device(inp["v"], dt, device)
        self.ctx_len = torch.from_numpy(inp["ctx_len"].astype(np.int32)).to(device)
        self.o = torch.empty(wl.B, wl.Hq, wl.Nq, wl.d, dtype=torch.float32, device=device)
        self.lse = torch.empty(wl.B, wl.Hq, wl.Nq, dtype=torch.float32, device=device)
        self.idx = None
        self.count = None
        if wl.H_I:
            self.q_idx = to_device(inp["q_idx"], wl.idx_q_dtype, device)
            self.k_idx = to_device(inp["k_idx"], wl.idx_k_dtype, device)
            w = torch.from_numpy(inp["w"].astype(np.float32)).to(device)
            self.w = w.view(1, 1, wl.H_I).expand(wl.B, wl.Nq, wl.H_I)
            mode = S.SCORE_WEIGHTED_RELU if wl.score_mode == "weighted_relu" else S.SCORE_DOT
            self.ix = S.indexer(self.q_idx, self.k_idx, self.w if mode == S.SCORE_WEIGHTED_RELU else None,
                                mode, wl.heads_per_group)
            # the score matrix of the separate indexer/top-K calls (block selection needs none)
            self.scores = None if wl.kind == "msa" else \
                torch.empty(wl.B, wl.G_sel, wl.Nq, wl.N, dtype=torch.float32, device=device)
            self.err = torch.empty(wl.B, wl.G_sel, wl.Nq, dtype=torch.float32, device=device)
            width = wl.top_pages + wl.n_local if wl.kind == "dsa_pages" else wl.topk
            self.idx = torch.empty(wl.B, wl.G_sel, wl.Nq, width, dtype=torch.int32, device=device)
            self.count = torch.empty(wl.B, wl.G_sel, wl.Nq, dtype=torch.int32, device=device)
            if wl.kind == "dsa_pages":
                self.sel = S.selection(S.SEL_PAGES, self.idx, block_size=wl.page_size)
            elif wl.kind == "msa":
                # one block list per KV group, read by every query head of the group
                self.idx = torch.empty(wl.B, wl.G_sel, wl.Nq, wl.top_blocks, dtype=torch.int32, device=device)
                self.sel = S.selection(S.SEL_BLOCKS, self.idx, window=wl.window, block_size=wl.block_size)
                self.fused = False
                self.k_blocks = torch.empty(wl.B, wl.N // wl.block_size, wl.G_k, wl.d_I, dtype=torch.float32,
                                            device=device)
                S.spattn_pool_index_keys(self.ix, self.ctx_len, wl.block_size, self.k_blocks)
            elif wl.kind == "dsa_two_level":
                self.sel = S.selection(S.SEL_INDEX, self.idx)
                self.fused = False
                # the block-key cache, formed once (a decode loop extends it a block at a time)
                self.k_blocks = torch.empty(wl.B, wl.N // wl.block_size, wl.G_k, wl.d_I, dtype=torch.float32,
                                            device=device)
                S.spattn_pool_index_keys(self.ix, self.ctx_len, wl.block_size, self.k_blocks)
            else:
                self.sel = S.selection(S.SEL_INDEX, self.idx)
                if self.fused and S.LIB.spattn_topk_workspace(None, S.ctypes.byref(self.ix), wl.topk,
                                                              S.TOPK_FUSED_INDEX) == S.SIZE_MAX:
                    self.fused = False      # this indexer shape has no fused kernel: separate calls
        elif wl.kind == "quest":
            width = wl.top_pages + wl.n_local
            self.idx = torch.empty(wl.B, wl.G_sel, wl.Nq, width, dtype=torch.int32, device=device)
            self.count = torch.empty(wl.B, wl.G_sel, wl.Nq, dtype=torch.int32, device=device)
            self.sel = S.selection(S.SEL_PAGES, self.idx, block_size=wl.page_size)
            # per-page key bounds, formed once (a decode loop refreshes a page's entry when it fills)
            self.bounds = torch.empty(wl.B, self.page_table.shape[1], wl.Hkv, 2 * wl.d, dtype=self.k.dtype,
                                      device=device)
            S.spattn_quest_page_bounds(self.k, self.pages, self.ctx_len, self.bounds)
        elif wl.kind in ("blocks", "nsa"):
            self.idx = torch.empty(wl.B, wl.Hq, wl.Nq, wl.top_blocks, dtype=torch.int32, device=device)
            self.count = torch.empty(wl.B, wl.Hq, wl.Nq, dtype=torch.int32, device=device)
            self.sel = S.selection(S.SEL_BLOCKS, self.idx, window=wl.window, block_size=wl.block_size)
            if wl.kind == "nsa":
                self.gates = torch.from_numpy(inp["gates"].astype(np.float32)).to(device)
        elif wl.kind == "window_global":
            self.sel = S.selection(S.SEL_WINDOW_GLOBAL, window=wl.window, n_global=wl.n_global, stride=wl.stride)
        else:
            self.sel = S.selection(S.SEL_DENSE)
        if wl.backward:
            self.d_o = torch.from_numpy(inp["d_o"].astype(np.float32)).to(device)
            self.dq = torch.empty_like(self.o)
            self.dk = torch.empty(self.k.shape, dtype=torch.float32, device=device)
            self.dv = torch.empty(self.v.shape, dtype=torch.float32, device=device)
        self.ws = torch.empty(self.ws_bytes(), dtype=torch.uint8, device=device)

    def ws_bytes(self) -> int:
        return max([v for v in self._ws_queries() if v != S.SIZE_MAX] + [16])

    def _ws_queries(self):
        q = []
        byref = S.ctypes.byref
        if self.wl.H_I:
            q.append(S.LIB.spattn_index_scores_workspace(byref(self.ix)))
            ts = S.tensor(self.scores)
            wl = self.wl
            if wl.kind == "msa":
                pass
            elif wl.kind == "dsa_pages":
                q.append(S.LIB.spattn_page_select_workspace(byref(ts), byref(self.ix), wl.page_size, wl.top_pages,
                                                            wl.n_local, S.TOPK_CERTIFIED))
                if self.fused:
                    q.append(S.LIB.spattn_page_select_workspace(None, byref(self.ix), wl.page_size, wl.top_pages,
                                                                wl.n_local, S.TOPK_FUSED_INDEX))
            else:
                q.append(S.LIB.spattn_topk_workspace(byref(ts), byref(self.ix), wl.topk, S.TOPK_CERTIFIED))
                if self.fused:
                    q.append(S.LIB.spattn_topk_workspace(None, byref(self.ix), wl.topk, S.TOPK_FUSED_INDEX))
        tq, tk = S.tensor(self.q), S.tensor(self.k)
        if self.wl.kind == "quest":
            q.append(S.LIB.spattn_quest_select_workspace(byref(tq), byref(S.tensor(self.bounds)), self.wl.page_size,
                                                         self.wl.top_pages, self.wl.n_local,
                                                         byref(S.tensor(self.idx))))
        if self.wl.kind in ("blocks", "nsa"):
            q.append(S.LIB.spattn_block_select_workspace(byref(tq), byref(tk), self.wl.block_size,
                                                         self.wl.top_blocks))
        if self.wl.backward:
            q.append(S.LIB.spattn_sparse_attn_bwd_workspace(byref(tq), byref(tk), byref(self.sel)))
        if self.wl.kind == "nsa":
            q.append(S.LIB.spattn_nsa_fwd_workspace(byref(tq), byref(tk), self.wl.block_size,
                                                    byref(S.tensor(self.idx)), self.wl.window))
        elif self.pages is not None:
            q.append(S.LIB.spattn_sparse_attn_fwd_paged_workspace(byref(tq), byref(tk), byref(self.pages),
                                                                  byref(self.sel)))
        else:
            q.append(S.LIB.spattn_sparse_attn_fwd_workspace(byref(tq), byref(tk), byref(self.sel)))
        return q

    # the individual stages
    def index_scores(self, stream=None):
        S.spattn_index_scores(self.ix, self.ctx_len, self.scores, self.err, self.ws, stream)

    def topk(self, stream=None):
        S.spattn_topk(self.scores, self.err, self.ix, self.ctx_len, self.wl.topk, S.TOPK_CERTIFIED,
                      self.idx, self.count, self.ws, stream)

    def topk_fused(self, stream=None):
        S.spattn_topk(None, None, self.ix, self.ctx_len, self.wl.topk, S.TOPK_FUSED_INDEX,
                      self.idx, self.count, self.ws, stream)

    def pool_blocks(self, stream=None):
        S.spattn_pool_index_keys(self.ix, self.ctx_len, self.wl.block_size, self.k_blocks, stream)

    def topk_two_level(self, stream=None):
        S.spattn_topk_two_level(self.ix, self.k_blocks, self.ctx_len, self.wl.block_size, self.wl.top_blocks,
                                self.wl.topk, self.idx, self.count, None, stream)

    def index_block_select(self, stream=None):
        S.spattn_index_block_select(self.ix, self.k_blocks, self.ctx_len, self.wl.block_size, self.wl.top_blocks,
                                    self.idx, self.count, stream)

    def page_select(self, stream=None):
        S.spattn_page_select(self.scores, self.err, self.ix, self.ctx_len, self.wl.page_size, self.wl.top_pages,
                             self.wl.n_local, S.TOPK_CERTIFIED, self.idx, self.count, self.ws, stream)

    def page_select_fused(self, stream=None):
        S.spattn_page_select(None, None, self.ix, self.ctx_len, self.wl.page_size, self.wl.top_pages,
                             self.wl.n_local, S.TOPK_FUSED_INDEX, self.idx, self.count, self.ws, stream)

    def quest_select(self, stream=None):
        S.spattn_quest_select(self.q, self.bounds, self.ctx_len, self.wl.page_size, self.wl.top_pages,
                              self.wl.n_local, self.idx, self.count, self.ws, stream)

    def block_select(self, stream=None):
        S.spattn_block_select(self.q, self.k, self.ctx_len, self.wl.block_size, self.wl.top_blocks,
                              self.idx, self.count, self.ws, stream)

    def attention(self, stream=None):
        if self.wl.kind == "nsa":
            S.spattn_nsa_fwd(self.q, self.k, self.v, self.ctx_len, 0.0, self.wl.block_size, self.idx, self.wl.window,
                             self.gates, self.o, self.ws, stream)
        elif self.pages is not None:
            S.spattn_sparse_attn_fwd_paged(self.q, self.k, self.v, self.pages, self.ctx_len, 0.0, self.sel, self.o,
                                           self.lse, self.ws, stream)
        else:
            S.spattn_sparse_attn_fwd(self.q, self.k, self.v, self.ctx_len, 0.0, self.sel, self.o, self.lse,
                                     self.ws, stream)

    def attention_bwd(self, stream=None):
        S.spattn_sparse_attn_bwd(self.q, self.k, self.v, self.ctx_len, 0.0, self.sel, self.o, self.lse, self.d_o,
                                 self.dq, self.dk, self.dv, self.ws, stream)

    def step(self, stream=None):
        if self.wl.H_I and self.fused and self.wl.kind == "dsa_pages":
            self.page_select_fused(stream)
        elif self.wl.H_I and self.fused:
            self.topk_fused(stream)
        elif self.wl.H_I and self.wl.kind == "dsa_two_level":
            self.topk_two_level(stream)
        elif self.wl.kind == "msa":
            self.index_block_select(stream)
        elif self.wl.H_I:
            self.index_scores(stream)
            if self.wl.kind == "dsa_pages":
                self.page_select(stream)
            else:
                self.topk(stream)
        elif self.wl.kind in ("blocks", "nsa"):
            self.block_select(stream)
        elif self.wl.kind == "quest":
            self.quest_select(stream)
        self.attention(stream)
        if self.wl.backward:
            self.attention_bwd(stream)
