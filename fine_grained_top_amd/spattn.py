"""Thin Python binding of libspattn (argument marshalling only).

Every function mirrors the C entry point of the same name in
``include/spattn.h``: torch tensors provide device pointers, shapes and
strides, and torch's current HIP stream is passed through. All computation
runs in the HIP kernels of ``libspattn.so``; if the library is missing the
import fails loudly instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspattn.so")

F32, BF16, FP8_E4M3, I32 = 0, 1, 2, 3
SCORE_DOT, SCORE_WEIGHTED_RELU = 0, 1
SEL_DENSE, SEL_INDEX, SEL_WINDOW_GLOBAL, SEL_BLOCKS, SEL_PAGES = 0, 1, 2, 3, 4
TOPK_CERTIFIED, TOPK_FUSED_INDEX = 1, 2

SIZE_MAX = ctypes.c_size_t(-1).value

STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "NO_DEVICE", 5: "LAUNCH"}


class SpattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libspattn {STATUS.get(status, status)}: {message}")
        self.status = status


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class Indexer(ctypes.Structure):
    _fields_ = [("q_idx", Tensor), ("k_idx", Tensor), ("w", Tensor),
                ("score_mode", ctypes.c_int32), ("heads_per_group", ctypes.c_int32)]


class Selection(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("idx", Tensor), ("window", ctypes.c_int32),
                ("n_global", ctypes.c_int32), ("block_size", ctypes.c_int32), ("stride", ctypes.c_int32)]


class KvPages(ctypes.Structure):
    _fields_ = [("page_table", Tensor), ("page_size", ctypes.c_int32)]


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_uint32
    sig = {
        "spattn_index_scores_workspace": (sz, [P(Indexer)]),
        "spattn_index_scores": (ctypes.c_int, [P(Indexer), vp, P(Tensor), vp, vp, sz, vp]),
        "spattn_topk_workspace": (sz, [P(Tensor), P(Indexer), i32, u32]),
        "spattn_topk": (ctypes.c_int, [P(Tensor), vp, P(Indexer), vp, i32, u32, P(Tensor), vp, vp, sz, vp]),
        "spattn_page_select_workspace": (sz, [P(Tensor), P(Indexer), i32, i32, i32, u32]),
        "spattn_page_select": (ctypes.c_int, [P(Tensor), vp, P(Indexer), vp, i32, i32, i32, u32, P(Tensor), vp,
                                              vp, sz, vp]),
        "spattn_pool_index_keys": (ctypes.c_int, [P(Indexer), vp, i32, P(Tensor), vp]),
        "spattn_topk_two_level_workspace": (sz, [P(Indexer), P(Tensor), i32, i32, i32]),
        "spattn_topk_two_level": (ctypes.c_int, [P(Indexer), P(Tensor), vp, i32, i32, i32, P(Tensor), vp, vp, sz,
                                                 vp]),
        "spattn_block_select_workspace": (sz, [P(Tensor), P(Tensor), i32, i32]),
        "spattn_block_select": (ctypes.c_int, [P(Tensor), P(Tensor), vp, i32, i32, P(Tensor), vp, vp, sz, vp]),
        "spattn_sparse_attn_fwd_workspace": (sz, [P(Tensor), P(Tensor), P(Selection)]),
        "spattn_sparse_attn_fwd": (ctypes.c_int, [P(Tensor), P(Tensor), P(Tensor), vp, ctypes.c_float,
                                                  P(Selection), P(Tensor), vp, vp, sz, vp]),
        "spattn_noalloc_scratch_bytes": (sz, []),
        "spattn_sparse_attn_fwd_noalloc": (ctypes.c_int, [P(Tensor), P(Tensor), P(Tensor), vp, ctypes.c_float,
                                                          P(Selection), P(Tensor), vp, vp]),
        "spattn_sparse_attn_fwd_paged_workspace": (sz, [P(Tensor), P(Tensor), P(KvPages), P(Selection)]),
        "spattn_sparse_attn_fwd_paged": (ctypes.c_int, [P(Tensor), P(Tensor), P(Tensor), P(KvPages), vp,
                                                        ctypes.c_float, P(Selection), P(Tensor), vp, vp, sz, vp]),
        "spattn_sparse_attn_bwd_workspace": (sz, [P(Tensor), P(Tensor), P(Selection)]),
        "spattn_sparse_attn_bwd": (ctypes.c_int, [P(Tensor), P(Tensor), P(Tensor), vp, ctypes.c_float, P(Selection),
                                                  P(Tensor), vp, P(Tensor), P(Tensor), P(Tensor), P(Tensor), vp, sz,
                                                  vp]),
        "spattn_nsa_fwd_workspace": (sz, [P(Tensor), P(Tensor), i32, P(Tensor), i32]),
        "spattn_nsa_fwd": (ctypes.c_int, [P(Tensor), P(Tensor), P(Tensor), vp, ctypes.c_float, i32, P(Tensor), i32,
                                          P(Tensor), P(Tensor), vp, sz, vp]),
        "spattn_index_block_select": (ctypes.c_int, [P(Indexer), P(Tensor), vp, i32, i32, P(Tensor), vp, vp]),
        "spattn_quest_page_bounds": (ctypes.c_int, [P(Tensor), P(KvPages), vp, P(Tensor), vp]),
        "spattn_quest_select_workspace": (sz, [P(Tensor), P(Tensor), i32, i32, i32, P(Tensor)]),
        "spattn_quest_select": (ctypes.c_int, [P(Tensor), P(Tensor), vp, i32, i32, i32, P(Tensor), vp, vp, sz,
                                               vp]),
        "spattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "spattn_version": (ctypes.c_char_p, []),
        "spattn_last_error_message": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()

_TORCH_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3,
             torch.uint8: FP8_E4M3, torch.int32: I32}


def tensor(t: Optional[torch.Tensor], dtype: Optional[int] = None) -> Tensor:
    """Describe a torch tensor (uint8 storage is read as fp8 E4M3FN)."""
    d = Tensor()
    if t is None:
        return d
    if t.dim() > 4:
        raise ValueError("at most 4 dims")
    d.data = t.data_ptr()
    d.dtype = _TORCH_DT[t.dtype] if dtype is None else dtype
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(rc: int) -> None:
    if rc != 0:
        raise SpattnError(rc, LIB.spattn_last_error_message().decode())


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is not None:
        return ws
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def indexer(q_idx: torch.Tensor, k_idx: torch.Tensor, w: Optional[torch.Tensor], score_mode: int,
            heads_per_group: int) -> Indexer:
    ix = Indexer()
    ix.q_idx = tensor(q_idx)
    ix.k_idx = tensor(k_idx)
    ix.w = tensor(w)
    ix.score_mode = score_mode
    ix.heads_per_group = heads_per_group
    ix._keep = (q_idx, k_idx, w)        # the struct holds raw pointers: keep the tensors alive with it
    return ix


def selection(mode: int, idx: Optional[torch.Tensor] = None, window: int = 0, n_global: int = 0,
              block_size: int = 0, stride: int = 0) -> Selection:
    s = Selection()
    s.mode = mode
    s.idx = tensor(idx)
    s.window = window
    s.n_global = n_global
    s.block_size = block_size
    s.stride = stride
    s._keep = idx
    return s


def kv_pages(page_table: torch.Tensor, page_size: int) -> KvPages:
    kp = KvPages()
    kp.page_table = tensor(page_table)
    kp.page_size = page_size
    kp._keep = page_table
    return kp


# ---------------------------------------------------------------- entry points
def spattn_index_scores(ix: Indexer, ctx_len: Optional[torch.Tensor], scores_out: torch.Tensor,
                        err_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    need = LIB.spattn_index_scores_workspace(ctypes.byref(ix))
    if need == ctypes.c_size_t(-1).value:
        raise SpattnError(1, LIB.spattn_last_error_message().decode())
    ws = _workspace(need, scores_out.device, ws)
    so = tensor(scores_out)
    _check(LIB.spattn_index_scores(ctypes.byref(ix), _ptr(ctx_len), ctypes.byref(so), _ptr(err_out),
                                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def spattn_topk(scores: Optional[torch.Tensor], err: Optional[torch.Tensor], ix: Optional[Indexer],
                ctx_len: Optional[torch.Tensor], k: int, flags: int, idx_out: torch.Tensor,
                count_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                stream=None) -> None:
    sc = tensor(scores) if scores is not None else None
    io = tensor(idx_out)
    ixp = ctypes.byref(ix) if ix is not None else None
    scp = ctypes.byref(sc) if sc is not None else None
    need = LIB.spattn_topk_workspace(scp, ixp, k, flags)
    ws = _workspace(need, idx_out.device, ws)
    _check(LIB.spattn_topk(scp, _ptr(err), ixp, _ptr(ctx_len), k, flags, ctypes.byref(io),
                           _ptr(count_out), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def spattn_page_select(scores: Optional[torch.Tensor], err: Optional[torch.Tensor], ix: Optional[Indexer],
                       ctx_len: Optional[torch.Tensor], page_size: int, top_pages: int, n_local: int, flags: int,
                       pg_idx_out: torch.Tensor, pg_count_out: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, stream=None) -> None:
    sc = tensor(scores) if scores is not None else None
    io = tensor(pg_idx_out)
    scp = ctypes.byref(sc) if sc is not None else None
    ixp = ctypes.byref(ix) if ix is not None else None
    need = LIB.spattn_page_select_workspace(scp, ixp, page_size, top_pages, n_local, flags)
    if need == SIZE_MAX:
        raise SpattnError(1, LIB.spattn_last_error_message().decode())
    ws = _workspace(need, pg_idx_out.device, ws)
    _check(LIB.spattn_page_select(scp, _ptr(err), ixp, _ptr(ctx_len), page_size, top_pages, n_local,
                                  flags, ctypes.byref(io), _ptr(pg_count_out), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)))


def spattn_quest_page_bounds(k_pool: torch.Tensor, pages: KvPages, ctx_len: Optional[torch.Tensor],
                             bounds_out: torch.Tensor, stream=None) -> None:
    _check(LIB.spattn_quest_page_bounds(ctypes.byref(tensor(k_pool)), ctypes.byref(pages), _ptr(ctx_len),
                                        ctypes.byref(tensor(bounds_out)), _stream(stream)))


def spattn_quest_select(q: torch.Tensor, bounds: torch.Tensor, ctx_len: Optional[torch.Tensor], page_size: int,
                        top_pages: int, n_local: int, pg_idx_out: torch.Tensor,
                        pg_count_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    tq, tb, io = tensor(q), tensor(bounds), tensor(pg_idx_out)
    need = LIB.spattn_quest_select_workspace(ctypes.byref(tq), ctypes.byref(tb), page_size, top_pages, n_local,
                                             ctypes.byref(io))
    if need == SIZE_MAX:
        raise SpattnError(1, LIB.spattn_last_error_message().decode())
    ws = _workspace(need, q.device, ws)
    _check(LIB.spattn_quest_select(ctypes.byref(tq), ctypes.byref(tb), _ptr(ctx_len), page_size, top_pages, n_local,
                                   ctypes.byref(io), _ptr(pg_count_out), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(stream)))


def spattn_pool_index_keys(ix: Indexer, ctx_len: Optional[torch.Tensor], block_size: int,
                           k_blocks_out: torch.Tensor, stream=None) -> None:
    _check(LIB.spattn_pool_index_keys(ctypes.byref(ix), _ptr(ctx_len), block_size, ctypes.byref(tensor(k_blocks_out)),
                                      _stream(stream)))


def spattn_topk_two_level(ix: Indexer, k_blocks: torch.Tensor, ctx_len: Optional[torch.Tensor], block_size: int,
                          top_blocks: int, k: int, idx_out: torch.Tensor, count_out: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None, stream=None) -> None:
    tb, io = tensor(k_blocks), tensor(idx_out)
    _check(LIB.spattn_topk_two_level(ctypes.byref(ix), ctypes.byref(tb), _ptr(ctx_len), block_size, top_blocks, k,
                                     ctypes.byref(io), _ptr(count_out), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(stream)))


def spattn_index_block_select(ix: Indexer, k_blocks: torch.Tensor, ctx_len: Optional[torch.Tensor], block_size: int,
                              top_blocks: int, blk_idx_out: torch.Tensor, blk_count_out: Optional[torch.Tensor] = None,
                              stream=None) -> None:
    _check(LIB.spattn_index_block_select(ctypes.byref(ix), ctypes.byref(tensor(k_blocks)), _ptr(ctx_len), block_size,
                                         top_blocks, ctypes.byref(tensor(blk_idx_out)), _ptr(blk_count_out),
                                         _stream(stream)))


def spattn_block_select(q: torch.Tensor, k: torch.Tensor, ctx_len: Optional[torch.Tensor], block_size: int,
                        top_blocks: int, blk_idx_out: torch.Tensor, blk_count_out: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None) -> None:
    tq, tk, to = tensor(q), tensor(k), tensor(blk_idx_out)
    need = LIB.spattn_block_select_workspace(ctypes.byref(tq), ctypes.byref(tk), block_size, top_blocks)
    if need == ctypes.c_size_t(-1).value:
        raise SpattnError(1, LIB.spattn_last_error_message().decode())
    ws = _workspace(need, q.device, ws)
    _check(LIB.spattn_block_select(ctypes.byref(tq), ctypes.byref(tk), _ptr(ctx_len), block_size, top_blocks,
                                   ctypes.byref(to), _ptr(blk_count_out), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)))


def spattn_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ctx_len: Optional[torch.Tensor],
                           scale: float, sel: Selection, o_out: torch.Tensor,
                           lse_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                           stream=None) -> None:
    tq, tk, tv, to = tensor(q), tensor(k), tensor(v), tensor(o_out)
    need = LIB.spattn_sparse_attn_fwd_workspace(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(sel))
    if need == ctypes.c_size_t(-1).value:
        raise SpattnError(1, LIB.spattn_last_error_message().decode())
    ws = _workspace(need, q.device, ws)
    _check(LIB.spattn_sparse_attn_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), _ptr(ctx_len),
                                      scale, ctypes.byref(sel), ctypes.byref(to), _ptr(lse_out), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(stream)))


def spattn_sparse_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   ctx_len: Optional[torch.Tensor], scale: float, sel: Selection,
                                   o_out: torch.Tensor, lse_out: Optional[torch.Tensor] = None,
                                   stream=None) -> None:
    tq, tk, tv, to = tensor(q), tensor(k), tensor(v), tensor(o_out)
    _check(LIB.spattn_sparse_attn_fwd_noalloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), _ptr(ctx_len),
                                              scale, ctypes.byref(sel), ctypes.byref(to), _ptr(lse_out),
                                              _stream(stream)))


def spattn_sparse_attn_fwd_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, pages: KvPages,
                                 ctx_len: Optional[torch.Tensor], scale: float, sel: Selection,
                                 o_out: torch.Tensor, lse_out: Optional[torch.Tensor] = None,
                                 ws: Optional[torch.Tensor] = None, stream=None) -> None:
    tq, tk, tv, to = tensor(q), tensor(k_pool), tensor(v_pool), tensor(o_out)
    need = LIB.spattn_sparse_attn_fwd_paged_workspace(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(pages),
                                                      ctypes.byref(sel))
    if need == SIZE_MAX:
        raise SpattnError(1, LIB.spattn_last_error_message().decode())
    ws = _workspace(need, q.device, ws)
    _check(LIB.spattn_sparse_attn_fwd_paged(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                            ctypes.byref(pages), _ptr(ctx_len), scale, ctypes.byref(sel),
                                            ctypes.byref(to), _ptr(lse_out), _ptr(ws),
                                            0 if ws is None else ws.numel(), _stream(stream)))


def spattn_sparse_attn_bwd_workspace(q: torch.Tensor, k: torch.Tensor, sel: Selection) -> int:
    tq, tk = tensor(q), tensor(k)
    return int(LIB.spattn_sparse_attn_bwd_workspace(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(sel)))


def spattn_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ctx_len: Optional[torch.Tensor],
                           scale: float, sel: Selection, o: torch.Tensor, lse: torch.Tensor, d_o: torch.Tensor,
                           dq_out: torch.Tensor, dk_out: torch.Tensor, dv_out: torch.Tensor,
                           ws: Optional[torch.Tensor] = None, stream=None) -> None:
    t = [tensor(x) for x in (q, k, v, o, d_o, dq_out, dk_out, dv_out)]
    _check(LIB.spattn_sparse_attn_bwd(ctypes.byref(t[0]), ctypes.byref(t[1]), ctypes.byref(t[2]), _ptr(ctx_len), scale,
                                      ctypes.byref(sel), ctypes.byref(t[3]), _ptr(lse), ctypes.byref(t[4]),
                                      ctypes.byref(t[5]), ctypes.byref(t[6]), ctypes.byref(t[7]), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(stream)))


def spattn_nsa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ctx_len: Optional[torch.Tensor], scale: float,
                   block_size: int, blk_idx: torch.Tensor, window: int, gates: torch.Tensor, o_out: torch.Tensor,
                   ws: Optional[torch.Tensor] = None, stream=None) -> None:
    tq, tk, tv, tb, tg, to = tensor(q), tensor(k), tensor(v), tensor(blk_idx), tensor(gates), tensor(o_out)
    need = LIB.spattn_nsa_fwd_workspace(ctypes.byref(tq), ctypes.byref(tk), block_size, ctypes.byref(tb), window)
    if need == SIZE_MAX:
        raise SpattnError(1, LIB.spattn_last_error_message().decode())
    ws = _workspace(need, q.device, ws)
    _check(LIB.spattn_nsa_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), _ptr(ctx_len), scale, block_size,
                              ctypes.byref(tb), window, ctypes.byref(tg), ctypes.byref(to), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream)))


def spattn_version() -> str:
    return LIB.spattn_version().decode()


def spattn_status_string(status: int) -> str:
    return LIB.spattn_status_string(status).decode()


def spattn_last_error_message() -> str:
    return LIB.spattn_last_error_message().decode()
