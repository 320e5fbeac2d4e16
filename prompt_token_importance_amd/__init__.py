"""Python binding of libkvs (attention-based prompt-token importance on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libkvs.so``; this module passes device pointers, sizes and the current HIP
stream through the C ABI declared in ``include/kvs.h`` and allocates output and
workspace tensors with PyTorch when the caller does not pass them.  There is no
CPU fallback: importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # loaded first so libkvs binds to the same HIP runtime as torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvs.so")

KVS_OK, KVS_EINVAL, KVS_EUNSUPPORTED, KVS_EWORKSPACE, KVS_EHIP, KVS_ESCRATCH = 0, -1, -2, -3, -4, -5
HEADS_NONE, HEADS_GROUP_SUM, HEADS_GROUP_MAX, HEADS_ALL_SUM = 0, 1, 2, 3
ACC_WRITE, ACC_ADD, ACC_MAX = 0, 1, 2
RED_NONE, RED_SUM, RED_MAX, RED_MEAN, RED_SUM_L1 = 0, 1, 2, 3, 4


class KvsError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_lib.kvs_status_string(status).decode()} ({status})")
        self.status = status


class ScoreArgs(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32), ("W", ctypes.c_int32), ("d_k", ctypes.c_int32),
        ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("q_pos0", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64), ("q_row_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64), ("k_tok_stride", ctypes.c_int64),
        ("s_ld", ctypes.c_int64),
        ("scale", ctypes.c_float), ("accumulate", ctypes.c_int32), ("phase", ctypes.c_int32),
    ]


class RawArgs(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32), ("W", ctypes.c_int32), ("d_k", ctypes.c_int32),
        ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("reduce", ctypes.c_int32),
        ("q_pos0", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64), ("q_row_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64), ("k_tok_stride", ctypes.c_int64),
        ("s_ld", ctypes.c_int64),
        ("scale", ctypes.c_float), ("accumulate", ctypes.c_int32),
    ]


class DeltaArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("d_k", ctypes.c_int32), ("H_q", ctypes.c_int32),
        ("H_kv", ctypes.c_int32), ("P", ctypes.c_int32), ("K_pages", ctypes.c_int32),
        ("L_recent", ctypes.c_int32), ("L_max", ctypes.c_int32),
        ("k_head_stride", ctypes.c_int64), ("k_tok_stride", ctypes.c_int64),
        ("scale", ctypes.c_float),
    ]


class BlockSelectArgs(ctypes.Structure):
    _fields_ = [
        ("Lq", ctypes.c_int32), ("L", ctypes.c_int32), ("d_k", ctypes.c_int32),
        ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("block", ctypes.c_int32),
        ("q_pos0", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64), ("q_row_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64), ("k_tok_stride", ctypes.c_int64),
        ("scale", ctypes.c_float), ("p_mass", ctypes.c_float),
    ]


class SelectArgs(ctypes.Structure):
    _fields_ = [
        ("budget", ctypes.c_int32), ("n_forced", ctypes.c_int32), ("pool", ctypes.c_int32),
        ("pool_k", ctypes.c_int32), ("cluster_P", ctypes.c_int32),
        ("cluster_theta", ctypes.c_float), ("cluster_r", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python prompt_token_importance_amd/build.py`"
            " (hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "kvs_status_string": (ctypes.c_char_p, [I32]),
        "kvs_version": (I32, []),
        "kvs_score_workspace": (SZ, [ctypes.POINTER(ScoreArgs)]),
        "kvs_score": (I32, [ctypes.POINTER(ScoreArgs), P, P, P, P, SZ, P]),
        "kvs_score_noalloc": (I32, [ctypes.POINTER(ScoreArgs), P, P, P, P]),
        "kvs_wait_limit": (I32, [I32]),
        "kvs_score_raw": (I32, [ctypes.POINTER(RawArgs), P, P, P, P]),
        "kvs_delta_workspace": (SZ, [ctypes.POINTER(DeltaArgs)]),
        "kvs_gather_kv": (I32, [P, P, I32, I32, I32, I64, I64, P, I64, P, I32, I32, P, P, P]),
        "kvs_delta_pages": (I32, [ctypes.POINTER(DeltaArgs), P, P, P, P, P, P, SZ, P]),
        "kvs_pool_pages": (I32, [P, I32, I32, I64, I32, I32, I32, I32, I32, P, P, P, P]),
        "kvs_topk_workspace": (SZ, [I32, I32, I32]),
        "kvs_topk": (I32, [P, I32, I32, I64, I32, P, I32, P, P, P, SZ, P]),
        "kvs_select_workspace": (SZ, [I32, I32, I32]),
        "kvs_select": (I32, [P, I32, I32, I64, ctypes.POINTER(SelectArgs), P, P, SZ, P]),
        "kvs_block_union_workspace": (SZ, [I32, I32, I32, I32]),
        "kvs_block_union_pagetable": (I32, [P, I32, I32, I32, I32, I32, P, P, P, SZ, P]),
        "kvs_token_pagetable_workspace": (SZ, [I32, I32, I32]),
        "kvs_token_pagetable": (I32, [P, I32, I32, I64, I32, I32, I32, P, P, P, SZ, P]),
        "kvs_aggregate_workspace": (SZ, [I32]),
        "kvs_aggregate_layers": (I32, [P, P, I32, I32, I64, I32, I32, P, SZ, P]),
        "kvs_cluster_priority": (I32, [P, P, I32, I32, I32, I32, F32, I32, P, P]),
        "kvs_block_select_workspace": (SZ, [ctypes.POINTER(BlockSelectArgs)]),
        "kvs_block_select": (I32, [ctypes.POINTER(BlockSelectArgs), P, P, P, P, SZ, P]),
        "kvs_block_select_cached": (I32, [ctypes.POINTER(BlockSelectArgs), P, P, P, I32, I32, P, P,
                                          SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTED = (
    "kvs_status_string", "kvs_version", "kvs_score_workspace", "kvs_score", "kvs_score_noalloc",
    "kvs_wait_limit",
    "kvs_score_raw",
    "kvs_delta_workspace", "kvs_delta_pages", "kvs_gather_kv",
    "kvs_pool_pages",
    "kvs_topk_workspace", "kvs_topk", "kvs_select_workspace", "kvs_select",
    "kvs_block_union_workspace", "kvs_block_union_pagetable",
    "kvs_token_pagetable_workspace", "kvs_token_pagetable",
    "kvs_aggregate_workspace", "kvs_aggregate_layers", "kvs_cluster_priority",
    "kvs_block_select_workspace", "kvs_block_select", "kvs_block_select_cached",
)


def library() -> ctypes.CDLL:
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st: int, what: str):
    if st != KVS_OK:
        raise KvsError(st, what)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def bf16_from_bits(bits, device="cuda") -> torch.Tensor:
    """uint16 bfloat16 bit patterns (NumPy) -> torch.bfloat16 tensor on device."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


# --------------------------------------------------------------------------- score
def score_args(*, L, W, d_k, H_q, H_kv, q_pos0, heads=HEADS_GROUP_SUM, scale=0.0, accumulate=False,
               q_head_stride=0, q_row_stride=0, k_head_stride=0, k_tok_stride=0, s_ld=0,
               phase=0) -> ScoreArgs:
    return ScoreArgs(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, heads=heads, q_pos0=q_pos0,
                     q_head_stride=q_head_stride, q_row_stride=q_row_stride,
                     k_head_stride=k_head_stride, k_tok_stride=k_tok_stride, s_ld=s_ld,
                     scale=scale, accumulate=int(bool(accumulate)), phase=phase)


def kvs_score_workspace(args: ScoreArgs) -> int:
    return int(_lib.kvs_score_workspace(ctypes.byref(args)))


def kvs_score(Q: torch.Tensor, K: torch.Tensor, args: ScoreArgs, S: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Window column scores; S float32 [H_kv, H_q or 1][s_ld] (allocated if None)."""
    rows = {HEADS_NONE: args.H_q, HEADS_ALL_SUM: 1}.get(args.heads, args.H_kv)
    if S is None:
        S = torch.empty(rows, args.s_ld or args.L, dtype=torch.float32, device=K.device)
    ws, nb = _workspace(kvs_score_workspace(args), K.device, ws)
    _check(_lib.kvs_score(ctypes.byref(args), _ptr(Q), _ptr(K), _ptr(S), _ptr(ws), nb,
                          _stream(stream)), "kvs_score")
    return S


def kvs_wait_limit(microseconds: int) -> int:
    """Sets the one-launch forms' wait bound (< 0: query only); returns the previous."""
    return int(_lib.kvs_wait_limit(int(microseconds)))


def kvs_score_noalloc(Q: torch.Tensor, K: torch.Tensor, args: ScoreArgs,
                      S: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvs_score with the library's static scratch instead of a workspace."""
    rows = {HEADS_NONE: args.H_q, HEADS_ALL_SUM: 1}.get(args.heads, args.H_kv)
    if S is None:
        S = torch.empty(rows, args.s_ld or args.L, dtype=torch.float32, device=K.device)
    _check(_lib.kvs_score_noalloc(ctypes.byref(args), _ptr(Q), _ptr(K), _ptr(S), _stream(stream)),
           "kvs_score_noalloc")
    return S


# --------------------------------------------------------------------------- raw logits
def raw_args(*, L, W, d_k, H_q, H_kv, q_pos0, reduce=RED_SUM, scale=0.0, accumulate=ACC_WRITE,
             q_head_stride=0, q_row_stride=0, k_head_stride=0, k_tok_stride=0, s_ld=0) -> RawArgs:
    return RawArgs(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, reduce=reduce, q_pos0=q_pos0,
                   q_head_stride=q_head_stride, q_row_stride=q_row_stride,
                   k_head_stride=k_head_stride, k_tok_stride=k_tok_stride, s_ld=s_ld,
                   scale=scale, accumulate=accumulate)


def kvs_score_raw(Q: torch.Tensor, K: torch.Tensor, args: RawArgs, S: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Raw logits reduced over all heads; S float32 [W][s_ld] (allocated if None)."""
    if S is None:
        S = torch.empty(args.W, args.s_ld or args.L, dtype=torch.float32, device=K.device)
    _check(_lib.kvs_score_raw(ctypes.byref(args), _ptr(Q), _ptr(K), _ptr(S), _stream(stream)),
           "kvs_score_raw")
    return S


# --------------------------------------------------------------------------- DELTA page sets
def delta_args(*, B, d_k, H_q, H_kv, L_max, P=16, K_pages=64, L_recent=8, k_head_stride=0,
               k_tok_stride=0, scale=0.0) -> DeltaArgs:
    return DeltaArgs(B=B, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P, K_pages=K_pages, L_recent=L_recent,
                     L_max=L_max, k_head_stride=k_head_stride, k_tok_stride=k_tok_stride,
                     scale=scale)


def kvs_delta_workspace(args: DeltaArgs) -> int:
    return int(_lib.kvs_delta_workspace(ctypes.byref(args)))


def kvs_delta_pages(Q: torch.Tensor, K_ptrs: torch.Tensor, L: torch.Tensor, args: DeltaArgs,
                    rho: Optional[torch.Tensor] = None, page_scores: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rho int32 [B][K_pages].  K_ptrs: int64 device tensor [B] of bf16 K base
    addresses; L: int32 device tensor [B] of context lengths."""
    if rho is None:
        rho = torch.empty(args.B, args.K_pages, dtype=torch.int32, device=Q.device)
    ws, nb = _workspace(kvs_delta_workspace(args), Q.device, ws)
    _check(_lib.kvs_delta_pages(ctypes.byref(args), _ptr(Q), _ptr(K_ptrs), _ptr(L), _ptr(rho),
                                _ptr(page_scores), _ptr(ws), nb, _stream(stream)), "kvs_delta_pages")
    return rho


# --------------------------------------------------------------------------- KV gather
def kvs_gather_kv(K: torch.Tensor, indices: torch.Tensor, n: int, *, V: Optional[torch.Tensor] = None,
                  unit: int = 1, idx_ld: int = 0, indptr: Optional[torch.Tensor] = None,
                  L: Optional[int] = None, H: Optional[int] = None, head_stride: int = 0,
                  tok_stride: int = 0, K_out: Optional[torch.Tensor] = None,
                  V_out: Optional[torch.Tensor] = None, stream=None):
    """Returns (K_out, V_out or None), each [H][n * unit][d_k].  K: [H][L][d_k]
    unless strides are given (then pass H and L)."""
    d_k = K.shape[-1]
    H = K.shape[0] if H is None else H
    L = K.shape[1] if L is None else L
    if K_out is None:
        K_out = torch.empty(H, n * unit, d_k, dtype=K.dtype, device=K.device)
    if V is not None and V_out is None:
        V_out = torch.empty(H, n * unit, d_k, dtype=V.dtype, device=V.device)
    _check(_lib.kvs_gather_kv(_ptr(K), _ptr(V), H, L, d_k, head_stride, tok_stride, _ptr(indices),
                              idx_ld, _ptr(indptr), n, unit, _ptr(K_out), _ptr(V_out),
                              _stream(stream)), "kvs_gather_kv")
    return K_out, V_out


# --------------------------------------------------------------------------- pool / pages
def kvs_pool_pages(S: torch.Tensor, n: int, *, head_reduce=RED_NONE, pool=RED_NONE, pool_k=7, P=0,
                   page_reduce=RED_SUM, ld: Optional[int] = None, want_pooled=True,
                   out: Optional[torch.Tensor] = None, stream=None):
    """Returns (pooled or None, page or None, page_arg or None); `out` (contiguous
    float32, rows x n) receives the pooled rows when given."""
    H = S.shape[0]
    ld = S.stride(0) if ld is None else ld
    rows = H if head_reduce == RED_NONE else 1
    pooled = out
    if pooled is None and (want_pooled or P == 0):
        pooled = torch.empty(rows, n, dtype=torch.float32, device=S.device)
    page = arg = None
    if P > 0:
        n_pages = (n + P - 1) // P
        page = torch.empty(rows, n_pages, dtype=torch.float32, device=S.device)
        arg = torch.empty(rows, n_pages, dtype=torch.int32, device=S.device)
    _check(_lib.kvs_pool_pages(_ptr(S), H, n, ld, head_reduce, pool, pool_k, P, page_reduce,
                               _ptr(pooled), _ptr(page), _ptr(arg), _stream(stream)), "kvs_pool_pages")
    return pooled, page, arg


# --------------------------------------------------------------------------- top-k
def kvs_topk(S: torch.Tensor, n: int, budget: int, *, priority: Optional[torch.Tensor] = None,
             n_forced: int = 0, ld: Optional[int] = None, idx: Optional[torch.Tensor] = None,
             val: Optional[torch.Tensor] = None, want_val: bool = False,
             ws: Optional[torch.Tensor] = None, stream=None):
    """int32 [H][budget + n_forced]: chosen indices ascending, then n .. n + n_forced - 1.

    With ``want_val`` (or a ``val`` tensor) also returns the kept scores, float32
    [H][budget + n_forced] in the order of the indices (NaN for the forced suffix):
    ``(idx, val)``."""
    H = S.shape[0]
    ld = S.stride(0) if ld is None else ld
    if idx is None:
        idx = torch.empty(H, budget + n_forced, dtype=torch.int32, device=S.device)
    if want_val and val is None:
        val = torch.empty(H, budget + n_forced, dtype=torch.float32, device=S.device)
    ws, nb = _workspace(int(_lib.kvs_topk_workspace(H, n, budget)), S.device, ws)
    _check(_lib.kvs_topk(_ptr(S), H, n, ld, budget, _ptr(priority), n_forced, _ptr(idx), _ptr(val),
                         _ptr(ws), nb, _stream(stream)), "kvs_topk")
    return (idx, val) if val is not None else idx


def select_args(*, budget, n_forced=0, pool=RED_NONE, pool_k=7, cluster_P=0, cluster_theta=0.0,
                cluster_r=0) -> SelectArgs:
    return SelectArgs(budget=budget, n_forced=n_forced, pool=pool, pool_k=pool_k,
                      cluster_P=cluster_P, cluster_theta=cluster_theta, cluster_r=cluster_r)


def kvs_select(S: torch.Tensor, n: int, args: SelectArgs, *, ld: Optional[int] = None,
               idx: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Pooled or cluster-prioritised top-k (same output as kvs_topk)."""
    H = S.shape[0]
    ld = S.stride(0) if ld is None else ld
    if idx is None:
        idx = torch.empty(H, args.budget + args.n_forced, dtype=torch.int32, device=S.device)
    ws, nb = _workspace(int(_lib.kvs_select_workspace(H, n, args.budget)), S.device, ws)
    _check(_lib.kvs_select(_ptr(S), H, n, ld, ctypes.byref(args), _ptr(idx), _ptr(ws), nb,
                           _stream(stream)), "kvs_select")
    return idx


# --------------------------------------------------------------------------- union
def kvs_block_union_pagetable(M: torch.Tensor, H_q: int, H_kv: int, sub_group: int = 0,
                              ws: Optional[torch.Tensor] = None, stream=None):
    """M uint8 [H_q][n_qb][n_kvb] -> (kv_indptr int32 [n_groups+1], kv_indices int32 [cap])."""
    _, n_qb, n_kvb = M.shape
    sg = (H_q // H_kv) if sub_group == 0 else sub_group
    n_groups = H_q // sg
    indptr = torch.empty(n_groups + 1, dtype=torch.int32, device=M.device)
    indices = torch.empty(n_groups * n_kvb, dtype=torch.int32, device=M.device)
    ws, nb = _workspace(int(_lib.kvs_block_union_workspace(H_q, H_kv, sub_group, n_kvb)), M.device, ws)
    _check(_lib.kvs_block_union_pagetable(_ptr(M), H_q, H_kv, sub_group, n_qb, n_kvb, _ptr(indptr),
                                          _ptr(indices), _ptr(ws), nb, _stream(stream)),
           "kvs_block_union_pagetable")
    return indptr, indices


# --------------------------------------------------------------------------- token page tables
def kvs_token_pagetable(idx: torch.Tensor, P: int, n_pages: int, rows_per_group: int = 1,
                        n: Optional[int] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """idx int32 [H][>= n] kept token positions -> (kv_indptr int32 [n_groups+1],
    kv_indices int32 [n_groups * n_pages]) of the pages they fall in, per group of rows."""
    H = idx.shape[0]
    n = idx.shape[1] if n is None else n
    n_groups = H // rows_per_group
    indptr = torch.empty(n_groups + 1, dtype=torch.int32, device=idx.device)
    indices = torch.empty(n_groups * n_pages, dtype=torch.int32, device=idx.device)
    ws, nb = _workspace(int(_lib.kvs_token_pagetable_workspace(H, rows_per_group, n_pages)),
                        idx.device, ws)
    _check(_lib.kvs_token_pagetable(_ptr(idx), H, n, idx.stride(0), rows_per_group, P, n_pages,
                                    _ptr(indptr), _ptr(indices), _ptr(ws), nb, _stream(stream)),
           "kvs_token_pagetable")
    return indptr, indices


# --------------------------------------------------------------------------- layers
def kvs_aggregate_layers(acc: torch.Tensor, S: torch.Tensor, n: int, mode: int, first_layer: bool,
                         ld: Optional[int] = None, ws: Optional[torch.Tensor] = None, stream=None):
    H = S.shape[0]
    ld = S.stride(0) if ld is None else ld
    ws, nb = _workspace(int(_lib.kvs_aggregate_workspace(n)), S.device, ws)
    _check(_lib.kvs_aggregate_layers(_ptr(acc), _ptr(S), H, n, ld, mode, int(bool(first_layer)),
                                     _ptr(ws), nb, _stream(stream)), "kvs_aggregate_layers")
    return acc


# --------------------------------------------------------------------------- clusters
def kvs_cluster_priority(page: torch.Tensor, page_arg: torch.Tensor, P: int, n: int, theta: float,
                         r: int, priority: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    H, n_pages = page.shape
    if priority is None:
        priority = torch.empty(H, n, dtype=torch.uint8, device=page.device)
    _check(_lib.kvs_cluster_priority(_ptr(page), _ptr(page_arg), H, n_pages, P, n, theta, r,
                                     _ptr(priority), _stream(stream)), "kvs_cluster_priority")
    return priority


# --------------------------------------------------------------------------- block select
def block_select_args(*, Lq, L, d_k, H_q, H_kv, q_pos0, block=64, p_mass=0.9, scale=0.0,
                      q_head_stride=0, q_row_stride=0, k_head_stride=0, k_tok_stride=0) -> BlockSelectArgs:
    return BlockSelectArgs(Lq=Lq, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, block=block, q_pos0=q_pos0,
                           q_head_stride=q_head_stride, q_row_stride=q_row_stride,
                           k_head_stride=k_head_stride, k_tok_stride=k_tok_stride,
                           scale=scale, p_mass=p_mass)


def kvs_block_select_workspace(args: BlockSelectArgs) -> int:
    return int(_lib.kvs_block_select_workspace(ctypes.byref(args)))


def kvs_block_select(Qc: torch.Tensor, K: torch.Tensor, args: BlockSelectArgs,
                     M: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    n_qb = (args.Lq + args.block - 1) // args.block
    n_kvb = (args.L + args.block - 1) // args.block
    if M is None:
        M = torch.empty(args.H_q, n_qb, n_kvb, dtype=torch.uint8, device=K.device)
    ws, nb = _workspace(kvs_block_select_workspace(args), K.device, ws)
    _check(_lib.kvs_block_select(ctypes.byref(args), _ptr(Qc), _ptr(K), _ptr(M), _ptr(ws), nb,
                                 _stream(stream)), "kvs_block_select")
    return M


def kvs_block_select_cached(Qc: torch.Tensor, K: torch.Tensor, args: BlockSelectArgs,
                            Kb: torch.Tensor, n_cached: int, M: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvs_block_select with the key-block means cached in Kb float32
    [H_kv][kb_cap][d_k]; the first n_cached blocks must already be valid."""
    n_qb = (args.Lq + args.block - 1) // args.block
    n_kvb = (args.L + args.block - 1) // args.block
    if M is None:
        M = torch.empty(args.H_q, n_qb, n_kvb, dtype=torch.uint8, device=K.device)
    ws, nb = _workspace(kvs_block_select_workspace(args), K.device, ws)
    _check(_lib.kvs_block_select_cached(ctypes.byref(args), _ptr(Qc), _ptr(K), _ptr(Kb), Kb.shape[1],
                                        n_cached, _ptr(M), _ptr(ws), nb, _stream(stream)),
           "kvs_block_select_cached")
    return M
