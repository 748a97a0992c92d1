"""Python binding of libidx.so, the MI355X block-scoring + top-K indexer.

Argument marshalling only: every function here checks tensor placement and
layout, passes raw device pointers and the current HIP stream to the C ABI
(include/idx.h) and returns the output tensors. All arithmetic runs in the HIP
kernels; there is no fallback path. PyTorch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["idx_score", "idx_topk", "idx_topk_bf16", "idx_select", "idx_select_noalloc", "idx_select_paged", "idx_select_prefill",
           "idx_prefill_workspace_bytes", "idx_pool_keys", "idx_assign", "idx_workspace_bytes",
           "idx_topk_workspace_bytes", "idx_assign_workspace_bytes", "idx_status_string",
           "idx_floor_empty", "idx_floor_read", "idx_floor_mfma", "lib_path", "load", "IDX_SORTED", "IDX_RADIX8",
           "IdxError",
           "SelectPlan", "plan_for"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libidx.so")

IDX_F32, IDX_BF16 = 0, 1
IDX_SORTED = 0x1
IDX_RADIX8 = 0x2  # four 8-bit radix passes, no linear-bin pass (same results)
IDX_CHUNK_SHIFT = 8

_c_int, _c_size, _vp, _u32 = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32
_SIGS = {
    "idx_score": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "idx_topk_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _u32]),
    "idx_topk": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _u32, _vp, _c_size, _vp]),
    "idx_topk_bf16": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _u32, _vp, _c_size,
                               _vp]),
    "idx_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _u32]),
    "idx_select": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                            _c_int, _c_int, _u32, _vp, _c_size, _vp]),
    "idx_select_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _u32, _vp]),
    "idx_select_paged": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                  _c_int, ctypes.c_int64, _c_int, _c_int, _c_int, _u32, _vp,
                                  _c_size, _vp]),
    "idx_pool_keys": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                               _vp]),
    "idx_prefill_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _u32]),
    "idx_select_prefill": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _u32, _vp, _c_size, _vp]),
    "idx_assign_workspace_bytes": (_c_size, [_c_int, _c_int]),
    "idx_assign": (_c_int, [_vp, _vp, _vp, _vp, ctypes.c_int64, _c_int, _c_int, _c_int, _vp,
                            _c_size, _vp]),
    "idx_status_string": (ctypes.c_char_p, [_c_int]),
    "idx_plan_create": (_c_int, [ctypes.POINTER(_vp), _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _u32]),
    "idx_plan_workspace_bytes": (_c_size, [_vp]),
    "idx_plan_select": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "idx_plan_destroy": (None, [_vp]),
    "idx_floor_empty": (_c_int, [_c_int, _vp]),
    "idx_floor_read": (_c_int, [_vp, _c_size, _vp, _vp, _c_int, _c_int, _vp]),
    "idx_floor_mfma": (_c_int, [_vp, _c_int, _c_int, _vp, _vp]),
}

_lib = None
_lock = threading.Lock()


class IdxError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {idx_status_string(status)} ({status})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libidx.so (once). Raises if it has not been built: there is no fallback."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(f"{_LIB_PATH} is missing; build it with "
                                   "`python -m block_scoring_top_amd.build`")
            lib = ctypes.CDLL(_LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(lib, name)
                fn.restype, fn.argtypes = res, args
            _lib = lib
    return _lib


def idx_status_string(status: int) -> str:
    return load().idx_status_string(status).decode()


def _ptr(t):
    # a plain int: ctypes converts it for the c_void_p arguments
    return None if t is None else t.data_ptr()


# torch's raw accessor for the current stream handle costs a tenth of building
# the Stream object (about 0.2 against 2 us a call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    """The current stream's handle on `device` (a torch.device or an index)."""
    if _raw_stream is not None:
        if isinstance(device, int):
            index = device
        else:
            index = device.index if device.index is not None else torch.cuda.current_device()
        return _raw_stream(index)
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t):
    if t.dtype == torch.float32:
        return IDX_F32
    if t.dtype in (torch.bfloat16, torch.uint16, torch.int16):
        return IDX_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn, st):
    if st != 0:
        raise IdxError(fn, st)


def _dev(*ts):
    d = ts[0].device
    for t in ts:
        if t is not None:
            if not t.is_cuda or t.device != d:
                raise ValueError("all tensors must live on the same GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
    return d


# one zero-filled workspace per (entry point, device, stream); the indexer kernels
# leave theirs zeroed
_ws_cache: dict = {}


def _workspace(device, nbytes, kind):
    key = (kind, device.index, _stream(device))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            # a zero-filled allocation would be recorded into the graph (and its
            # fill replayed with it): pass ws= to calls that are captured
            raise RuntimeError(f"{kind}: no workspace for this stream while a graph is being "
                               "captured; pass ws= (a zero-filled buffer of the size "
                               "*_workspace_bytes returns)")
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def idx_workspace_bytes(B, N_pad, H, K, flags=0) -> int:
    return load().idx_workspace_bytes(B, N_pad, H, K, flags)


def idx_topk_workspace_bytes(B, N, K, flags=0) -> int:
    return load().idx_topk_workspace_bytes(B, N, K, flags)


def idx_assign_workspace_bytes(C, D) -> int:
    return load().idx_assign_workspace_bytes(C, D)


def idx_score(q, c, seq_len, page_size=16, scores=None):
    """scores[b,n] = sum_h q[b,h].c[b,n] for n < ceil(seq_len[b]/page_size), else -inf."""
    lib = load()
    dev = _dev(q, c, seq_len, scores)
    B, H, D = q.shape
    N_pad = c.shape[1]
    if scores is None:
        scores = torch.empty(B, N_pad, dtype=torch.float32, device=dev)
    _check("idx_score", lib.idx_score(_ptr(q), _ptr(c), _ptr(seq_len), _ptr(scores), B, H, D,
                                      N_pad, page_size, _dtype_code(q), _stream(dev)))
    return scores


def idx_topk(scores, K, n_valid=None, sorted=False, ids=None, counts=None, ws=None,
             radix8=False):
    """Row-wise top-K indices (ties to the lower index), padded with -1. float32
    scores go to idx_topk, bfloat16 ones to idx_topk_bf16. radix8: the select
    with four 8-bit radix passes (IDX_RADIX8; the same results)."""
    if scores.dtype == torch.bfloat16:
        return idx_topk_bf16(scores, K, n_valid, sorted, ids, counts, ws, radix8)
    lib = load()
    dev = _dev(scores, n_valid, ids, counts, ws)
    B, N = scores.shape
    if ids is None:
        ids = torch.empty(B, K, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, dtype=torch.int32, device=dev)
    flags = (IDX_SORTED if sorted else 0) | (IDX_RADIX8 if radix8 else 0)
    nbytes = lib.idx_topk_workspace_bytes(B, N, K, flags)
    if ws is None and nbytes:
        ws = _workspace(dev, nbytes, "topk")
    _check("idx_topk", lib.idx_topk(_ptr(scores), _ptr(n_valid), _ptr(ids), _ptr(counts), B, N, K,
                                    flags, _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(dev)))
    return ids, counts


def idx_topk_bf16(scores, K, n_valid=None, sorted=False, ids=None, counts=None, ws=None,
                  radix8=False):
    """idx_topk over bfloat16 scores (16-bit keys, half the bytes read). The
    library rejects radix8 here (IDX_ERR_UNSUPPORTED)."""
    lib = load()
    dev = _dev(scores, n_valid, ids, counts, ws)
    if scores.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("idx_topk_bf16 takes bfloat16 scores")
    B, N = scores.shape
    if ids is None:
        ids = torch.empty(B, K, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, dtype=torch.int32, device=dev)
    flags = (IDX_SORTED if sorted else 0) | (IDX_RADIX8 if radix8 else 0)
    nbytes = lib.idx_topk_workspace_bytes(B, N, K, flags)
    if ws is None and nbytes:
        ws = _workspace(dev, nbytes, "topk")
    _check("idx_topk_bf16", lib.idx_topk_bf16(_ptr(scores), _ptr(n_valid), _ptr(ids),
                                              _ptr(counts), B, N, K, flags, _ptr(ws),
                                              0 if ws is None else ws.numel(), _stream(dev)))
    return ids, counts


def idx_select(q, c, seq_len, K, page_size=16, sorted=False, return_scores=False, ids=None,
               counts=None, scores_out=None, ws=None, chunk_log2=0, radix8=False):
    """Fused score + mask + top-K. Returns (ids, counts, scores_out or None).
    radix8: the select with four 8-bit radix passes (IDX_RADIX8; the same
    results)."""
    lib = load()
    dev = _dev(q, c, seq_len, ids, counts, scores_out, ws)
    B, H, D = q.shape
    N_pad = c.shape[1]
    if ids is None:
        ids = torch.empty(B, K, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, dtype=torch.int32, device=dev)
    if return_scores and scores_out is None:
        scores_out = torch.empty(B, N_pad, dtype=torch.float32, device=dev)
    flags = ((IDX_SORTED if sorted else 0) | (IDX_RADIX8 if radix8 else 0)
             | (int(chunk_log2) << IDX_CHUNK_SHIFT))
    nbytes = lib.idx_workspace_bytes(B, N_pad, H, K, flags)
    if ws is None:
        ws = _workspace(dev, nbytes, "select")
    _check("idx_select", lib.idx_select(_ptr(q), _ptr(c), _ptr(seq_len), _ptr(ids), _ptr(counts),
                                        _ptr(scores_out), B, H, D, N_pad, page_size, K,
                                        _dtype_code(q), flags, _ptr(ws), ws.numel(), _stream(dev)))
    return ids, counts, scores_out


def idx_select_noalloc(q, c, seq_len, K, page_size=16, sorted=False, return_scores=False,
                       ids=None, counts=None, scores_out=None, chunk_log2=0, radix8=False):
    """idx_select without a workspace: the library's static per-GPU scratch holds
    the arrival counters and staging (calls on one GPU must not overlap).
    Returns (ids, counts, scores_out or None)."""
    lib = load()
    dev = _dev(q, c, seq_len, ids, counts, scores_out)
    B, H, D = q.shape
    N_pad = c.shape[1]
    if ids is None:
        ids = torch.empty(B, K, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, dtype=torch.int32, device=dev)
    if return_scores and scores_out is None:
        scores_out = torch.empty(B, N_pad, dtype=torch.float32, device=dev)
    flags = ((IDX_SORTED if sorted else 0) | (IDX_RADIX8 if radix8 else 0)
             | (int(chunk_log2) << IDX_CHUNK_SHIFT))
    _check("idx_select_noalloc", lib.idx_select_noalloc(
        _ptr(q), _ptr(c), _ptr(seq_len), _ptr(ids), _ptr(counts), _ptr(scores_out), B, H, D,
        N_pad, page_size, K, _dtype_code(q), flags, _stream(dev)))
    return ids, counts, scores_out


def idx_select_paged(q, c_pool, kv_indptr, kv_indices, K, max_pages, sorted=False,
                     return_scores=False, ids=None, counts=None, scores_out=None, ws=None,
                     chunk_log2=0):
    """Fused score + top-K over a paged centroid pool: request b's slots are
    kv_indices[kv_indptr[b]:kv_indptr[b+1]] (at most max_pages of them).
    Returns (ids, counts, scores_out or None); ids are slot positions."""
    lib = load()
    dev = _dev(q, c_pool, kv_indptr, kv_indices, ids, counts, scores_out, ws)
    if kv_indptr.dtype != torch.int32 or kv_indices.dtype != torch.int32:
        raise TypeError("kv_indptr and kv_indices must be int32")
    B, H, D = q.shape
    if kv_indptr.numel() != B + 1:
        raise ValueError("kv_indptr must hold B + 1 entries")
    n_rows = c_pool.shape[0]
    if ids is None:
        ids = torch.empty(B, K, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, dtype=torch.int32, device=dev)
    if return_scores and scores_out is None:
        scores_out = torch.empty(B, max_pages, dtype=torch.float32, device=dev)
    flags = (IDX_SORTED if sorted else 0) | (int(chunk_log2) << IDX_CHUNK_SHIFT)
    nbytes = lib.idx_workspace_bytes(B, max_pages, H, K, flags)
    if ws is None:
        ws = _workspace(dev, nbytes, "select")
    _check("idx_select_paged", lib.idx_select_paged(
        _ptr(q), _ptr(c_pool), _ptr(kv_indptr), _ptr(kv_indices), _ptr(ids), _ptr(counts),
        _ptr(scores_out), B, H, D, n_rows, kv_indices.numel(), max_pages, K, _dtype_code(q),
        flags, _ptr(ws), ws.numel(), _stream(dev)))
    return ids, counts, scores_out


def idx_pool_keys(k, seq_len, N_pad, page_size=16, c=None):
    """Block centroids: c[b,n] = mean of the keys k[b, tokens of block n]
    (k [B,S_pad,128], float32 or bf16). Rows past a request's blocks are not
    written (a new c is zero-filled)."""
    lib = load()
    dev = _dev(k, seq_len, c)
    B, S_pad, D = k.shape
    if c is None:
        c = torch.zeros(B, N_pad, D, dtype=k.dtype, device=dev)
    _check("idx_pool_keys", lib.idx_pool_keys(_ptr(k), _ptr(seq_len), _ptr(c), B, S_pad, D, N_pad,
                                              page_size, _dtype_code(k), _stream(dev)))
    return c


def idx_prefill_workspace_bytes(B, T, N_pad, K, flags=0) -> int:
    return load().idx_prefill_workspace_bytes(B, T, N_pad, K, flags)


def idx_select_prefill(q, c, pos0, K, page_size=16, sorted=False, return_scores=False, ids=None,
                       counts=None, scores_out=None, ws=None):
    """Per-token scores and top-K of T prompt tokens per request (q [B,T,H,D],
    c [B,N_pad,D], bf16). Returns (ids [B,T,K], counts [B,T], scores_out or None)."""
    lib = load()
    dev = _dev(q, c, pos0, ids, counts, scores_out, ws)
    B, T, H, D = q.shape
    N_pad = c.shape[1]
    if ids is None:
        ids = torch.empty(B, T, K, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.empty(B, T, dtype=torch.int32, device=dev)
    if return_scores and scores_out is None:
        scores_out = torch.empty(B, T, N_pad, dtype=torch.float32, device=dev)
    flags = IDX_SORTED if sorted else 0
    nbytes = lib.idx_prefill_workspace_bytes(B, T, N_pad, K, flags)
    if ws is None:
        ws = _workspace(dev, nbytes, "prefill")
    _check("idx_select_prefill", lib.idx_select_prefill(
        _ptr(q), _ptr(c), _ptr(pos0), _ptr(ids), _ptr(counts), _ptr(scores_out), B, T, H, D,
        N_pad, page_size, K, _dtype_code(q), flags, _ptr(ws), ws.numel(), _stream(dev)))
    return ids, counts, scores_out


def idx_assign(x, c, return_best=False, assign=None, best=None, ws=None):
    """k-means assignment: argmax_j (2 x.c_j - |c_j|^2), ties to the lower j."""
    lib = load()
    dev = _dev(x, c, assign, best, ws)
    N, D = x.shape
    C = c.shape[0]
    if assign is None:
        assign = torch.empty(N, dtype=torch.int32, device=dev)
    if return_best and best is None:
        best = torch.empty(N, dtype=torch.float32, device=dev)
    nbytes = lib.idx_assign_workspace_bytes(C, D)
    if ws is None:
        ws = _workspace(dev, nbytes, "assign")
    _check("idx_assign", lib.idx_assign(_ptr(x), _ptr(c), _ptr(assign), _ptr(best), N, C, D,
                                        _dtype_code(x), _ptr(ws), ws.numel(), _stream(dev)))
    return assign, best


def idx_floor_empty(blocks=1):
    """One empty launch of `blocks` workgroups (measurement floor)."""
    _check("idx_floor_empty", load().idx_floor_empty(blocks, _stream(torch.cuda.current_device())))


def idx_floor_read(src, nbytes, sink, ticket=None, blocks=256, threads=256):
    """Stream-read the first `nbytes` bytes of `src` (measurement floor); with a
    zeroed one-word `ticket`, every workgroup then takes a ticket on it."""
    dev = _dev(src, sink, ticket)
    if nbytes > src.numel() * src.element_size() or sink.numel() < blocks:
        raise ValueError("idx_floor_read: buffer too small")
    _check("idx_floor_read", load().idx_floor_read(_ptr(src), nbytes, _ptr(sink), _ptr(ticket),
                                                   blocks, threads, _stream(dev)))


def idx_floor_mfma(frags, blocks, iters, sink):
    """`blocks` x 4 waves of back-to-back bf16 matrix products, `iters` rounds of
    four per wave on operands from `frags` (16 KiB; measurement floor); each
    thread writes one word to `sink`."""
    dev = _dev(frags, sink)
    if frags.numel() * frags.element_size() < 16384 or sink.numel() < 256 * blocks:
        raise ValueError("idx_floor_mfma: buffer too small")
    _check("idx_floor_mfma", load().idx_floor_mfma(_ptr(frags), blocks, iters, _ptr(sink),
                                                   _stream(dev)))


class SelectPlan:
    """idx_select for one call signature, resolved once by the library
    (idx_plan_create: kernel instance, workgroup size and chunking fixed up
    front), with its own zero-filled workspace on `device`. Calling it checks
    only that the tensors match the signature; capture() records plan calls
    into a HIP graph. Calls of one plan must not overlap (one workspace)."""

    def __init__(self, B, H, N_pad, K, dtype=torch.bfloat16, page_size=16, sorted=False,
                 device=None, chunk_log2=0):
        lib = load()
        if dtype not in (torch.bfloat16, torch.float32):
            raise TypeError(f"unsupported dtype {dtype}")
        self.B, self.H, self.N_pad, self.K, self.page_size = B, H, N_pad, K, page_size
        self.dtype, self.sorted = dtype, sorted
        flags = (IDX_SORTED if sorted else 0) | (int(chunk_log2) << IDX_CHUNK_SHIFT)
        handle = _vp()
        _check("idx_plan_create", lib.idx_plan_create(
            ctypes.byref(handle), B, H, 128, N_pad, page_size, K,
            IDX_BF16 if dtype == torch.bfloat16 else IDX_F32, flags))
        self._lib, self._handle = lib, handle
        dev = torch.device(device if device is not None else "cuda")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.ws = torch.zeros(max(lib.idx_plan_workspace_bytes(handle), 256), dtype=torch.uint8,
                              device=dev)

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h is not None and h.value is not None:
            self._lib.idx_plan_destroy(h)
            self._handle = None

    def __call__(self, q, c, seq_len, ids=None, counts=None, scores_out=None):
        """Returns (ids, counts, scores_out or None), as idx_select does."""
        dev = _dev(q, c, seq_len, ids, counts, scores_out)
        if dev != self.device:
            raise ValueError("the plan's workspace lives on another device")
        if (tuple(q.shape) != (self.B, self.H, 128) or tuple(c.shape) != (self.B, self.N_pad, 128)
                or q.dtype != self.dtype or c.dtype != self.dtype or seq_len.numel() != self.B):
            raise ValueError("tensors do not match the plan's signature")
        if ids is None:
            ids = torch.empty(self.B, self.K, dtype=torch.int32, device=dev)
        if counts is None:
            counts = torch.empty(self.B, dtype=torch.int32, device=dev)
        _check("idx_plan_select", self._lib.idx_plan_select(
            self._handle, _ptr(q), _ptr(c), _ptr(seq_len), _ptr(ids), _ptr(counts),
            _ptr(scores_out), _ptr(self.ws), self.ws.numel(), _stream(dev)))
        return ids, counts, scores_out

    def capture(self, q, c, seq_len, ids, counts, scores_out=None, calls=1):
        """A HIP graph of `calls` plan calls on these buffers (they must stay
        alive while the graph is replayed); one eager call first runs on the
        capturing stream."""
        side = torch.cuda.Stream(self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            self(q, c, seq_len, ids, counts, scores_out)
        torch.cuda.current_stream(self.device).wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                self(q, c, seq_len, ids, counts, scores_out)
        return g


_plan_cache: dict = {}


def plan_for(B, H, N_pad, K, dtype=torch.bfloat16, page_size=16, sorted=False, device=None):
    """The cached SelectPlan of a signature (created on first use)."""
    dev = torch.device(device if device is not None else "cuda")
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (B, H, N_pad, K, dtype, page_size, bool(sorted), index)
    p = _plan_cache.get(key)
    if p is None:
        p = SelectPlan(B, H, N_pad, K, dtype, page_size, sorted, torch.device("cuda", index))
        _plan_cache[key] = p
    return p
