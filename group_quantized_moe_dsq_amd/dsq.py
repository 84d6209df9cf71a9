"""Thin ctypes binding of libdsq (include/dsq.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libdsq.so.  If the library is missing this module raises; there is
no fallback of any kind.  Tensors are torch tensors on the GPU; calls enqueue
on torch's current stream (or the one passed in).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsq.so")

DSQ_OK = 0
STATUS = {0: "DSQ_OK", -1: "DSQ_ERR_INVALID_ARG", -2: "DSQ_ERR_SHAPE", -3: "DSQ_ERR_ALIGN",
          -4: "DSQ_ERR_WORKSPACE", -5: "DSQ_ERR_UNSUPPORTED", -6: "DSQ_ERR_NO_DEVICE",
          -7: "DSQ_ERR_HIP", -8: "DSQ_ERR_OVERFLOW", -9: "DSQ_ERR_LAYOUT"}
MATH_FP32, MATH_BF16_MFMA, MATH_AUTO = 0, 1, 2
FLAG_DEGENERATE, FLAG_NONFINITE = 1, 2
LAYOUT_VERSION = 1

EXPORTS = ["dsq_status_string", "dsq_packed_bytes", "dsq_qweight_init", "dsq_pack_weights",
           "dsq_gemv", "dsq_gemm_workspace_bytes", "dsq_gemm", "dsq_moe_route_topk",
           "dsq_moe_group_workspace_bytes", "dsq_moe_group",
           "dsq_moe_workspace_bytes", "dsq_moe_ffn", "dsq_moe_ffn_noalloc",
           "dsq_topk_workspace_bytes", "dsq_topk",
           "dsq_gemv_topk", "dsq_moe_block_workspace_bytes", "dsq_moe_block",
           "dsq_expert_cache_init", "dsq_expert_cache_plan", "dsq_moe_cached_workspace_bytes",
           "dsq_moe_ffn_cached"]


class DsqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class QWeightDesc(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("K", ctypes.c_int64),
                ("N", ctypes.c_int64), ("batch", ctypes.c_int64),
                ("layout_version", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("data", ctypes.c_void_p)]


class ExpertCacheDesc(ctypes.Structure):
    _fields_ = [("gate", QWeightDesc), ("up", QWeightDesc), ("down", QWeightDesc),
                ("host_gate", ctypes.c_void_p), ("host_up", ctypes.c_void_p),
                ("host_down", ctypes.c_void_p), ("E", ctypes.c_int32), ("slots", ctypes.c_int32),
                ("slot_of", ctypes.c_void_p), ("expert_of", ctypes.c_void_p),
                ("last_use", ctypes.c_void_p), ("clock", ctypes.c_uint64),
                ("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64),
                ("bytes_copied", ctypes.c_uint64)]


_lib = None


def lib():
    """Open libdsq.so; raise if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m group_quantized_moe_dsq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        pd = ctypes.POINTER(QWeightDesc)
        L.dsq_status_string.argtypes = [i32]
        L.dsq_status_string.restype = ctypes.c_char_p
        L.dsq_packed_bytes.argtypes = [i32, i32, i64, i64, i64]
        L.dsq_packed_bytes.restype = sz
        L.dsq_qweight_init.argtypes = [pd, i32, i32, i64, i64, i64, vp]
        L.dsq_qweight_init.restype = i32
        L.dsq_pack_weights.argtypes = [vp, pd, i64, i64, vp, vp]
        L.dsq_pack_weights.restype = i32
        L.dsq_gemv.argtypes = [pd, i64, vp, vp, vp]
        L.dsq_gemv.restype = i32
        L.dsq_gemm_workspace_bytes.argtypes = [i64, i64, i64, i32]
        L.dsq_gemm_workspace_bytes.restype = sz
        L.dsq_gemm.argtypes = [pd, i64, vp, vp, i64, i32, vp, sz, vp]
        L.dsq_gemm.restype = i32
        L.dsq_moe_route_topk.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
        L.dsq_moe_route_topk.restype = i32
        L.dsq_moe_group_workspace_bytes.argtypes = [i64, i32, i32]
        L.dsq_moe_group_workspace_bytes.restype = sz
        L.dsq_moe_group.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.dsq_moe_group.restype = i32
        L.dsq_moe_workspace_bytes.argtypes = [i64, i32, i32, i64, i64, i32]
        L.dsq_moe_workspace_bytes.restype = sz
        L.dsq_moe_ffn.argtypes = [vp, vp, vp, pd, pd, pd, i64, i32, i32, vp, vp, sz, vp, vp, vp,
                                  vp, vp]
        L.dsq_moe_ffn.restype = i32
        L.dsq_moe_ffn_noalloc.argtypes = [vp, vp, vp, pd, pd, pd, i64, i32, i32, vp, vp, vp, vp,
                                          vp, vp]
        L.dsq_moe_ffn_noalloc.restype = i32
        L.dsq_moe_block_workspace_bytes.argtypes = [i64, i32, i32, i64, i64, i32]
        L.dsq_moe_block_workspace_bytes.restype = sz
        L.dsq_moe_block.argtypes = [vp, vp, ctypes.c_float, vp, vp, pd, pd, pd, i64, i32, i32, vp,
                                    vp, sz, vp, vp, vp, vp, vp, vp]
        L.dsq_moe_block.restype = i32
        pc = ctypes.POINTER(ExpertCacheDesc)
        L.dsq_expert_cache_init.argtypes = [pc, pd, pd, pd, vp, vp, vp, i32, vp, vp, vp]
        L.dsq_expert_cache_init.restype = i32
        L.dsq_expert_cache_plan.argtypes = [pc, vp, i64, vp, vp, vp, vp]
        L.dsq_expert_cache_plan.restype = i32
        L.dsq_moe_cached_workspace_bytes.argtypes = [i64, i32, i32, i32, i64, i64, i32]
        L.dsq_moe_cached_workspace_bytes.restype = sz
        L.dsq_moe_ffn_cached.argtypes = [vp, vp, vp, pc, i64, i32, i32, vp, vp, sz, vp, vp, vp, vp,
                                         vp, vp]
        L.dsq_moe_ffn_cached.restype = i32
        L.dsq_topk_workspace_bytes.argtypes = [i64, i32]
        L.dsq_topk_workspace_bytes.restype = sz
        L.dsq_topk.argtypes = [vp, i64, i32, vp, vp, vp, sz, vp]
        L.dsq_topk.restype = i32
        L.dsq_gemv_topk.argtypes = [pd, i64, vp, vp, i32, vp, vp, vp, sz, vp]
        L.dsq_gemv_topk.restype = i32
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != DSQ_OK:
        raise DsqError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")


def status_string(s: int) -> str:
    return lib().dsq_status_string(s).decode()


def packed_bytes(bits: int, group: int, K: int, N: int, batch: int = 1) -> int:
    return int(lib().dsq_packed_bytes(bits, group, K, N, batch))


class QWeight:
    """A packed weight W[batch][N][K]: a uint8 device buffer plus its
    descriptor.  The buffer is allocated here (torch caching allocator), never
    inside libdsq."""

    def __init__(self, bits: int, group: int, K: int, N: int, batch: int = 1,
                 device="cuda", buf: torch.Tensor | None = None):
        nbytes = packed_bytes(bits, group, K, N, batch)
        if nbytes == 0:
            raise DsqError(-2, f"dsq_packed_bytes(bits={bits}, group={group}, K={K}, N={N})")
        if buf is None:
            buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-buf.data_ptr()) % 256
        self._storage = buf
        self.buf = buf[off:off + nbytes]
        self.bits, self.group, self.K, self.N, self.batch = bits, group, K, N, batch
        self.desc = QWeightDesc()
        _check(lib().dsq_qweight_init(ctypes.byref(self.desc), bits, group, K, N, batch,
                                      ctypes.c_void_p(self.buf.data_ptr())), "dsq_qweight_init")

    @property
    def nbytes(self) -> int:
        return self.buf.numel()


def pack_weights(src: torch.Tensor, out: QWeight, first: int = 0, flags=None, stream=None):
    """Quantize fp32 src [count][N][K] (or [N][K]) into entries first.. of out."""
    _need(src, torch.float32, "src")
    count = 1 if src.dim() == 2 else src.shape[0]
    if src.shape[-2:] != (out.N, out.K):
        raise ValueError(f"src shape {tuple(src.shape)} does not match N={out.N} K={out.K}")
    if flags is not None:
        _need(flags, torch.int32, "flags")
    _check(lib().dsq_pack_weights(_ptr(src), ctypes.byref(out.desc), first, count, _ptr(flags),
                                  _stream(stream)), "dsq_pack_weights")


def gemv(W: QWeight, x: torch.Tensor, y: torch.Tensor | None = None, expert: int = 0,
         stream=None) -> torch.Tensor:
    _need(x, torch.float32, "x")
    if y is None:
        y = torch.empty(W.N, dtype=torch.float32, device=x.device)
    _check(lib().dsq_gemv(ctypes.byref(W.desc), expert, _ptr(x), _ptr(y), _stream(stream)),
           "dsq_gemv")
    return y


def topk_workspace_bytes(N: int, k: int) -> int:
    return int(lib().dsq_topk_workspace_bytes(N, k))


def _workspace(workspace, need, device):
    if workspace is None and need:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, 0
    off = (-workspace.data_ptr()) % 256
    return ctypes.c_void_p(workspace.data_ptr() + off), workspace.numel() - off


def topk(y: torch.Tensor, k: int, idx=None, values=None, workspace=None, stream=None):
    """The k largest of y in rank order (value desc, smaller index on ties,
    NaN last): returns (idx int32 [k], values fp32 [k])."""
    _need(y, torch.float32, "y")
    N = y.numel()
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=y.device)
    if values is None:
        values = torch.empty(k, dtype=torch.float32, device=y.device)
    wptr, wbytes = _workspace(workspace, topk_workspace_bytes(N, k), y.device)
    _check(lib().dsq_topk(_ptr(y), N, k, _ptr(idx), _ptr(values), wptr, wbytes,
                          _stream(stream)), "dsq_topk")
    return idx, values


def gemv_topk(W: QWeight, x: torch.Tensor, k: int, y: torch.Tensor | None = None, expert: int = 0,
              idx=None, values=None, workspace=None, stream=None):
    """Output head: y = W[expert] x, then the k largest of y; returns
    (y, idx, values)."""
    _need(x, torch.float32, "x")
    if y is None:
        y = torch.empty(W.N, dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=x.device)
    if values is None:
        values = torch.empty(k, dtype=torch.float32, device=x.device)
    wptr, wbytes = _workspace(workspace, topk_workspace_bytes(W.N, k), x.device)
    _check(lib().dsq_gemv_topk(ctypes.byref(W.desc), expert, _ptr(x), _ptr(y), k, _ptr(idx),
                               _ptr(values), wptr, wbytes, _stream(stream)), "dsq_gemv_topk")
    return y, idx, values


def gemm_workspace_bytes(M: int, N: int, K: int, math: int) -> int:
    return int(lib().dsq_gemm_workspace_bytes(M, N, K, math))


def gemm(W: QWeight, X: torch.Tensor, Y: torch.Tensor | None = None, expert: int = 0,
         math: int = MATH_AUTO, workspace: torch.Tensor | None = None, stream=None):
    _need(X, torch.float32, "X")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, W.N), dtype=torch.float32, device=X.device)
    need = gemm_workspace_bytes(M, W.N, W.K, math)
    if workspace is None and need:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=X.device)
    wptr, wbytes = None, 0
    if workspace is not None:
        off = (-workspace.data_ptr()) % 256
        wptr = ctypes.c_void_p(workspace.data_ptr() + off)
        wbytes = workspace.numel() - off
    _check(lib().dsq_gemm(ctypes.byref(W.desc), expert, _ptr(X), _ptr(Y), M, math, wptr, wbytes,
                          _stream(stream)), "dsq_gemm")
    return Y


def moe_route_topk(logits: torch.Tensor, top_k: int, bias: torch.Tensor | None = None,
                   idx=None, weights=None, stream=None):
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    if idx is None:
        idx = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _check(lib().dsq_moe_route_topk(_ptr(logits), _ptr(bias), T, E, top_k, _ptr(idx),
                                    _ptr(weights), _stream(stream)), "dsq_moe_route_topk")
    return idx, weights


def moe_group_workspace_bytes(T: int, E: int, top_k: int) -> int:
    return int(lib().dsq_moe_group_workspace_bytes(T, E, top_k))


def moe_group(idx: torch.Tensor, E: int, workspace=None, stream=None):
    """Stable grouping of the routing entries idx [T][top_k] by expert:
    returns (counts [E], offsets [E+1], perm [T*k], pos [T*k]), int32."""
    _need(idx, torch.int32, "idx")
    T, k = idx.shape
    dev = idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    pos = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    wptr, wbytes = _workspace(workspace, moe_group_workspace_bytes(T, E, k), dev)
    _check(lib().dsq_moe_group(_ptr(idx) if T else None, T, E, k, _ptr(counts), _ptr(offsets),
                               _ptr(perm), _ptr(pos), wptr, wbytes, _stream(stream)),
           "dsq_moe_group")
    return counts, offsets, perm[:T * k], pos[:T * k]


def moe_workspace_bytes(T: int, E: int, top_k: int, H: int, I: int, math: int) -> int:
    return int(lib().dsq_moe_workspace_bytes(T, E, top_k, H, I, math))


class MoeLayer:
    """Packed weights of one routed MoE layer (router fp32 [E][H])."""

    def __init__(self, router_w: torch.Tensor, gate: QWeight, up: QWeight, down: QWeight,
                 bias: torch.Tensor | None = None, top_k: int = 6):
        self.router_w, self.gate, self.up, self.down = router_w, gate, up, down
        self.bias, self.top_k = bias, top_k
        self.E, self.H, self.I = gate.batch, gate.K, gate.N


def moe_ffn(layer: MoeLayer, X: torch.Tensor, math: int = MATH_AUTO, Y=None,
            workspace: torch.Tensor | None = None, logits_out=None, idx_out=None, w_out=None,
            counts_out=None, stream=None):
    _need(X, torch.float32, "X")
    T = X.shape[0]
    if Y is None:
        Y = torch.empty((T, layer.H), dtype=torch.float32, device=X.device)
    need = moe_workspace_bytes(T, layer.E, layer.top_k, layer.H, layer.I, math)
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=X.device)
    off = (-workspace.data_ptr()) % 256
    _check(lib().dsq_moe_ffn(_ptr(X), _ptr(layer.router_w), _ptr(layer.bias),
                             ctypes.byref(layer.gate.desc), ctypes.byref(layer.up.desc),
                             ctypes.byref(layer.down.desc), T, layer.top_k, math, _ptr(Y),
                             ctypes.c_void_p(workspace.data_ptr() + off),
                             workspace.numel() - off, _ptr(logits_out), _ptr(idx_out),
                             _ptr(w_out), _ptr(counts_out), _stream(stream)), "dsq_moe_ffn")
    return Y


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def moe_ffn_noalloc(layer: MoeLayer, X: torch.Tensor, math: int = MATH_AUTO, Y=None,
                    logits_out=None, idx_out=None, w_out=None, counts_out=None, stream=None):
    """dsq_moe_ffn_noalloc: the MoE layer on the library's fixed scratch (no
    workspace argument; calls that overlap on one device race)."""
    _need(X, torch.float32, "X")
    T = X.shape[0]
    if Y is None:
        Y = torch.empty((T, layer.H), dtype=torch.float32, device=X.device)
    _check(lib().dsq_moe_ffn_noalloc(_ptr(X), _ptr(layer.router_w), _ptr(layer.bias),
                                     ctypes.byref(layer.gate.desc), ctypes.byref(layer.up.desc),
                                     ctypes.byref(layer.down.desc), T, layer.top_k, math,
                                     _ptr(Y), _ptr(logits_out), _ptr(idx_out), _ptr(w_out),
                                     _ptr(counts_out), _stream(stream)), "dsq_moe_ffn_noalloc")
    return Y


def moe_block_workspace_bytes(T: int, E: int, top_k: int, H: int, I: int, math: int) -> int:
    return int(lib().dsq_moe_block_workspace_bytes(T, E, top_k, H, I, math))


def moe_block(layer: MoeLayer, X: torch.Tensor, norm_w: torch.Tensor, eps: float = 1e-6,
              math: int = MATH_AUTO, Y=None, workspace: torch.Tensor | None = None, xn_out=None,
              logits_out=None, idx_out=None, w_out=None, counts_out=None, stream=None):
    """Y = X + moe_ffn(rmsnorm(X) * norm_w); Y may be X (in-place update)."""
    _need(X, torch.float32, "X")
    _need(norm_w, torch.float32, "norm_w")
    T = X.shape[0]
    if Y is None:
        Y = torch.empty((T, layer.H), dtype=torch.float32, device=X.device)
    need = moe_block_workspace_bytes(T, layer.E, layer.top_k, layer.H, layer.I, math)
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=X.device)
    off = (-workspace.data_ptr()) % 256
    _check(lib().dsq_moe_block(_ptr(X), _ptr(norm_w), float(eps), _ptr(layer.router_w),
                               _ptr(layer.bias), ctypes.byref(layer.gate.desc),
                               ctypes.byref(layer.up.desc), ctypes.byref(layer.down.desc), T,
                               layer.top_k, math, _ptr(Y),
                               ctypes.c_void_p(workspace.data_ptr() + off),
                               workspace.numel() - off, _ptr(xn_out), _ptr(logits_out),
                               _ptr(idx_out), _ptr(w_out), _ptr(counts_out), _stream(stream)),
           "dsq_moe_block")
    return Y


class ExpertCache:
    """Host-resident experts streamed into `slots` HBM slots, least recently
    used out.  The host stores hold E packed entries of each matrix in pinned
    memory (fill them with store()); the tables live in numpy arrays owned
    here.  Counters: hits, misses (requests), bytes_copied."""

    def __init__(self, bits: int, group: int, H: int, I: int, E: int, slots: int,
                 device="cuda", pinned: bool = True):
        self.gate = QWeight(bits, group, H, I, slots, device=device)
        self.up = QWeight(bits, group, H, I, slots, device=device)
        self.down = QWeight(bits, group, I, H, slots, device=device)
        self.E, self.slots, self.H, self.I = E, slots, H, I
        self.strides = [packed_bytes(bits, group, H, I), packed_bytes(bits, group, H, I),
                        packed_bytes(bits, group, I, H)]
        self.host = [torch.empty(E * st, dtype=torch.uint8, pin_memory=pinned)
                     for st in self.strides]
        self.slot_of = np.full(E, -1, np.int32)
        self.expert_of = np.full(slots, -1, np.int32)
        self.last_use = np.zeros(slots, np.uint64)
        self.desc = ExpertCacheDesc()
        _check(lib().dsq_expert_cache_init(
            ctypes.byref(self.desc), ctypes.byref(self.gate.desc), ctypes.byref(self.up.desc),
            ctypes.byref(self.down.desc), ctypes.c_void_p(self.host[0].data_ptr()),
            ctypes.c_void_p(self.host[1].data_ptr()), ctypes.c_void_p(self.host[2].data_ptr()), E,
            self.slot_of.ctypes.data, self.expert_of.ctypes.data, self.last_use.ctypes.data),
            "dsq_expert_cache_init")

    def store(self, e: int, wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor):
        """Pack expert e's fp32 weights (on the GPU) into the host stores."""
        for m, (w, src) in enumerate(((wg, self.gate), (wu, self.up), (wd, self.down))):
            q = QWeight(src.bits, src.group, src.K, src.N, 1, device=w.device)
            pack_weights(w.contiguous(), q)
            st = self.strides[m]
            self.host[m][e * st:(e + 1) * st].copy_(q.buf[:st])

    def plan(self, experts: np.ndarray):
        """Host-only slot mapping of one call: (slots, fill_experts, fill_slots)."""
        ex = np.ascontiguousarray(experts, np.int32).reshape(-1)
        n = ex.size
        so, fe, fs = (np.empty(max(n, 1), np.int32) for _ in range(3))
        nf = ctypes.c_int64(0)
        _check(lib().dsq_expert_cache_plan(ctypes.byref(self.desc), ex.ctypes.data, n,
                                           so.ctypes.data, fe.ctypes.data, fs.ctypes.data,
                                           ctypes.byref(nf)), "dsq_expert_cache_plan")
        return so[:n], fe[:nf.value], fs[:nf.value]

    @property
    def hits(self):
        return int(self.desc.hits)

    @property
    def misses(self):
        return int(self.desc.misses)

    @property
    def bytes_copied(self):
        return int(self.desc.bytes_copied)


def moe_cached_workspace_bytes(T, E, slots, top_k, H, I, math) -> int:
    return int(lib().dsq_moe_cached_workspace_bytes(T, E, slots, top_k, H, I, math))


def moe_ffn_cached(router_w: torch.Tensor, bias, cache: ExpertCache, X: torch.Tensor, top_k: int,
                   math: int = MATH_AUTO, Y=None, workspace=None, logits_out=None, idx_out=None,
                   w_out=None, stream=None):
    """One MoE layer with its experts behind `cache` (synchronises the stream
    once: the host must see the routing)."""
    _need(X, torch.float32, "X")
    T = X.shape[0]
    if Y is None:
        Y = torch.empty((T, cache.H), dtype=torch.float32, device=X.device)
    need = moe_cached_workspace_bytes(T, cache.E, cache.slots, top_k, cache.H, cache.I, math)
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=X.device)
    off = (-workspace.data_ptr()) % 256
    host_idx = np.empty(max(T * top_k, 1), np.int32)
    host_slots = np.empty(max(T * top_k, 1), np.int32)
    _check(lib().dsq_moe_ffn_cached(_ptr(X), _ptr(router_w), _ptr(bias), ctypes.byref(cache.desc),
                                    T, top_k, math, _ptr(Y),
                                    ctypes.c_void_p(workspace.data_ptr() + off),
                                    workspace.numel() - off, host_idx.ctypes.data,
                                    host_slots.ctypes.data, _ptr(logits_out), _ptr(idx_out),
                                    _ptr(w_out), _stream(stream)), "dsq_moe_ffn_cached")
    cache.last_slots = host_slots[:T * top_k].reshape(T, top_k)
    return Y
