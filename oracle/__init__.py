"""CPU oracle for the group-quantized matmul and the routed MoE FFN.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``.  Nothing in the GPU library imports it,
and nothing it computes is ever fed by a GPU result.

The arithmetic lives in ``oracle.c`` (plain C99 + OpenMP, built with
``-O2 -ffp-contract=off``); this module only marshals numpy arrays and
composes the per-expert reference into a whole MoE layer.

Sources: "Hand-writing a DeepSeek inference engine in pure C"
(hnwysp.cn/news/134870) §2.1, §2.3, §3.2-§3.5, §5.1; "ds4 code walkthrough"
(the RMSNorm epsilon); "Running a 284B-parameter LLM
from 3.2 GB of RAM in plain C" (feinterview.poetries.top), section on bitwise
identical CPU paths.

Parity status: every function here is pinned by tests under
``tests/test_oracle_*.py`` (closed forms, exact-arithmetic special cases,
invariants, brute force, library special cases).  The last bits of libm's
``exp`` inside softmax and silu are pinned only through closed-form values
(softmax of ln-spaced logits, large-logit shift invariance); everything
downstream of ``exp`` is compared under a tolerance, never bitwise.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-std=c99", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]

FLAG_DEGENERATE = 1
FLAG_NONFINITE = 2


# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source (a
# host-only library; gcc, no GPU code): every out-of-bounds access, leak-free
# misuse of malloc'd scratch or undefined operation aborts the process.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
            "-g"]


def build(force: bool = True, out: str = None, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU code involved).
    With sanitize=True the library is instrumented with ASan/UBSan and
    written to `out` (it can only be loaded into a process whose main program
    preloads the ASan runtime)."""
    dst = out or _LIB
    if force or not os.path.exists(dst):
        tmp = dst + ".tmp"
        flags = [*CFLAGS, *(SANITIZE if sanitize else [])]
        subprocess.check_call(["gcc", *flags, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, dst)
    return dst


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.orc_set_threads.argtypes = [i32]
        L.orc_max_threads.restype = i32
        L.orc_quantize.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, vp]
        L.orc_quantize.restype = i64
        L.orc_dequant_f64.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp]
        L.orc_dequant_f32.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp]
        L.orc_matmul_f64.argtypes = [vp, i64, vp, i64, i64, vp, vp]
        L.orc_qmatmul_f32.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, i32, vp]
        L.orc_router_f64.argtypes = [vp, i64, vp, vp, i32, i64, vp, vp]
        L.orc_route.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.orc_route.restype = i32
        L.orc_group.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.orc_group.restype = i32
        L.orc_topk_f32.argtypes = [vp, i64, i32, vp, vp]
        L.orc_topk_f32.restype = i32
        L.orc_rmsnorm_f64.argtypes = [vp, vp, i64, i64, ctypes.c_double, vp]
        L.orc_rmsnorm_f64.restype = i32
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_sb4_quantize.argtypes = [vp, i64, i64, vp, vp]
        L.orc_sb4_quantize.restype = i64
        L.orc_sb4_dequant_f64.argtypes = [vp, i64, i64, vp]
        L.orc_sb4_dequant_f64.restype = i32
        L.orc_silu_f64.argtypes = [ctypes.c_double]
        L.orc_silu_f64.restype = ctypes.c_double
        L.orc_dsilu_f64.argtypes = [ctypes.c_double]
        L.orc_dsilu_f64.restype = ctypes.c_double
        L.orc_expert_f64.argtypes = [vp, i64, i64] + [vp] * 9 + [i32, i32] + [vp] * 6
        L.orc_moe_f32.argtypes = ([vp, i64, i64, i64, i32, i32, vp, vp] + [vp] * 9
                                  + [i32, i32, i32, vp, vp, vp])
        L.orc_moe_f32.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def silu(z: float) -> float:
    """The oracle's silu(z) = z / (1 + e^-z) in fp64 (used by orc_expert_f64)."""
    return float(lib().orc_silu_f64(float(z)))


def dsilu(z: float) -> float:
    """The oracle's d/dz silu(z) in fp64 (the tolerance helper of orc_expert_f64)."""
    return float(lib().orc_dsilu_f64(float(z)))


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# --------------------------------------------------------------------------
# Quantized weights in the oracle's canonical format
# --------------------------------------------------------------------------
class QMat:
    """Canonical quantized matrix W[rows][K] (see oracle.c for the format)."""

    def __init__(self, q, scale, zp, flags, rows, K, bits, group):
        self.q, self.scale, self.zp, self.flags = q, scale, zp, flags
        self.rows, self.K, self.bits, self.group = rows, K, bits, group

    def dequant_f64(self) -> np.ndarray:
        w = np.empty((self.rows, self.K), np.float64)
        lib().orc_dequant_f64(_p(self.q), _p(self.scale), _p(self.zp), self.rows, self.K,
                              self.bits, self.group, _p(w))
        return w

    def dequant_f32(self) -> np.ndarray:
        w = np.empty((self.rows, self.K), np.float32)
        lib().orc_dequant_f32(_p(self.q), _p(self.scale), _p(self.zp), self.rows, self.K,
                              self.bits, self.group, _p(w))
        return w


def quantize(w: np.ndarray, bits: int, group: int) -> QMat:
    """Group-wise asymmetric quantization of w[rows][K] along K
    (hnwysp.cn/news/134870 §3.2)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    qb = K if bits == 8 else K // 2
    q = np.empty((rows, qb), np.uint8)
    ng = K // group
    scale = np.empty((rows, ng), np.float32)
    zp = np.empty((rows, ng), np.float32)
    flags = np.empty((rows, ng), np.uint8)
    n = lib().orc_quantize(_p(w), rows, K, bits, group, _p(q), _p(scale), _p(zp), _p(flags))
    if n < 0:
        raise ValueError(f"orc_quantize rejected bits={bits} group={group} K={K}")
    return QMat(q, scale, zp, flags, rows, K, bits, group)


def unpack_q(m: QMat) -> np.ndarray:
    """Integer codes q[rows][K] (0..2^bits-1) from the canonical bytes."""
    if m.bits == 8:
        return m.q.astype(np.int32)
    out = np.empty((m.rows, m.K), np.int32)
    out[:, 0::2] = m.q & 0x0F
    out[:, 1::2] = m.q >> 4
    return out


# --------------------------------------------------------------------------
# Two-level super-block 4-bit format (see oracle.c for the reading of the
# block's fields): blocks[rows][K/256][144] =
#   [fp16 d][fp16 dmin][12 bytes: sc_0..7, m_0..7 as 6-bit fields][128 B codes]
# --------------------------------------------------------------------------
SB_K = 256
SB_BYTES = 144


class SB4Mat:
    def __init__(self, blocks, flags, rows, K):
        self.blocks, self.flags, self.rows, self.K = blocks, flags, rows, K

    def dequant_f64(self) -> np.ndarray:
        w = np.empty((self.rows, self.K), np.float64)
        if lib().orc_sb4_dequant_f64(_p(self.blocks), self.rows, self.K, _p(w)) != 0:
            raise ValueError("orc_sb4_dequant_f64: invalid arguments")
        return w


def sb4_quantize(w: np.ndarray) -> SB4Mat:
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    if K % SB_K:
        raise ValueError("sb4_quantize: K must be a multiple of 256")
    blocks = np.empty((rows, K // SB_K, SB_BYTES), np.uint8)
    flags = np.empty((rows, K // SB_K), np.uint8)
    if lib().orc_sb4_quantize(_p(w), rows, K, _p(blocks), _p(flags)) < 0:
        raise ValueError("orc_sb4_quantize: invalid arguments")
    return SB4Mat(blocks, flags, rows, K)


def f16_bits(values) -> np.ndarray:
    """fp32 -> binary16 bits (round to nearest even), one value at a time."""
    v = np.ascontiguousarray(values, np.float32).reshape(-1)
    return np.array([lib().orc_f32_to_f16(float(x)) for x in v], np.uint16)


def f16_value(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).reshape(-1)
    return np.array([lib().orc_f16_to_f64(int(h)) for h in b], np.float64)


def qmatmul_sb4_ref(X: np.ndarray, m: SB4Mat):
    """Reference for the super-block GEMV/GEMM: exact fp64 weights, fp64 sums."""
    return matmul_f64(X, m.dequant_f64())


# --------------------------------------------------------------------------
# Matmul
# --------------------------------------------------------------------------
def matmul_f64(X: np.ndarray, W: np.ndarray):
    """Y = X W^T and S = |X| |W|^T in fp64, plain sequential-k loops."""
    X = np.ascontiguousarray(X, np.float64)
    W = np.ascontiguousarray(W, np.float64)
    M, K = X.shape
    N = W.shape[0]
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    lib().orc_matmul_f64(_p(X), M, _p(W), N, K, _p(Y), _p(S))
    return Y, S


def qmatmul_ref(X: np.ndarray, m: QMat):
    """Reference for the fused-dequant matmul: exact fp64 weights, fp64 sums."""
    return matmul_f64(X, m.dequant_f64())


def qmatmul_f32(X: np.ndarray, m: QMat) -> np.ndarray:
    """The pages' fp32 CPU method: dequant inside the inner loop, OpenMP over
    outputs, fixed 16-way accumulator tree."""
    X = np.ascontiguousarray(X, np.float32)
    M, K = X.shape
    assert K == m.K
    Y = np.empty((M, m.rows), np.float32)
    lib().orc_qmatmul_f32(_p(X), M, _p(m.q), _p(m.scale), _p(m.zp), m.rows, m.K, m.bits,
                          m.group, _p(Y))
    return Y


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------
def router_f64(X: np.ndarray, Wr: np.ndarray, bias=None):
    X = np.ascontiguousarray(X, np.float64)
    Wr = np.ascontiguousarray(Wr, np.float64)
    T, H = X.shape
    E = Wr.shape[0]
    L = np.empty((T, E), np.float64)
    S = np.empty((T, E), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float64)
    lib().orc_router_f64(_p(X), T, _p(Wr), None if b is None else _p(b), E, H, _p(L), _p(S))
    return L, S


def route(logits: np.ndarray, k: int):
    """softmax (max-subtracted) + top-k by (logit desc, index desc) + renorm."""
    L = np.ascontiguousarray(logits, np.float64)
    T, E = L.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty((T,), np.float64)
    if lib().orc_route(_p(L), T, E, k, _p(idx), _p(w), _p(gap)) != 0:
        raise ValueError("orc_route: invalid arguments or non-finite logits")
    return idx, w, gap


def rmsnorm_f64(X: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row of X (fp32 [T][H]) with weight g (fp32 [H]) and
    epsilon eps, in fp64: x / sqrt(mean(x^2) + eps) * g."""
    X = np.ascontiguousarray(X, np.float32)
    X2 = X.reshape(-1, X.shape[-1])
    g = np.ascontiguousarray(g, np.float32).reshape(-1)
    if g.size != X2.shape[1]:
        raise ValueError("rmsnorm_f64: weight length differs from the row length")
    out = np.empty(X2.shape, np.float64)
    if lib().orc_rmsnorm_f64(_p(X2), _p(g), X2.shape[0], X2.shape[1], float(eps), _p(out)) != 0:
        raise ValueError("orc_rmsnorm_f64: invalid arguments")
    return out.reshape(X.shape)


def topk(y: np.ndarray, k: int):
    """Output-head selection: the k largest of y (fp32) by (value desc, index
    asc), NaN last; returns (idx int32 [k], values float32 [k])."""
    y = np.ascontiguousarray(y, np.float32).reshape(-1)
    idx = np.empty((k,), np.int32)
    val = np.empty((k,), np.float32)
    if lib().orc_topk_f32(_p(y), y.size, k, _p(idx), _p(val)) != 0:
        raise ValueError("orc_topk_f32: invalid arguments")
    return idx, val


def group(idx: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    counts = np.empty((E,), np.int32)
    offsets = np.empty((E + 1,), np.int32)
    perm = np.empty((T * k,), np.int32)
    if lib().orc_group(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm)) != 0:
        raise ValueError("orc_group: expert id out of range")
    return counts, offsets, perm


# --------------------------------------------------------------------------
# Experts and the MoE layer
# --------------------------------------------------------------------------
class Expert:
    """Quantized SwiGLU expert: gate/up [I][H], down [H][I]."""

    def __init__(self, gate: QMat, up: QMat, down: QMat):
        self.gate, self.up, self.down = gate, up, down
        self.H = gate.K
        self.I = gate.rows
        self.bits, self.group = gate.bits, gate.group


def quantize_expert(wg, wu, wd, bits, group) -> Expert:
    return Expert(quantize(wg, bits, group), quantize(wu, bits, group), quantize(wd, bits, group))


def expert_f64(x: np.ndarray, ex: Expert, want_gu: bool = False):
    """One expert on one token in fp64: returns y [H], Sd [H], Pd [H]
    (and g, u, h when want_gu)."""
    x = np.ascontiguousarray(x, np.float64)
    H, I = ex.H, ex.I
    y = np.empty(H, np.float64)
    Sd = np.empty(H, np.float64)
    Pd = np.empty(H, np.float64)
    g = np.empty(I, np.float64) if want_gu else None
    u = np.empty(I, np.float64) if want_gu else None
    h = np.empty(I, np.float64) if want_gu else None
    G, U, D = ex.gate, ex.up, ex.down
    lib().orc_expert_f64(_p(x), H, I, _p(G.q), _p(G.scale), _p(G.zp), _p(U.q), _p(U.scale),
                         _p(U.zp), _p(D.q), _p(D.scale), _p(D.zp), ex.bits, ex.group, _p(y),
                         _p(Sd), _p(Pd), None if g is None else _p(g),
                         None if u is None else _p(u), None if h is None else _p(h))
    if want_gu:
        return y, Sd, Pd, g, u, h
    return y, Sd, Pd


def moe_combine_f64(X: np.ndarray, tokens, idx: np.ndarray, w: np.ndarray, experts):
    """Y[t] = sum_i w[t,i] * expert_{idx[t,i]}(X[t]) in slot order, fp64, for
    the listed tokens.  `experts` maps expert id -> Expert.  Also returns the
    tolerance helpers S_Y = sum_i w_i * Sd_i and P_Y = sum_i w_i * Pd_i."""
    H = X.shape[1]
    Y = np.zeros((len(tokens), H), np.float64)
    SY = np.zeros_like(Y)
    PY = np.zeros_like(Y)
    for r, t in enumerate(tokens):
        for i in range(idx.shape[1]):
            y, Sd, Pd = expert_f64(X[t], experts[int(idx[t, i])])
            Y[r] += w[t, i] * y
            SY[r] += w[t, i] * Sd
            PY[r] += w[t, i] * Pd
    return Y, SY, PY


def moe_f32(X: np.ndarray, idx: np.ndarray, w: np.ndarray, experts: dict, E: int,
            grouped: bool = True) -> np.ndarray:
    """The pages' fp32 CPU MoE (timed baseline)."""
    X = np.ascontiguousarray(X, np.float32)
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T, H = X.shape
    k = idx.shape[1]
    any_ex = next(iter(experts.values()))
    I = any_ex.I
    arrs = {name: (ctypes.c_void_p * E)() for name in
            ("gq", "gs", "gz", "uq", "us", "uz", "dq", "ds", "dz")}
    for e, ex in experts.items():
        for pre, m in (("g", ex.gate), ("u", ex.up), ("d", ex.down)):
            arrs[pre + "q"][e] = m.q.ctypes.data
            arrs[pre + "s"][e] = m.scale.ctypes.data
            arrs[pre + "z"][e] = m.zp.ctypes.data
    h_ws = np.empty((T * k, I), np.float32)
    y_ws = np.empty((T * k, H), np.float32)
    Y = np.empty((T, H), np.float32)
    rc = lib().orc_moe_f32(_p(X), T, H, I, E, k, _p(idx), _p(w),
                           *[arrs[n] for n in ("gq", "gs", "gz", "uq", "us", "uz", "dq", "ds",
                                               "dz")],
                           any_ex.bits, any_ex.group, 1 if grouped else 0, _p(h_ws), _p(y_ws),
                           _p(Y))
    if rc != 0:
        raise ValueError("orc_moe_f32 failed")
    return Y
