"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer and
run over every entry point at small, ragged shapes (CPU only).  The oracle
mallocs scratch in its routing, grouping and MoE routines and indexes packed
INT4 bytes by hand; an out-of-bounds access or an undefined operation there
aborts the child process and fails this test."""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle
oracle._LIB = sys.argv[2]
rng = np.random.default_rng(7)
for bits, group, rows, K in ((8, 64, 5, 192), (4, 64, 3, 128), (4, 128, 7, 256), (8, 128, 1, 128)):
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    w[0, :group] = 1.0                         # a degenerate group
    if rows > 2:
        w[2, 3] = np.nan                       # a non-finite group
    m = oracle.quantize(w, bits, group)
    m.dequant_f64(); m.dequant_f32()
    X = rng.standard_normal((3, K)).astype(np.float32)
    oracle.qmatmul_ref(X, m); oracle.qmatmul_f32(X, m)
    oracle.unpack_q(m)
sb = oracle.sb4_quantize((rng.standard_normal((3, 512)) * 0.02).astype(np.float32))
sb.dequant_f64()
oracle.f16_bits([1.0, 65504.0, 1e-8, 7e4]); oracle.f16_value([0x3c00, 0x0001])
E, H, I, T, k = 9, 128, 64, 7, 3
L, S = oracle.router_f64(rng.standard_normal((T, H)), rng.standard_normal((E, H)),
                         rng.standard_normal(E))
idx, wts, gap = oracle.route(L, k)
oracle.group(idx, E)
ex = {}
for e in range(E):
    ex[e] = oracle.quantize_expert(*((rng.standard_normal(s) * 0.02).astype(np.float32)
                                     for s in ((I, H), (I, H), (H, I))), 4, 64)
Xf = rng.standard_normal((T, H)).astype(np.float32)
oracle.expert_f64(Xf[0].astype(np.float64), ex[0], want_gu=True)
oracle.moe_combine_f64(Xf.astype(np.float64), range(T), idx, wts, ex)
for grouped in (True, False):
    oracle.moe_f32(Xf, idx, wts.astype(np.float32), ex, E, grouped=grouped)
oracle.rmsnorm_f64(Xf, np.ones(H, np.float32), 1e-6)
y = rng.standard_normal(1001).astype(np.float32); y[5] = np.nan
oracle.topk(y, 1); oracle.topk(y, 50); oracle.topk(y, 1001)
oracle.silu(0.5); oracle.dsilu(-0.5)
print("sanitized oracle ok")
'''


def _asan_runtime():
    try:
        p = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.build(force=True, out=os.path.join(d, "liboracle_san.so"), sanitize=True)
        env = dict(os.environ, LD_PRELOAD=rt, OMP_NUM_THREADS="2",
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT, lib], env=env,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and "sanitized oracle ok" in r.stdout, \
            f"rc={r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
