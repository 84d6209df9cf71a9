"""Re-entrancy: the compute calls keep no state between calls, so calls on two
streams at once (each with its own workspace and outputs) give the same
bytes as the same calls one after another.  Two default-priority streams
each run a series of MoE (decode and grouped), GEMM (split-K and grouped)
and GEMV calls on different inputs; every output is compared bitwise with a
sequential run on the current stream."""
import pytest
import torch

from gpu_util import MoeFixture, pack_gpu, say
from group_quantized_moe_dsq_amd import dsq, synth

pytestmark = pytest.mark.gpu


def inputs(shape, seed):
    return synth.normal(shape, 1.0, 9, synth.X, seed, device="cuda")


def test_two_streams_match_sequential():
    fx = MoeFixture(16, 512, 256, 4, 64, seed=9, bias_std=0.5)
    k = 4
    lay = fx.layer(k)
    H, I, E = fx.H, fx.I, fx.E
    N, K = 512, 2048
    W = pack_gpu(synth.normal((N, K), 0.02, 9, synth.W, 1, device="cuda"), 8, 128)

    # one job per (stream, round): the MoE layer at T = 1 and T = 40, the
    # bf16 split-K GEMM, the FP32 grouped GEMM and the GEMV, each on its own
    # inputs, outputs and workspace
    def make_jobs(tag):
        jobs = []
        for r, (T, math) in enumerate([(1, dsq.MATH_FP32), (40, dsq.MATH_FP32),
                                       (64, dsq.MATH_BF16_MFMA)]):
            X = inputs((T, H), 1000 * tag + r)
            Y = torch.empty((T, H), device="cuda")
            ws = torch.empty(dsq.moe_workspace_bytes(T, E, k, H, I, math) + 256,
                             dtype=torch.uint8, device="cuda")
            jobs.append((f"moe T={T}", lambda X=X, Y=Y, ws=ws, math=math:
                         dsq.moe_ffn(lay, X, math=math, Y=Y, workspace=ws), Y))
        for M, math in [(64, dsq.MATH_BF16_MFMA), (8, dsq.MATH_FP32)]:
            X = inputs((M, K), 1000 * tag + 10 + M)
            Y = torch.empty((M, N), device="cuda")
            ws = torch.empty(dsq.gemm_workspace_bytes(M, N, K, math) + 256, dtype=torch.uint8,
                             device="cuda")
            jobs.append((f"gemm M={M}", lambda X=X, Y=Y, ws=ws, math=math:
                         dsq.gemm(W, X, Y, math=math, workspace=ws), Y))
        x = inputs((K,), 1000 * tag + 99)
        y = torch.empty(N, device="cuda")
        jobs.append(("gemv", lambda x=x, y=y: dsq.gemv(W, x, y), y))
        return jobs

    jobs = [make_jobs(0), make_jobs(1)]
    torch.cuda.synchronize()
    # sequential reference on the current stream
    refs = []
    for js in jobs:
        for name, call, out in js:
            call()
            torch.cuda.synchronize()
            refs.append(out.clone())
    # the same jobs interleaved on two streams, three times over
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        say(f"two streams, pass {rep}")
        for js in jobs:
            for _, _, out in js:
                out.fill_(float("nan"))
        torch.cuda.synchronize()
        for i in range(len(jobs[0])):
            for j in (0, 1):
                with torch.cuda.stream(s[j]):
                    jobs[j][i][1]()
        torch.cuda.synchronize()
        n = 0
        for js in jobs:
            for name, _, out in js:
                assert torch.equal(out, refs[n]), f"{name}: two-stream result differs (pass {rep})"
                n += 1
