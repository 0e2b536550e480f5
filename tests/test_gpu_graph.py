"""HIP graph capture of the hot path.  The library only enqueues kernels on
the caller's stream (no allocation, copy, memset or synchronisation), so a
step can be captured once and replayed.  Each graph is replayed several
times on new inputs copied into its static buffers, with eager work and
synchronisations between replays, and every replay must give the eager
path's bytes."""
import numpy as np
import pytest

import block_scaled_precision_blockwise_amd as bsq
import synth

from gpu_helpers import assert_bytes_equal, empty, host, say, to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def test_graph_replays_the_blockwise_step():
    """1x128 activation quantizer, 128x128 weight quantizer and the GEMM,
    captured as one graph: at 1024 x 2048 x 2048 the GEMM runs the split-K
    kernel, at 2048 x 4096 x 4096 the big-tile kernel."""
    torch = _torch()
    for (M, N, K) in ((1024, 2048, 2048), (2048, 4096, 4096)):
        say("graph blockwise step", M, N, K)
        a = empty((M, K), torch.float32)
        b = empty((N, K), torch.float32)
        aq = empty((M, K), torch.uint8)
        bq = empty((N, K), torch.uint8)
        sa = empty((M, K // 128), torch.float32)
        sb = empty((N // 128, K // 128), torch.float32)
        y = empty((M, N), torch.float32)

        def step():
            bsq.bsq_quant_fp8_rowblock(a, aq, sa, 128)
            bsq.bsq_quant_fp8_tile(b, bq, sb, 128, 128)
            bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)

        a.copy_(to_dev(synth.randn_f32((M, K), 900)))
        b.copy_(to_dev(synth.randn_f32((N, K), 901)))
        step()  # warm-up outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for rep in range(3):
            a32 = synth.randn_f32((M, K), 910 + 2 * rep)
            b32 = synth.randn_f32((N, K), 911 + 2 * rep)
            a.copy_(to_dev(a32))
            b.copy_(to_dev(b32))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = [host(t).copy() for t in (aq, bq, sa, sb, y)]
            # eager on the same inputs, into the same buffers
            junk = torch.randn(1 << 20, device=a.device).sum()  # unrelated eager work
            y.fill_(float("nan"))
            step()
            torch.cuda.synchronize()
            want = [host(t) for t in (aq, bq, sa, sb, y)]
            for name, gt, wt in zip(("aq", "bq", "sa", "sb", "y"), got, want):
                assert_bytes_equal(gt.view(np.uint8) if gt.dtype == np.uint8 else gt.view(np.uint32),
                                   wt.view(np.uint8) if wt.dtype == np.uint8 else wt.view(np.uint32),
                                   f"{name}, replay {rep}")
            del junk
        del g


def test_graph_replays_the_mxfp8_backward():
    """The one-call MXFP8 backward (one quantizer launch, two GEMMs) as a
    graph, replayed on new dY, W, X."""
    torch = _torch()
    M, N, K = 1024, 768, 512
    say("graph mxfp8 backward", M, N, K)
    dY = empty((M, N), torch.bfloat16)
    W = empty((N, K), torch.bfloat16)
    X = empty((M, K), torch.bfloat16)
    dX = empty((M, K), torch.bfloat16)
    dW = empty((N, K), torch.bfloat16)
    ws = empty((bsq.bsq_mxfp8_backward_workspace_bytes(M, N, K),), torch.uint8)

    def step():
        bsq.bsq_mxfp8_backward(dY, W, X, dX, dW, ws)

    def load(seed):
        for t, shp, s in ((dY, (M, N), 0), (W, (N, K), 1), (X, (M, K), 2)):
            t.copy_(to_dev(synth.randn_bf16_bits(shp, seed + s)).view(torch.bfloat16))

    load(920)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        load(930 + 3 * rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(dX).copy(), host(dW).copy()]
        dX.zero_()
        dW.zero_()
        step()
        torch.cuda.synchronize()
        assert_bytes_equal(got[0], host(dX), f"dX, replay {rep}")
        assert_bytes_equal(got[1], host(dW), f"dW, replay {rep}")
    del g
