"""The int8 per-channel composite without a workspace, against the same
composite with a caller workspace: two calls in a row (the second smaller,
so it runs over what the first left in the library's scratch), every
output byte-equal, and the smaller one also against the oracle."""
import numpy as np
import pytest

import block_scaled_precision_blockwise_amd as bsq
import synth
from oracle import matmul as OM
from oracle import quantize as OQ

from gpu_helpers import assert_bytes_equal, empty, filled, host, say, to_dev

pytestmark = pytest.mark.gpu


def _outs(B, Din, Dout):
    import torch
    return (filled((Din, Dout), torch.int8, 0x55), filled((Dout,), torch.float32, float("nan")),
            filled((B, Din), torch.int8, 0x55), filled((B,), torch.float32, float("nan")),
            filled((B, Dout), torch.float32, float("nan")))


def _both(B, Din, Dout, seed):
    import torch
    x, w = synth.int8_workload(B, Din, Dout, seed, seed + 1, zero_rows=(1, 7), zero_cols=(0, 3))
    dx, dw = to_dev(x), to_dev(w)
    ref = _outs(B, Din, Dout)
    work = empty((max(bsq.bsq_int8_workspace_bytes(Din, Dout), 16),), torch.uint8)
    bsq.bsq_int8_per_channel_matmul(dx, dw, *ref, work)
    got = _outs(B, Din, Dout)
    bsq.bsq_int8_per_channel_matmul_noalloc(dx, dw, *got)
    names = ("w_q", "w_scales", "x_q", "x_scales", "y")
    for n, g, r in zip(names, got, ref):
        hg, hr = host(g), host(r)
        if hg.dtype == np.float32:
            hg, hr = hg.view(np.uint32), hr.view(np.uint32)
        assert_bytes_equal(hg, hr, n)
    return x, w, [host(t) for t in got]


def test_int8_noalloc_matches_the_workspace_call_twice():
    say("int8 no-alloc, first call: the largest the scratch holds", 2048, 4096, 4096)
    assert bsq.bsq_int8_noalloc_max_bytes() >= 4096 * 4096
    _both(2048, 4096, 4096, 10)
    say("int8 no-alloc, second call: smaller, over the first call's scratch", 300, 384, 272)
    x, w, (wq, ws, xq, xs, y) = _both(300, 384, 272, 20)
    rxq, rxs = OQ.int8_rows(x)
    rwq, rws = OQ.int8_cols(w)
    a, y64, y32 = OM.int8_matmul(rxq, rwq, rxs, rws)
    assert_bytes_equal(xq, rxq, "x codes vs oracle")
    assert_bytes_equal(wq, rwq, "w codes vs oracle")
    assert_bytes_equal(y.view(np.uint32), y32.view(np.uint32), "y vs oracle")


def test_int8_noalloc_refuses_more_than_its_scratch():
    import torch
    B, Din, Dout = 4, 4096, 4112
    say("int8 no-alloc, too large", B, Din, Dout)
    with pytest.raises(NotImplementedError):
        bsq.bsq_int8_per_channel_matmul_noalloc(empty((B, Din), torch.float32), empty((Din, Dout), torch.float32),
                                                *_outs(B, Din, Dout))
