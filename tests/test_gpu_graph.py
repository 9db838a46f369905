"""fq_run captured in a HIP graph (through torch.cuda.graph) and replayed: every replay gives
the same bits as an eager run.  The capture holds kernels only (the pipelined 256 x 256 path
zeroes its slice counter with a kernel, not a memset); between replays the outputs are
overwritten by eager fills, so each replay must write every slice again and the counter must
start from zero on every replay."""
import numpy as np
import pytest
import torch

import flatquant_transform_quant_amd as fq
import synth
from gpu_util import DEV, fetch, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key,K", [("c4", 300), ("c2", 1031), ("c3", 257), ("c5", 40)])
def test_graph_replays_equal_eager(key, K):
    w = synth.WORKLOADS[key]
    say(f"[gpu] graph capture {key} K={K}")
    x, p1, p2 = synth.make_inputs(w, 0, K)
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    p2d = to_dev(p2, w.dtype) if p2 is not None else None
    out, sc = fq.empty_outputs(K, w.M, w.N, w.mode, DEV)
    ex = fq.Executor(xd, p1d, p2d, out, sc, w.mode, w.clip_ratio, w.dst_type_max)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager runs first (one-time lookups happen outside the capture)
        ex.run(side)
        ex.run(side)
    torch.cuda.synchronize()
    ref = fetch(out, sc, w.mode, K)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ex.run()
    for rep in range(3):
        out.view(torch.uint8).fill_(0xEE)
        sc.view(torch.uint8).fill_(0xEE)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = fetch(out, sc, w.mode, K)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), f"{key} replay {rep}"
    del g
    ex.destroy()
