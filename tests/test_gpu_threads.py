"""Calls on distinct executors from several host threads at once, each thread on its own
stream: every output equals that of the same call made alone (the C ABI keeps no state
shared between executors; the 256 x 256 per-token kernel's slice counter lives in each
call's own workspace).  Two's-complement int4 per token on M = N = 256 (slice tickets) and
MXFP4 per group on M = 64, N = 128 run side by side."""
import threading

import numpy as np
import pytest
import torch

import flatquant_transform_quant_amd as fq
import synth
from gpu_util import DEV, fetch, run_lib, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(key, K, seed):
    w = synth.WORKLOADS[key]
    x, p1, p2 = synth.make_inputs(w, seed, seed + K)  # slices seed .. seed + K - 1
    xd, p1d = to_dev(x, w.dtype), to_dev(p1, w.dtype)
    p2d = to_dev(p2, w.dtype) if p2 is not None else None
    return w, xd, p1d, p2d


def test_concurrent_threads_on_their_own_streams_equal_lone_calls():
    jobs = [_inputs("c4", 300, 11), _inputs("c3", 2048, 12), _inputs("c4", 257, 13), _inputs("c2", 4096, 14)]
    say(f"[gpu] {len(jobs)} threads: " + ", ".join(f"{w.name} K={xd.shape[0]}" for w, xd, _, _ in jobs))
    results = [[] for _ in jobs]
    errors = []
    start = threading.Barrier(len(jobs))

    def work(i):
        try:
            w, xd, p1d, p2d = jobs[i]
            K = xd.shape[0]
            s = torch.cuda.Stream(DEV)
            start.wait()
            for _ in range(4):
                out, sc = fq.empty_outputs(K, w.M, w.N, w.mode, DEV)
                with torch.cuda.stream(s):
                    fq.quantize(xd, p1d, p2d, out, sc, w.mode, w.clip_ratio, w.dst_type_max, stream=s)
                s.synchronize()
                results[i].append(fetch(out, sc, w.mode, K))
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    # the lone calls come after, so that in a fresh process the threads make the first
    # call of each kernel (and of its launcher's cached device figures) together
    refs = [fetch(*run_lib(xd, p1d, p2d, w.mode, w.clip_ratio, w.dst_type_max), w.mode, xd.shape[0])
            for w, xd, p1d, p2d in jobs]
    for i, (ref, got) in enumerate(zip(refs, results)):
        assert len(got) == 4
        for codes, scale in got:
            assert np.array_equal(ref[0], codes), f"job {i}: codes differ"
            assert np.array_equal(ref[1], scale), f"job {i}: scales differ"
