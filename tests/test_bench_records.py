"""bench.py's use of the committed rocprofv3 summaries (CPU only): the record a workload's
line takes its traffic from is the fused kernel's own summary of that workload -- not a
GEMM summary whose file name ends with the workload its A operand came from, nor a
dequantization summary -- and the GEMM lookup finds the GEMM summaries by product."""
import glob
import json
import os

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FUSED = {"generic", "mfma_small", "mfma_wide1", "mfma_wide2", "mfma_wide2t", "mfma_wide1s"}


def _records():
    out = []
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("machine-readable:"):
                    out.append((os.path.basename(f), json.loads(line.split(":", 1)[1])))
    return out


def test_every_summary_has_a_machine_readable_record():
    files = glob.glob(os.path.join(ROOT, "profiles", "*.md"))
    assert files and len(_records()) == len(files)


def test_workload_lookup_takes_the_fused_kernels_own_summary():
    # (a summary whose kernel has changed since is not used: then the lookup gives None)
    for key, w in synth.WORKLOADS.items():
        info = bench.profile_info(w)
        assert info is None or (info["kernel"] in FUSED and info["workload"] == w.name), (key, info)
        for k in FUSED:  # a lookup for one kernel never returns another kernel's summary
            ik = bench.profile_info(w, kernel=k)
            assert ik is None or (ik["kernel"] == k and ik["workload"] == w.name), (key, k, ik)
        deq = bench.profile_info(w, "dequant")
        assert deq is None or (deq["kernel"] == "dequant" and deq["workload"] == w.name), (key, deq)


def test_gemm_summaries_are_found_by_product():
    for f, r in _records():
        if "product" in r:
            assert r["kernel"] in ("mx_gemm_kernel", "int4_gemm_kernel") and "workload" not in r, f
