"""Host-side pieces of bench.py (CPU): the strict top-10 check it reports
beside the CPU oracle agrees with the test suite's, and a multi-GPU request
is refused with a message, before anything touches a GPU."""
import json
import os
import subprocess
import sys

import numpy as np

from parity import top10_strict_swaps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_top10_matches_test_suite():
    base = np.linspace(1.0, 0.0, 100)
    same = base.copy()
    swapped = base.copy()
    swapped[[3, 4]] = swapped[[4, 3]]       # inside the top ten
    below = base.copy()
    below[[20, 21]] = below[[21, 20]]       # below the top ten
    edge = base.copy()
    edge[[9, 10]] = edge[[10, 9]]           # the tenth and eleventh trade places
    for got, want in ((same, 0), (swapped, 1), (below, 0), (edge, 1)):
        assert bench.strict_top10_swaps(got, base) == want
        assert (top10_strict_swaps(got, base) > 0) == bool(want)
    rng = np.random.default_rng(5)
    for _ in range(200):
        ref = rng.standard_normal(100)
        got = ref + rng.standard_normal(100) * rng.choice([0.0, 1e-3, 3e-2, 0.3])
        assert bench.strict_top10_swaps(got, ref) == int(top10_strict_swaps(got, ref) > 0)


def test_multi_gpu_request_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
