"""Write the oracle's expected scores for the GPU parity tests at the 0.6B shape.

Everything here comes from the float64 oracle (``oracle/``) and the seeded
input generators (``synth/``): no value is read from the HIP library.  Run from
the repository root on the CPU:

    python tests/golden/make_golden.py            # every file
    python tests/golden/make_golden.py stress     # one of: stress, c64

Files (JSON, scores as float64 repr):
  oracle_stress_subset.json  the L = 4096, K = 512 stress request (workload 5,
      request 0): candidates 0, 131, 300 and 511 scored by oracle_mis on their
      own.  Candidates never see each other, so these equal the full-K
      packed scores ("DuoLM: Fast and Effective Personalized Recommendation
      with Language Models", 研究动机: the identity s^MIS = s).
  oracle_c64_batch.json  the first 64 requests of the C = 64 x K = 100 headline
      pool (workload 3), every candidate: 6,400 scores.

The inputs are the 0.6B-shaped ranker of seed 0 with its item table exported
by the oracle from the seeded encoder outputs (rho = RMS of the token
embedding, gain 1, epsilon 1e-6).
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import OracleModel, export_table, oracle_mis, reference_scale, widen_bf16  # noqa: E402

STRESS_PICK = [0, 131, 300, 511]
C64_REQUESTS = 64


def model_06b():
    cfg = synth.QWEN3_0P6B
    w = synth.make_weights(cfg, seed=0)
    a = synth.table_encoder_outputs(cfg)
    rho = reference_scale(widen_bf16(w["embed"]))
    D = np.empty(a.shape, np.uint16)
    for i in range(0, a.shape[0], 16384):
        D[i:i + 16384] = export_table(a[i:i + 16384], rho, synth.TABLE_GAMMA, synth.TABLE_EPS)
    return cfg, OracleModel.from_arrays(cfg, w, D)


def _write(name, obj):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(obj, f, indent=1)
        f.write("\n")


def stress(cfg, model):
    (req,) = synth.make_requests(5, cfg, n_requests=1)
    t0 = time.time()
    s = oracle_mis(model, req.prefix, req.cands[STRESS_PICK])
    _write("oracle_stress_subset.json", {
        "what": "oracle_mis scores of a candidate subset of the L = 4096, K = 512 stress request",
        "workload": "0.6B-shaped ranker seed 0; synth workload 5 request 0 (16 instruction ids + 60 x (marker, "
                    "VID, 66 feedback ids)); item table exported by the oracle",
        "made_by": "python tests/golden/make_golden.py stress",
        "L": int(req.L), "K": int(req.K), "candidates": STRESS_PICK,
        "scores": [float(x) for x in s],
    })
    print(f"stress: {time.time() - t0:.1f} s", flush=True)


def c64(cfg, model):
    reqs = synth.make_requests(3, cfg, n_requests=C64_REQUESTS)
    t0 = time.time()
    scores = []
    for i, r in enumerate(reqs):
        scores.append([float(x) for x in oracle_mis(model, r.prefix, r.cands)])
        if i % 8 == 7:
            print(f"c64: {i + 1} requests, {time.time() - t0:.1f} s", flush=True)
    _write("oracle_c64_batch.json", {
        "what": "oracle_mis scores of every candidate of the first 64 headline requests",
        "workload": "0.6B-shaped ranker seed 0; synth workload 3 (C = 64, K = 100, varlen prefixes), requests "
                    "0..63 of the seeded pool; item table exported by the oracle",
        "made_by": "python tests/golden/make_golden.py c64",
        "prefix_len": [int(r.L) for r in reqs],
        "scores": scores,
    })


def main():
    which = sys.argv[1:] or ["stress", "c64"]
    cfg, model = model_06b()
    for w in which:
        {"stress": stress, "c64": c64}[w](cfg, model)


if __name__ == "__main__":
    main()
