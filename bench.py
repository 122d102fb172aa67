"""Throughput benchmark of the MIS ranker forward on one MI355X.

Workload: the Qwen3-0.6B-shaped ranker (random init, bf16 weights, 200k-row
fp16 item table exported from synthetic encoder outputs by the library's own
export entry point) scoring batches of C = 64 synthetic requests packed
varlen, K = 100 candidate VIDs each, history of 1/3/5/10 items with
clip(Poisson(40), 5, 120) feedback tokens per item.  One step = one
duolm_score_batch_dev call over 64 requests (embedding gather, 28 decoder
layers, score head), with the packed ids already resident in device memory.
Requests are consumed in order from a seeded pool of 10,000.  Closed loop: the
next call starts when the previous one returns.

Prints one JSON line: scores/s and p99 latency; the roofline of the dominant
kernel and of every projection GEMM and of candidate-branch attention (timed
live with HIP events on the launching stream); the pages' comparison points
measured here (one-request latency, MIS against independent scoring at C = 1
and C = 64, graph replay against eager launch at C = 1, 8 and 64); an open-loop
Poisson run; and the CPU oracle's rate on bounded samples, with the GPU's
scores of the oracle's sample requests compared against it (largest relative
error, and requests whose top ten candidates are not the oracle's, in order).

Before each phase a 16-byte copy kernel (k_copy) is launched as a marker, so
that a rocprofv3 kernel trace of this run can be cut into phases (python -m
shared_prefix_scoring_amd.rocprof_summary trace DIR): 1 the serving timed
region, 2 a one-lane eager warm-up, 3 the one-lane eager timed region (the
GEMM rooflines), 4 a warm-up of the split-attention launches, 5 the
branch-attention timing, then the comparison points.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "candidate scores/sec on 1 MI355X (0.6B ranker, K=100, C=64); p99 ms"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# The pages' figures on one H100 (trained model, Amazon Books, 100 candidates
# per request; "DuoLM: Fast and Effective Personalized Recommendation with
# Language Models", 实验结果 and the execution-mode ablation row of its results
# table): context only, other hardware and data.
PAGES = {"scores_per_s_c64": 26404.0, "scores_per_s_c1": 8870.0, "p99_ms_c1": 12.35, "p99_ms_c64": 536.9,
         "independent_scores_per_s_c64": 851.48, "mis_gain_c1": 4.81, "mis_gain_c64": 29.3,
         "graph_gain_c1": 3.54, "graph_gain_c64": 1.06}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def src_hash(*names):
    from shared_prefix_scoring_amd.rocprof_summary import code_hash
    return code_hash(names)


GEMM_SRC = ("k_gemm.hip", "common.h", "launch.h")
ATTN_SRC = ("k_attn.hip", "common.h", "launch.h")


def load_ranker(cfg, w):
    """The ranker with its item table made by the library's export entry point
    from the seeded encoder outputs (rho from the library's reference scale)."""
    import torch
    import shared_prefix_scoring_amd as spa
    import synth
    ranker = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    da = torch.from_numpy(synth.table_encoder_outputs(cfg)).cuda()
    ranker.export_vid_table(da.data_ptr(), spa.DUOLM_DTYPE_F32, cfg.n_vid, ranker.reference_scale(),
                            synth.TABLE_GAMMA, synth.TABLE_EPS)
    del da
    torch.cuda.empty_cache()
    return ranker


def host_table(ranker, cfg):
    """The item table's rows on the host (for requests that ship their item
    vectors inline), made by the library's export entry point."""
    import torch
    import shared_prefix_scoring_amd as spa
    import synth
    da = torch.from_numpy(synth.table_encoder_outputs(cfg)).cuda()
    dz = torch.empty((cfg.n_vid, cfg.d_model), dtype=torch.int16, device="cuda")
    spa.duolm_export_item_vectors(da.data_ptr(), spa.DUOLM_DTYPE_F32, cfg.n_vid, cfg.d_model,
                                  ranker.reference_scale(), synth.TABLE_GAMMA, synth.TABLE_EPS, dz.data_ptr())
    torch.cuda.synchronize()
    return dz.cpu().numpy().view(np.uint16)


def host_cpu():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return {"model": model, "os_cpu_count": os.cpu_count(), "blas_threads": blas}


def strict_top10_swaps(got, ref):
    """1 if the GPU's ten best candidates, in order, differ from the oracle's."""
    g = np.argsort(-np.asarray(got, np.float64), kind="stable")[:10]
    r = np.argsort(-np.asarray(ref, np.float64), kind="stable")[:10]
    return int(not np.array_equal(g, r))


def cpu_baseline(cfg, w, pool, budget_s, ranker=None):
    """The float64 oracle as written (untuned), on the host cores:
      - value: consecutive requests of the headline pool until about budget_s
        of wall time has been spent;
      - the one-request workload (L = 452, K = 100), five repeats;
      - brute-force independent scoring (one causal forward per candidate):
        the tiny workload in full, and a stated subset of the one-request
        workload's candidates (the full request is ~100x the subset);
      - with `ranker`, the GPU's scores of the sampled requests against the
        oracle's (gpu_vs_oracle).
    The oracle's item table is its own export of the same encoder outputs;
    building it and the oracle's weights is not timed."""
    import synth
    from oracle import OracleModel, brute_force_independent, export_table, oracle_mis, reference_scale, widen_bf16
    a = synth.table_encoder_outputs(cfg)
    rho = reference_scale(widen_bf16(w["embed"]))
    D = np.empty(a.shape, np.uint16)
    for i in range(0, a.shape[0], 16384):
        D[i:i + 16384] = export_table(a[i:i + 16384], rho, synth.TABLE_GAMMA, synth.TABLE_EPS)
    del a
    model = OracleModel.from_arrays(cfg, w, D)
    hc = host_cpu()
    n_scores, n_req = 0, 0
    refs = []
    t0 = time.perf_counter()
    for r in pool:
        refs.append(oracle_mis(model, r.prefix, r.cands))
        n_scores += r.K
        n_req += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    out = {"value": n_scores / dt, "unit": "candidate scores/s", "cores": hc["blas_threads"], "kind": "oracle",
           "sample": f"{n_req} consecutive requests ({n_scores} candidate scores) of the headline pool, one at a "
                     f"time, float64 NumPy, {dt:.1f} s", "host": hc}
    if ranker is not None:
        # the same requests scored on the GPU (one call) against the oracle's
        # scores: |error| relative to max(1, |s|), and requests whose top ten
        # (in order) differ from the oracle's
        got = ranker.score([(r.prefix, r.cands) for r in pool[:n_req]])
        errs, swaps, o = [], 0, 0
        for r, ref in zip(pool[:n_req], refs):
            g = got[o:o + r.K]
            o += r.K
            errs.append(float(np.max(np.abs(g - ref) / np.maximum(1.0, np.abs(ref)))))
            swaps += strict_top10_swaps(g, ref)
        out["gpu_vs_oracle"] = {"requests": n_req, "max_rel_err": round(max(errs), 5),
                                "requests_with_strict_top10_swap": swaps,
                                "tolerance": "2e-2 relative to max(1, |s|)"}
    (r2,) = synth.make_requests(2, cfg)
    ts = []
    for _ in range(5):
        t1 = time.perf_counter()
        oracle_mis(model, r2.prefix, r2.cands)
        ts.append(time.perf_counter() - t1)
    out["one_request_L452_K100"] = {"repeats": 5, "s_per_request_median": round(float(np.median(ts)), 3),
                                    "scores_per_s": round(r2.K / float(np.median(ts)), 1)}
    pick = [0, 1]
    t1 = time.perf_counter()
    brute_force_independent(model, r2.prefix, r2.cands, which=pick)
    bf = (time.perf_counter() - t1) / len(pick)
    out["brute_force_L452"] = {"sample": f"candidates {pick} of the one-request workload", "s_per_candidate": round(bf, 3),
                               "scores_per_s": round(1.0 / bf, 3),
                               "s_per_request_extrapolated": round(bf * r2.K, 1)}
    tcfg = synth.TINY
    tw = synth.make_weights(tcfg, seed=0)
    tmodel = OracleModel.from_arrays(tcfg, tw, synth.make_vid_table(tcfg))
    (rt,) = synth.make_requests(1, tcfg)
    t1 = time.perf_counter()
    brute_force_independent(tmodel, rt.prefix, rt.cands)
    tb = time.perf_counter() - t1
    t1 = time.perf_counter()
    oracle_mis(tmodel, rt.prefix, rt.cands)
    tm = time.perf_counter() - t1
    out["tiny_L48_K8"] = {"brute_force_s": round(tb, 4), "oracle_mis_s": round(tm, 4)}
    return out


def open_loop(ranker, pack, rate, n_requests, seed, C, use_graph, stream):
    """Poisson arrivals at `rate` requests/s; the server takes up to C queued
    requests per call.  Each call runs the whole serving path from structured
    requests (item VIDs, feedback ids, candidate VIDs): the host packer
    assembles the ranker input, ids go up from the page-locked staging buffer,
    scores come back the same way (PCIe-inclusive).  `pack` holds the pool's
    requests, marshalled once.  Returns per-request latencies (completion -
    arrival) in ms and the wall time."""
    import synth
    import shared_prefix_scoring_amd as spa
    arrivals = synth.poisson_arrivals(n_requests, rate, seed)
    lat = np.empty(n_requests)
    buf = np.empty(spa.duolm_packed_size(pack), dtype=np.int32)
    t0 = time.perf_counter()
    nxt = 0
    while nxt < n_requests:
        now = time.perf_counter() - t0
        if arrivals[nxt] > now:
            time.sleep(arrivals[nxt] - now)
            now = time.perf_counter() - t0
        end = nxt
        while end < n_requests and end - nxt < C and arrivals[end] <= now:
            end += 1
        start = nxt % pack.n
        cnt = min(end - nxt, pack.n - start)
        ids, L, K, M = spa.duolm_pack_requests(pack, ids=buf, start=start, count=cnt)
        ranker.score_packed(L, K, M, ids, use_graph=use_graph, stream=stream)
        done = time.perf_counter() - t0
        lat[nxt:nxt + cnt] = (done - arrivals[nxt:nxt + cnt]) * 1e3
        nxt += cnt
    return lat, time.perf_counter() - t0


def pack_pool(pool, cid, cfg):
    import shared_prefix_scoring_amd as spa
    import synth
    marker, instr = synth.template(cid, cfg)
    return spa.PackInput(instr, marker, [(r.items, r.feedback, r.cands, r.m, r.m) for r in pool])


def bench_packer(ranker, cfg):
    """The host input packer ([digest] 实验结果: the pages' single-process CPU
    input compilation failed 1,491 times at 200 requests/s).  Packing rate of
    the headline pool (10,000 requests, C = 64 per call) on 1 and 8 threads;
    the host serving path (pack + score from page-locked staging) against the
    device entry point; and a 200 requests/s Poisson open loop."""
    import torch
    import shared_prefix_scoring_amd as spa
    import synth
    pool = synth.make_requests(3, cfg)
    pack = pack_pool(pool, 3, cfg)
    buf = np.empty(spa.duolm_packed_size(pack), dtype=np.int32)
    out = {}
    for nt in (1, 8):
        t0 = time.perf_counter()
        for s in range(0, pack.n, 64):
            spa.duolm_pack_requests(pack, n_threads=nt, ids=buf, start=s, count=min(64, pack.n - s))
        dt = time.perf_counter() - t0
        out[f"pack_requests_per_s_{nt}thr"] = round(pack.n / dt)
    t0 = time.perf_counter()
    spa.duolm_pack_requests(pack, n_threads=8, ids=buf)
    dt = time.perf_counter() - t0
    out["pack_10k_one_call_8thr_ms"] = round(dt * 1e3, 2)
    stream = torch.cuda.current_stream().cuda_stream
    calls = 20
    for c in range(calls):  # capture every shape bucket the timed calls use
        ids, L, K, M = spa.duolm_pack_requests(pack, ids=buf, start=64 * c, count=64)
        ranker.score_packed(L, K, M, ids, stream=stream)
    t0 = time.perf_counter()
    for c in range(calls):
        ids, L, K, M = spa.duolm_pack_requests(pack, ids=buf, start=64 * c, count=64)
        ranker.score_packed(L, K, M, ids, stream=stream)
    host_ms = (time.perf_counter() - t0) * 1e3 / calls
    dev = []
    for c in range(calls):
        ids, L, K, M = spa.duolm_pack_requests(pack, ids=buf, start=64 * c, count=64)
        dev.append((torch.from_numpy(ids.copy()).cuda(), L, K, M,
                    torch.empty(int(K.sum()), dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for d_ids, L, K, M, d_out in dev:
        ranker.score_dev(L, K, d_ids.data_ptr(), d_out.data_ptr(), stream=stream, cand_len=M)
    torch.cuda.synchronize()
    dev_ms = (time.perf_counter() - t0) * 1e3 / calls
    out["host_path_call_ms"] = round(host_ms, 3)
    out["device_path_call_ms"] = round(dev_ms, 3)
    lat, wall = open_loop(ranker, pack, 200.0, 2000, 300, 64, True, stream)
    out["open_loop_200rps"] = {"requests": 2000, "p50_ms": round(float(np.percentile(lat, 50)), 2),
                               "p99_ms": round(float(np.percentile(lat, 99)), 2),
                               "achieved_rps": round(2000 / wall, 1)}
    return out


def bench_rating(ranker, cfg, D, C, rounds):
    """Rating-style regime: 256 requests of K=8 at C=8.  Graph replay against
    eager launch (device-resident ids), and VID ids against shipping the
    1024-d fp16 item vectors in the request (host entry point, PCIe-inclusive)."""
    import torch
    import synth
    reqs = synth.make_requests(4, cfg)
    batches = [reqs[i:i + C] for i in range(0, len(reqs), C)]
    stream = torch.cuda.current_stream().cuda_stream
    dev = []
    for b in batches:
        ids, L, K = synth.pack_ids(b)
        dev.append((torch.from_numpy(ids).cuda(), L, K, torch.empty(int(K.sum()), device="cuda")))

    def run_dev(graph):
        for x in dev:
            ranker.score_dev(x[1], x[2], x[0].data_ptr(), x[3].data_ptr(), use_graph=graph, stream=stream)

    def as_ids(b):
        return [(r.prefix, r.cands) for r in b]

    def as_inline(b):
        out = []
        for r in b:
            ids = np.concatenate([r.prefix, r.cands])
            out.append((r.prefix, r.cands, D[ids[ids >= cfg.vocab] - cfg.vocab]))
        return out

    host_ids = [as_ids(b) for b in batches]
    host_inl = [as_inline(b) for b in batches]
    res = {}
    for name, fn in [("graph_dev", lambda: run_dev(True)), ("eager_dev", lambda: run_dev(False)),
                     ("ids_host", lambda: [ranker.score(h, stream=stream) for h in host_ids]),
                     ("inline_host", lambda: [ranker.score(h, stream=stream) for h in host_inl])]:
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(rounds):
            fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / rounds
        res[name] = {"requests_per_s": round(len(reqs) / dt, 1), "scores_per_s": round(len(reqs) * 8 / dt, 1),
                     "ms_per_call": round(dt / len(batches) * 1e3, 3)}
    ids_bytes = np.mean([4 * (r.L + r.K) for r in reqs])
    vec_bytes = np.mean([4 * (r.L + r.K) + 2 * cfg.d_model * int(np.sum(np.concatenate([r.prefix, r.cands]) >= cfg.vocab))
                         for r in reqs])
    res["payload_bytes_per_request"] = {"ids": round(float(ids_bytes), 1), "inline_vectors": round(float(vec_bytes), 1),
                                        "cut": round(1 - float(ids_bytes / vec_bytes), 4)}
    res["launches_per_call"] = "1 graph (graph) or 226 kernels (eager)"
    return res


def bench_latency(ranker, cfg, calls):
    """One request at a time (L = 452, K = 100): per-call latency with graph
    replay and eagerly, device-resident ids and the host entry point."""
    import torch
    import synth
    import shared_prefix_scoring_amd as spa
    (req,) = synth.make_requests(2, cfg)
    ids, L, K = synth.pack_ids([req])
    d_ids = torch.from_numpy(ids).cuda()
    d_s = torch.empty(int(K.sum()), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    mark_src = torch.zeros(4, dtype=torch.int32, device="cuda")
    mark_dst = torch.empty_like(mark_src)
    res = {"request": {"L": int(req.L), "K": int(req.K)}}
    for name, fn in [
        ("graph_dev", lambda: ranker.score_dev(L, K, d_ids.data_ptr(), d_s.data_ptr(), use_graph=True, stream=stream)),
        ("eager_dev", lambda: ranker.score_dev(L, K, d_ids.data_ptr(), d_s.data_ptr(), use_graph=False, stream=stream)),
        ("graph_host", lambda: ranker.score([(req.prefix, req.cands)], use_graph=True, stream=stream)),
    ]:
        # a 16-byte copy kernel marks the phase boundary in a kernel trace
        spa.duolm_copy_device(mark_dst.data_ptr(), mark_src.data_ptr(), 16, stream)
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(calls):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            t.append((time.perf_counter() - t0) * 1e3)
        t = np.array(t)
        res[name] = {"p50_ms": round(float(np.median(t)), 3), "p99_ms": round(float(np.percentile(t, 99)), 3),
                     "scores_per_s": round(float(req.K / np.median(t) * 1e3), 1)}
    return res


def bench_multivec(ranker, cfg, rounds):
    """Items of m = 8 vectors (every history item and candidate spans 8 VID
    rows; a candidate is an 8-row causal branch), candidate counts cycled over
    {5, 20, 50, 100}: 256 requests as calls of C = 8 and of C = 1."""
    import torch
    import synth
    reqs = synth.make_requests(6, cfg)
    stream = torch.cuda.current_stream().cuda_stream
    res = {"m": 8, "requests": len(reqs)}
    for C in (1, 8):
        calls = []
        for i in range(0, len(reqs), C):
            b = reqs[i:i + C]
            ids, L, K = synth.pack_ids(b)
            calls.append((torch.from_numpy(ids).cuda(), L, K, torch.empty(int(K.sum()), device="cuda"),
                          max(r.K for r in b)))

        def run(x):
            ranker.score_dev(x[1], x[2], x[0].data_ptr(), x[3].data_ptr(), use_graph=True, stream=stream,
                             cand_len=8)

        for x in calls:
            run(x)
        torch.cuda.synchronize()
        lat, lat100 = [], []
        t0 = time.perf_counter()
        for _ in range(rounds):
            for x in calls:
                t1 = time.perf_counter()
                run(x)
                torch.cuda.synchronize()
                dt = (time.perf_counter() - t1) * 1e3
                lat.append(dt)
                if C == 1 and x[4] == 100:
                    lat100.append(dt)
        wall = time.perf_counter() - t0
        n_scores = sum(int(x[2].sum()) for x in calls) * rounds
        res[f"C{C}"] = {"requests_per_s": round(len(reqs) * rounds / wall, 1),
                        "scores_per_s": round(n_scores / wall, 1),
                        "call_p50_ms": round(float(np.median(lat)), 3)}
        if lat100:
            res[f"C{C}"]["p50_ms_N100"] = round(float(np.median(lat100)), 3)
    return res


def bench_stress(ranker, cfg, n_req, n_ind):
    """L=4096, K=512: MIS over n_req requests in one call, against independent
    scoring (prefix replicated per candidate, full causal forward) of the
    first n_ind candidates of the first two requests (median call times)."""
    import torch
    import synth
    reqs = synth.make_requests(5, cfg, n_requests=n_req)
    mis_in = [(r.prefix, r.cands) for r in reqs]
    ranker.score(mis_in)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):  # median of five calls
        t0 = time.perf_counter()
        mis = ranker.score(mis_in)
        ts.append(time.perf_counter() - t0)
    t_mis = float(np.median(ts))
    ind_in = [(r.prefix, r.cands[:n_ind]) for r in reqs[:2]]
    ranker.score(ind_in, mode=1)
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        ind = ranker.score(ind_in, mode=1)
        ts.append(time.perf_counter() - t0)
    t_ind = float(np.median(ts))
    ref = np.concatenate([mis[i * 512:i * 512 + n_ind] for i in range(2)])
    rate_mis = len(mis) / t_mis
    rate_ind = len(ind) / t_ind
    return {"mis": {"requests": n_req, "rows": int(sum(r.L + r.K for r in reqs)), "seconds": round(t_mis, 3),
                    "scores_per_s": round(rate_mis, 1)},
            "independent": {"sample": f"first {n_ind} candidates of 2 requests", "rows": 2 * n_ind * 4097,
                            "seconds": round(t_ind, 3), "scores_per_s": round(rate_ind, 1)},
            "mis_speedup": round(rate_mis / rate_ind, 1),
            "max_abs_diff_mis_vs_independent": float(np.max(np.abs(ref - ind)))}


def bench_export(ranker, cfg, reps):
    """Offline export of the item table: 200,000 encoder outputs of d_model
    values into FP16 rows (RMS normalise, reference scale, gain), input already
    in HBM; plus the reference scale over the token embedding.  HBM-bound:
    algorithmic bytes = rows * d * (input bytes + 2)."""
    import torch
    import shared_prefix_scoring_amd as spa
    import synth
    n, d = 200_000, cfg.d_model
    a32 = synth.encoder_outputs(n, d, seed=11)
    rho = ranker.reference_scale()
    out = {"rows": n, "d": d, "rho": rho}
    stream = torch.cuda.current_stream().cuda_stream
    dz = torch.empty(n * d, dtype=torch.int16, device="cuda")
    for name, dt, host in (("f32", spa.DUOLM_DTYPE_F32, a32),
                           ("bf16", spa.DUOLM_DTYPE_BF16, synth.f32_to_bf16_bits(a32))):
        da = torch.from_numpy(host.view(np.uint8).reshape(-1)).cuda()
        for _ in range(3):
            spa.duolm_export_item_vectors(da.data_ptr(), dt, n, d, rho, 0.0, 1e-6, dz.data_ptr(), stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            spa.duolm_export_item_vectors(da.data_ptr(), dt, n, d, rho, 0.0, 1e-6, dz.data_ptr(), stream)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = n * d * (host.itemsize + 2)
        out[name] = {"us_per_launch": round(us, 1), "rows_per_s": round(n / us * 1e6),
                     "GBs": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 3)}
        del da
    # attainable streaming rate: a plain 16-byte copy of the same byte count as
    # the fp32 export (819 MB read + 410 MB written ~ 615 MB each way)
    nb = (n * d * 6 // 2) // 16 * 16
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        spa.duolm_copy_device(dst.data_ptr(), src.data_ptr(), nb, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        spa.duolm_copy_device(dst.data_ptr(), src.data_ptr(), nb, stream)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    out["copy_same_bytes"] = {"us_per_launch": round(us, 1), "GBs": round(2 * nb / us / 1e3, 1)}
    del src, dst
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        ranker.reference_scale()
    us = (time.perf_counter() - t0) * 1e6 / reps
    nbytes = cfg.vocab * d * 2
    out["reference_scale"] = {"us_per_call_incl_sync": round(us, 1), "GBs": round(nbytes / us / 1e3, 1)}
    return out


def bench_session(ranker, cfg, steps):
    """In-session incremental personalisation ([digest] 未来方向 (3)): 64 users
    with the headline workload's histories; at every step each user gets one
    new history item (marker, VID, clip(Poisson(40), 5, 120) feedback ids) and
    100 candidates are scored.  Incremental: the session appends the item's
    rows to its cached prefix K/V and scores.  Recompute: the whole prefix is
    prefilled again with the candidates (one-call MIS).  Both return the same
    scores bit for bit (checked)."""
    import synth
    C, K = 64, 100
    users = synth.make_requests(3, cfg, n_requests=C, seed=77)
    marker, _ = synth.template(3, cfg)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(177)))
    V, N = cfg.vocab, cfg.n_vid
    ranker.kv_pool_init(C * (600 + (steps + 3) * 130))
    sess = [ranker.session() for _ in range(C)]
    prefixes = [u.prefix.copy() for u in users]
    ranker.step(sess, prefixes)  # the users' histories so far
    out = {"users": C, "candidates": K, "steps": steps}
    t_inc, t_full, rows_inc, rows_full = 0.0, 0.0, 0, 0
    for step in range(steps + 2):  # two untimed warm-up steps (graph capture)
        new = []
        for _ in range(C):
            f = int(np.clip(rng.poisson(40), 5, 120))
            new.append(np.concatenate([[marker, V + int(rng.integers(0, N))],
                                       rng.integers(0, V, size=f)]).astype(np.int32))
        cands = [(V + rng.choice(N, size=K, replace=False)).astype(np.int32) for _ in range(C)]
        prefixes = [np.concatenate([p, x]) for p, x in zip(prefixes, new)]
        t0 = time.perf_counter()
        got = ranker.step(sess, new, cands)
        t1 = time.perf_counter()
        want = ranker.score(list(zip(prefixes, cands)))
        t2 = time.perf_counter()
        if not np.array_equal(got, want):
            raise RuntimeError("session scores differ from one-call scores")
        if step >= 2:
            t_inc += t1 - t0
            t_full += t2 - t1
            rows_inc += sum(len(x) for x in new) + C * K
            rows_full += sum(len(p) for p in prefixes) + C * K
    for x in sess:
        x.close()
    out["mean_prefix_len_end"] = round(float(np.mean([len(p) for p in prefixes])), 1)
    out["incremental"] = {"ms_per_step": round(t_inc / steps * 1e3, 3), "scores_per_s": round(C * K * steps / t_inc),
                          "rows_per_step": round(rows_inc / steps)}
    out["recompute"] = {"ms_per_step": round(t_full / steps * 1e3, 3), "scores_per_s": round(C * K * steps / t_full),
                        "rows_per_step": round(rows_full / steps)}
    out["speedup"] = round(t_full / t_inc, 2)
    return out


def gemm_roofline(stats, classes, name):
    st = [stats[c] for c in classes if stats[c].launches]
    launches = sum(x.launches for x in st)
    if launches == 0:
        return None
    ms = sum(x.total_ms for x in st)
    flops = sum(x.flops for x in st)
    ach = flops / (ms * 1e-3) / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4), "launches": launches, "avg_launch_ms": round(ms / launches, 4),
            "flops_per_launch": flops / launches, "ms_per_step": ms}


def traffic_from_profile(name, kernel_hash):
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    return t.get("bytes_per_launch") if t.get("kernel_src_hash") == kernel_hash else None


def headline(args, cfg, w, ranker):
    import torch
    import shared_prefix_scoring_amd as spa
    import synth
    log("generating requests")
    pool = synth.make_requests(3, cfg, n_requests=args.pool)
    C = args.concurrency
    n_calls = args.warmup + args.steps
    batches = []
    for i in range(n_calls):
        k = 0 if args.same_batch else i
        reqs = [pool[(k * C + j) % len(pool)] for j in range(C)]
        ids, L, K = synth.pack_ids(reqs)
        batches.append((torch.from_numpy(ids).cuda(), L, K,
                        torch.empty(int(K.sum()), dtype=torch.float32, device="cuda")))
    mark_src = torch.zeros(4, dtype=torch.int32, device="cuda")
    mark_dst = torch.empty_like(mark_src)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
    stream = torch.cuda.current_stream().cuda_stream

    def marker():  # a 16-byte copy kernel: phase boundary in a kernel trace
        spa.duolm_copy_device(mark_dst.data_ptr(), mark_src.data_ptr(), 16, stream)

    def call(b, lanes=0, graph=use_graph, mode=0):
        ranker.score_dev(b[1], b[2], b[0].data_ptr(), b[3].data_ptr(), use_graph=graph, stream=stream,
                         max_lanes=lanes, mode=mode)

    def timed_steps(lanes, graph=use_graph):
        lat = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, n_calls):
            ts = time.perf_counter()
            call(batches[i], lanes, graph)
            lat.append(time.perf_counter() - ts)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, lat

    log("warmup")
    for i in range(args.warmup):
        call(batches[i], args.max_lanes)
    if use_graph:
        # steady state of a serving process: every shape bucket the timed
        # batches fall in has its graphs captured
        for i in range(args.warmup, n_calls):
            call(batches[i], args.max_lanes)
    # phase 1, the timed region: the serving configuration, no kernel timing
    # (a batch this size runs as two concurrent halves, one per execution lane)
    marker()  # phase 1
    dt, lat = timed_steps(args.max_lanes)
    n_scores = sum(int(b[2].sum()) for b in batches[args.warmup:])
    rows = [int(b[1].sum() + b[2].sum()) for b in batches[args.warmup:]]
    value = n_scores / dt
    # phases 2-3: the projection GEMMs timed live with HIP events recorded on
    # the launching stream around every launch, over a second timed region of
    # the same steps run as one eager launch per call, so each kernel has the
    # chip to itself (with two concurrent halves a launch's duration would
    # include time the other half's kernels share the chip; event-record
    # nodes inside a graph add a few more microseconds per launch than events
    # recorded between eager launches)
    log("one-lane timed region (GEMM timing)")
    gemm_classes = ["gemm_qkv", "gemm_o", "gemm_gateup", "gemm_down"]
    ranker.set_profiling(gemm_classes)
    marker()  # phase 2: one-lane warm-up
    for i in range(args.warmup, n_calls):
        call(batches[i], 1, False)
    ranker.set_profiling(gemm_classes)  # reset the counters
    marker()  # phase 3: the one-lane timed region
    dt1, _ = timed_steps(1, graph=False)
    stats = {c: ranker.kernel_stats(c) for c in gemm_classes}
    # phases 4-5: candidate-branch attention, one eager launch per call, its
    # tiles launched on their own (prefix tiles in a launch of their own
    # beside them)
    ranker.set_profiling(["attn_branch"])
    marker()  # phase 4: warm-up of the split-attention launches
    for i in range(args.warmup, min(n_calls, args.warmup + 10)):
        call(batches[i], 1, False)
    ranker.set_profiling(["attn_branch"])
    marker()  # phase 5: the branch-attention timing
    for i in range(args.warmup, min(n_calls, args.warmup + 10)):
        call(batches[i], 1, False)
    torch.cuda.synchronize()
    br = ranker.kernel_stats("attn_branch")
    ranker.set_profiling([])
    if br.launches == 0 or any(st.launches == 0 for st in stats.values()):
        raise RuntimeError("no timed launches recorded for the roofline kernels")
    per = {"all": gemm_roofline(stats, gemm_classes, "k_gemm, all four projections of every layer"),
           "qkv": gemm_roofline(stats, ["gemm_qkv"], "k_gemm, QKV projection (bf16 store)"),
           "o": gemm_roofline(stats, ["gemm_o"], "k_gemm, O projection (+ fp32 residual)"),
           "gateup": gemm_roofline(stats, ["gemm_gateup"], "k_gemm, gate/up projection (+ SwiGLU)"),
           "down": gemm_roofline(stats, ["gemm_down"], "k_gemm, down projection (+ fp32 residual)")}
    # kernels (one template instantiation each at this shape): the residual
    # epilogue GEMM serves both the O and the down projections
    kernels = {"gemm_resid": gemm_roofline(stats, ["gemm_o", "gemm_down"],
                                           "k_gemm residual-epilogue instantiation (O and down projections)"),
               "gemm_gateup": per["gateup"], "gemm_qkv": per["qkv"]}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    roof = dict(kernels[dom])
    roof["traffic"] = traffic_from_profile(dom, src_hash(*GEMM_SRC))
    roof["timed"] = ("a second timed region over the same steps, one eager launch per call (no concurrent halves), "
                     "HIP events recorded on the launching stream around every projection GEMM launch; the dominant "
                     "kernel is the one with the most device time per step")
    roof["ms_per_step"] = round(roof["ms_per_step"] / args.steps, 3)
    for v in per.values():
        v["ms_per_step"] = round(v["ms_per_step"] / args.steps, 3)
    per["qkv"]["traffic"] = traffic_from_profile("gemm_qkv", src_hash(*GEMM_SRC))
    per["gateup"]["traffic"] = traffic_from_profile("gemm_gateup", src_hash(*GEMM_SRC))
    br_ms = br.total_ms / br.launches
    br_bytes = br.bytes / br.launches
    br_ach = br_bytes / (br_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "candidate scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 3),
        "ms_per_step_one_lane_gemm_timed": round(dt1 / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES["scores_per_s_c64"], 3),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-0.6b-shaped ranker, C=64 requests x K=100 candidates, varlen prefixes",
                   "requests_per_step": C, "candidates_per_request": 100,
                   "execution_lanes": "two concurrent halves per call" if args.max_lanes != 1 else "one launch per call",
                   "mean_rows_per_step": round(float(np.mean(rows)), 1), "graph": use_graph,
                   "graphs_primed": use_graph, "inputs": "packed ids resident in HBM",
                   "item_table": "200k x 1024 fp16, exported from seeded encoder outputs by the library"},
        "p99_ms": round(float(np.percentile(np.array(lat) * 1e3, 99)), 3),
        "closed_loop_call_ms": {"p50": round(float(np.percentile(np.array(lat) * 1e3, 50)), 3),
                                "p99": round(float(np.percentile(np.array(lat) * 1e3, 99)), 3)},
        "roofline": roof,
        "gemm_rooflines": per,
        "roofline_branch_attn": {"kernel": "k_attn branch-only instantiation (candidate-branch tiles)", "bound": "hbm",
                                 "timed": "10 eager one-launch calls after the timed regions, branch tiles launched "
                                          "on their own, HIP events recorded on the launching stream around each "
                                          "launch",
                                 "achieved": round(br_ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(br_ach / PEAK_HBM_GBS, 4), "launches": br.launches,
                                 "avg_launch_ms": round(br_ms, 4), "bytes_per_launch": br_bytes,
                                 "traffic": traffic_from_profile("attn_branch", src_hash(*ATTN_SRC))},
    }
    if args.extras:
        out["pages_comparisons"] = comparisons(args, cfg, ranker, batches, lat, marker, stream)
    if args.open_loop > 0:
        log("open-loop Poisson run")
        req_rate = value / 100.0 * 0.9
        pack = pack_pool(pool, 3, cfg)
        # prime the graphs of the batch sizes the open loop will produce, then
        # warm the graph cache as a serving process would be: an untimed open
        # loop of the same rate with other arrivals (another seed), whose
        # batches fall in the shape buckets the timed run mostly meets
        for c in range(1, C + 1):
            ids, L, K, M = spa.duolm_pack_requests(pack, count=c)
            ranker.score_packed(L, K, M, ids, use_graph=use_graph, stream=stream)
        open_loop(ranker, pack, req_rate, args.open_loop // 2, seed=7, C=C, use_graph=use_graph, stream=stream)
        ol_lat, ol_wall = open_loop(ranker, pack, req_rate, args.open_loop, seed=103, C=C,
                                    use_graph=use_graph, stream=stream)
        out["p99_ms"] = round(float(np.percentile(ol_lat, 99)), 3)
        out["open_loop"] = {"arrivals": "Poisson", "rate_req_per_s": round(req_rate, 1),
                            "requests": args.open_loop, "max_batch": C,
                            "p50_ms": round(float(np.percentile(ol_lat, 50)), 3),
                            "p99_ms": out["p99_ms"],
                            "scores_per_s": round(args.open_loop * 100 / ol_wall, 1),
                            "path": "structured requests -> host packer -> page-locked staging -> "
                                    "scores to host (PCIe-inclusive)",
                            "warmup": "an untimed open loop of half as many requests, other arrivals"}
    if args.cpu_baseline_s > 0:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, w, pool, args.cpu_baseline_s, ranker)
    return out


def comparisons(args, cfg, ranker, batches, lat_c64, marker, stream):
    """The pages' comparison points measured on this path: one-request
    latency, MIS against independent scoring (prefix recomputed per
    candidate) at C = 1 and C = 64, graph replay against eager launch at C = 1,
    8 and 64.  The pages' H100 figures ride along as context."""
    import torch
    import synth

    def med_ms(fn, n, warm=2):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(n):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            t.append((time.perf_counter() - t0) * 1e3)
        return np.array(t)

    def dev(reqs):
        ids, L, K = synth.pack_ids(reqs)
        return (torch.from_numpy(ids).cuda(), L, K, torch.empty(int(K.sum()), dtype=torch.float32, device="cuda"))

    def run(b, graph=True, mode=0):
        ranker.score_dev(b[1], b[2], b[0].data_ptr(), b[3].data_ptr(), use_graph=graph, stream=stream, mode=mode)

    out = {}
    log("comparison points: one request (L = 452, K = 100)")
    marker()
    one = dev(synth.make_requests(2, cfg))
    t_g = med_ms(lambda: run(one), 100, warm=5)
    mis1 = one[3].clone()
    t_e = med_ms(lambda: run(one, graph=False), 30)
    t_i = med_ms(lambda: run(one, mode=1), 5)  # leaves the independent scores in one[3]
    out["c1_latency"] = {"p50_ms": round(float(np.median(t_g)), 3), "p99_ms": round(float(np.percentile(t_g, 99)), 3),
                         "scores_per_s": round(100 / float(np.median(t_g)) * 1e3, 1),
                         "pages_h100": {"p99_ms": PAGES["p99_ms_c1"], "scores_per_s": PAGES["scores_per_s_c1"]}}
    out["c1_graph_vs_eager"] = {"graph_ms": round(float(np.median(t_g)), 3), "eager_ms": round(float(np.median(t_e)), 3),
                                "gain": round(float(np.median(t_e) / np.median(t_g)), 3),
                                "pages_h100_gain": PAGES["graph_gain_c1"]}
    out["c1_mis_vs_independent"] = {"mis_ms": round(float(np.median(t_g)), 3),
                                    "independent_ms": round(float(np.median(t_i)), 3),
                                    "gain": round(float(np.median(t_i) / np.median(t_g)), 2),
                                    "max_abs_diff": float((one[3] - mis1).abs().max()),
                                    "pages_h100_gain": PAGES["mis_gain_c1"]}
    log("comparison points: C = 64 (independent scoring and eager launch of one headline batch)")
    marker()
    b0 = batches[args.warmup]
    t_mis = float(np.median(np.array(lat_c64) * 1e3))
    t_ind = med_ms(lambda: run(b0, mode=1), 2, warm=1)
    ind = b0[3].clone()
    run(b0)
    torch.cuda.synchronize()
    t_eag = med_ms(lambda: run(b0, graph=False), 5)
    n = int(b0[2].sum())
    out["c64_mis_vs_independent"] = {
        "mis_ms": round(t_mis, 3), "independent_ms": round(float(np.median(t_ind)), 3),
        "independent_scores_per_s": round(n / float(np.median(t_ind)) * 1e3, 1),
        "gain": round(float(np.median(t_ind)) / t_mis, 2),
        "independent_rows": int(sum((int(l) + 1) * int(k) for l, k in zip(b0[1], b0[2]))),
        "max_abs_diff": float((b0[3] - ind).abs().max()),
        "pages_h100": {"gain": PAGES["mis_gain_c64"], "independent_scores_per_s": PAGES["independent_scores_per_s_c64"]}}
    out["c64_graph_vs_eager"] = {"graph_ms": round(t_mis, 3), "eager_ms": round(float(np.median(t_eag)), 3),
                                 "gain": round(float(np.median(t_eag)) / t_mis, 3),
                                 "pages_h100_gain": PAGES["graph_gain_c64"]}
    log("comparison points: rating regime (C = 8, K = 8)")
    marker()
    rq = synth.make_requests(4, cfg)
    rb = [dev(rq[i:i + 8]) for i in range(0, len(rq), 8)]
    tg = med_ms(lambda: [run(b) for b in rb], 3, warm=1) / len(rb)
    te = med_ms(lambda: [run(b, graph=False) for b in rb], 3, warm=1) / len(rb)
    out["c8_k8_graph_vs_eager"] = {"graph_ms_per_call": round(float(np.median(tg)), 3),
                                   "eager_ms_per_call": round(float(np.median(te)), 3),
                                   "gain": round(float(np.median(te) / np.median(tg)), 3)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--concurrency", type=int, default=64)
    ap.add_argument("--pool", type=int, default=10_000, help="requests in the seeded pool")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--max-lanes", type=int, default=0,
                    help="execution lanes of the timed region (0: library default, two halves for large calls; 1: one)")
    ap.add_argument("--cpu-baseline-s", type=float, default=12.0, help="0 disables the oracle timing")
    ap.add_argument("--open-loop", type=int, default=10_000,
                    help="requests in the Poisson-arrival run (0 disables it)")
    ap.add_argument("--extras", type=int, default=1, help="0 skips the pages' comparison points")
    ap.add_argument("--same-batch", action="store_true",
                    help="every call scores the pool's first 64 requests (counter runs: one geometry per kernel)")
    ap.add_argument("--calib-copy", action="store_true", help="run only the copy kernel (counter calibration)")
    ap.add_argument("--workload", choices=["headline", "latency", "rating", "multivec", "stress", "export", "packer", "session"],
                    default="headline",
                    help="headline: C=64 x K=100 (the metric); latency: one L=452 x K=100 request per call; "
                         "rating: K=8 at C=8, graph vs eager and ids vs inline vectors; multivec: items of 8 "
                         "vectors, K in {5,20,50,100}, C=1 and C=8; stress: L=4096 x K=512, MIS vs independent; "
                         "export: the offline FP16 export of a 200k-row item table; packer: the host input "
                         "packer and the host serving path; session: incremental history appends against "
                         "prefix recompute")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the ranker runs on one GPU only; multi-GPU scaling is not implemented "
                                   "(requests are independent, so the path would shard by request)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import shared_prefix_scoring_amd as spa
    import synth

    if args.calib_copy:
        n = 1 << 30
        a = torch.empty(n // 4, dtype=torch.int32, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            spa.duolm_copy_device(b.data_ptr(), a.data_ptr(), n)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "launches": 3}), flush=True)
        return

    cfg = synth.QWEN3_0P6B
    log("generating weights; exporting the item table")
    w = synth.make_weights(cfg, seed=0)
    ranker = load_ranker(cfg, w)
    if args.workload != "headline":
        if args.workload == "rating":
            res = bench_rating(ranker, cfg, host_table(ranker, cfg), C=8, rounds=5)
        elif args.workload == "latency":
            res = bench_latency(ranker, cfg, calls=100)
        elif args.workload == "multivec":
            res = bench_multivec(ranker, cfg, rounds=3)
        elif args.workload == "export":
            res = bench_export(ranker, cfg, reps=20)
        elif args.workload == "packer":
            res = bench_packer(ranker, cfg)
        elif args.workload == "session":
            res = bench_session(ranker, cfg, steps=5)
        else:
            res = bench_stress(ranker, cfg, n_req=16, n_ind=32)
        print(json.dumps({"workload": args.workload, **res}), flush=True)
        ranker.close()
        return
    out = headline(args, cfg, w, ranker)
    print(json.dumps(out), flush=True)
    ranker.close()


if __name__ == "__main__":
    main()
