"""Benchmark: verified draft tokens/s of one speculative-decoding output step
(Markov-head propose + lossless verify with the fused confidence label) on
one MI355X, and its fraction of the HBM roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

Workload (default c2): R=32 requests, gamma=7, V=129280, r=256, bf16
Markov weights, fp32 base/target logits, sampled, T=1, every position
verified.  Inputs are seeded synthetic data resident in HBM before timing.
A step is one spec_markov_propose + one spec_verify (c* and p_t(x_k)
included) with round = step index.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft tokens/s (propose+verify) at V=129280, gamma=7; % HBM roofline"
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published
PROFILE_DIR = os.path.join(ROOT, "profiles")
_PROPOSE = ["draft_sampling_verify_amd/csrc/propose.hip", "draft_sampling_verify_amd/csrc/common.h"]
_VERIFY = ["draft_sampling_verify_amd/csrc/verify.hip", "draft_sampling_verify_amd/csrc/common.h"]
KERNEL_SOURCES = {
    "propose_fused": _PROPOSE,
    "clear_flags": _PROPOSE,
    "draft_tile": _PROPOSE,
    "propose_pick": _PROPOSE,
    "target_rows": _VERIFY,
    "verify_sweep": _VERIFY,
    "verify_resolve": _VERIFY,
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the kernel's sources with comments and blank lines removed
    (a comment edit does not invalidate a counter measurement)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(l.rstrip() for l in text.splitlines() if l.strip())
        h.update(text.encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(kernel: str, cfg, K: int) -> float:
    """Compulsory HBM bytes of ONE launch of `kernel` (what it must read and
    write for its own job, each distinct byte once).  K = verified rows."""
    R, g, V, r = cfg.R, cfg.gamma, cfg.V, cfg.r
    wb = 2 if cfg.bf16 else 4
    ng = (V + 127) // 128
    if kernel == "propose_fused":   # all positions: U rows, W2 once, W1 rows; x, p_d(x), (M, S) out
        return 4.0 * R * g * V + wb * r * V + wb * R * g * r + 16.0 * R * g
    if kernel == "clear_flags":
        return 4.0 * (ng + R + 1)
    if kernel == "draft_tile":      # one position: U_k rows, W2, W1 rows; (max, sum) partials out
        return 4.0 * R * V + wb * r * V + wb * R * r + 8.0 * R * ng
    if kernel == "target_rows":     # every target row once; (max, sum, argmax) partials out
        return (R + K) * (4.0 * V + 12.0 * ng)
    if kernel == "verify_sweep":    # U and target rows of every verified row, W2, W1 rows; partials out
        return K * (8.0 * V + wb * r + 8.0 * ng) + wb * r * V
    if kernel == "propose_pick":    # partials of every request + one granule rescan
        return R * (8.0 * ng + 128 * (4.0 + wb * r) + 16.0)
    if kernel == "verify_resolve":
        return R * (8.0 * ng * (g + 2) + 128 * (8.0 + wb * r))
    if kernel == "plan":            # verified lengths in, row maps out
        return R * 4.0 + K * 16.0 + (R + K) * 8.0
    if kernel == "schedule":        # confidences and the SPS table in, lengths out
        return 4.0 * R * g + 4.0 * cfg.sps_len + 4.0 * R
    return float("nan")


def step_algorithmic_bytes(cfg, K: int) -> float:
    """Whole-step compulsory bytes: every input byte once (W2 once per call)."""
    R, g, V, r = cfg.R, cfg.gamma, cfg.V, cfg.r
    wb = 2 if cfg.bf16 else 4
    propose = 4.0 * R * g * V + wb * r * V + wb * R * g * r + 16.0 * R * g
    verify = 4.0 * K * V + 4.0 * (R + K) * V + wb * r * V + wb * K * r + 16.0 * R * (g + 1)
    return propose + verify


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def mfma_report(cfg, K: int, kernels: dict) -> dict:
    """The Markov-bias contraction's rate on the matrix cores: 2 r V flops
    per biased row (propose: R gamma rows, verify sweep: K rows), over each
    kernel's time.  Not the bound (about 128 flop per HBM byte against a
    ridge near 312), reported for completeness."""
    out = {"peak_TFLOPs": PEAK_BF16_TFLOPS, "dtype": "bf16" if cfg.bf16 else "fp32"}
    for name, rows in (("propose_fused", cfg.R * cfg.gamma), ("draft_tile", cfg.R), ("verify_sweep", K)):
        if name in kernels:
            fl = 2.0 * cfg.r * cfg.V * rows
            tf = fl / (kernels[name]["avg_us"] * 1e-6) / 1e12
            out[name] = {"flop_per_launch": fl, "TFLOPs": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel's sources changed since."""
    path = os.path.join(PROFILE_DIR, "pmc_%s_%s.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"source_sha256:\s*([0-9a-f]+)", text)
    m_t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_h or not m_t or m_h.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_t.group(1))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_requests(args):
    """Worker of the all-cores leg: the oracle on its share of requests,
    rounds 0, 1, ... until `seconds` have passed; returns (tokens, t0, t1)."""
    cfg, reqs, seconds = args
    import oracle
    import workloads
    d = workloads.make(cfg, requests=reqs, threads=1)
    T = np.float32(cfg.T)
    t0 = time.perf_counter()
    done, rnd = 0, 0
    while True:
        for i in range(len(reqs)):
            sub = {k: d[k][i:i + 1] for k in ("U", "Lt", "x0", "req_ids")}
            p = oracle.markov_propose(sub["U"], d["W1"], d["W2"], sub["x0"], T, False, 1, rnd,
                                      req_ids=sub["req_ids"])
            oracle.verify(sub["U"], d["W1"], d["W2"], sub["x0"], p["x"], sub["Lt"], T, False, 1, rnd,
                          req_ids=sub["req_ids"])
            done += cfg.gamma
        rnd += 1
        if time.perf_counter() - t0 >= seconds:
            return done, t0, time.perf_counter()


def cpu_baseline(cfg, gpu_x=None, gpu_n_acc=None, gpu_y=None, seconds_target=12.0, all_cores_seconds=8.0):
    """The oracle (single-threaded C, fp64) on a bounded sample of requests
    of the same workload: propose + verify with c*, timed on the host.  The
    single-core leg runs in conditioned mode on the GPU's own round-0 tokens
    (same arithmetic as a free run), so it also counts the GPU's decisions
    that differ from the oracle's and how many lie within 1e-6 of a boundary.
    A second leg runs the same oracle in one process per host core (at most
    16) over request shards and reports the aggregate rate."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    import oracle
    import workloads
    oracle.build()
    T = np.float32(cfg.T)
    done, t_total, reqs = 0, 0.0, []
    par = {"decisions": 0, "low_margin": 0, "token_mismatches": 0, "hard_mismatches": 0,
           "verify_requests": 0, "verify_differ": 0, "verify_differ_outside_margin": 0}
    rid = 0
    while t_total < seconds_target and rid < cfg.R:
        d = workloads.make(cfg, requests=[rid])
        xc = None if gpu_x is None else gpu_x[rid:rid + 1]
        t0 = time.perf_counter()
        p = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], T, False, 1, 0, req_ids=d["req_ids"],
                                  x_cond=xc, allow_blank=True)
        xs = p["x"] if xc is None else xc
        v = oracle.verify(d["U"], d["W1"], d["W2"], d["x0"], xs, d["Lt"], T, False, 1, 0, req_ids=d["req_ids"])
        t_total += time.perf_counter() - t0
        if xc is not None:
            mism = p["x"] != xc
            low = p["margin"] < 1e-6
            par["decisions"] += int(xc.size)
            par["low_margin"] += int(low.sum())
            par["token_mismatches"] += int(mism.sum())
            par["hard_mismatches"] += int((mism & ~low).sum())
            par["verify_requests"] += 1
            na = int(gpu_n_acc[rid])
            if na != int(v["n_acc"][0]) or int(gpu_y[rid, na]) != int(v["y"][0, na]):
                par["verify_differ"] += 1
                k = min(na, int(v["n_acc"][0]))
                near = (v["acc_margin"][0, :k + 1] < 1e-6).any() or v["y_margin"][0, na] < 1e-6
                par["verify_differ_outside_margin"] += int(not near)
        reqs.append(rid)
        done += cfg.gamma
        rid += 1
    nproc = os.cpu_count() or 1
    out = {"value": round(done / t_total, 2), "unit": "verified draft tokens/s", "cores": 1, "kind": "oracle",
           "sample": "%d of %d requests of workload %s (propose + verify with c*, round 0), %.1f s "
                     "single-threaded" % (len(reqs), cfg.R, cfg.name, t_total),
           "host_nproc": nproc, "host_cpu": _cpu_model()}
    if gpu_x is not None:
        out["parity_on_sample"] = par
    # all host cores: one process per core (at most 16), request shards
    n = max(1, min(16, nproc))
    shards = [list(range(i, cfg.R, n)) for i in range(n) if i < cfg.R]
    try:
        ctx = multiprocessing.get_context("spawn")
        with ProcessPoolExecutor(len(shards), mp_context=ctx) as ex:
            res = list(ex.map(_oracle_requests, [(cfg, sh, all_cores_seconds) for sh in shards]))
        tok = sum(r[0] for r in res)
        wall = max(r[2] for r in res) - min(r[1] for r in res)
        out["all_cores"] = {"value": round(tok / wall, 2), "cores": len(shards),
                            "sample": "the %d requests of %s in %d processes (one per core, rounds 0, 1, ... for "
                                      "about %.0f s each), %d draft tokens in %.1f s wall" %
                                      (cfg.R, cfg.name, len(shards), all_cores_seconds, tok, wall)}
    except Exception as e:   # the single-core figure stands on its own
        out["all_cores"] = {"error": repr(e)}
    return out


def cluster_bench(spec, workloads, dev, stream, n):
    """Time spec_cluster_propose and spec_cluster_verify on the gemma_e2b
    workload (inputs resident); per-kernel times from the library's events."""
    import torch
    d = workloads.make_cluster("gemma_e2b")
    cfg = d["cfg"]

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    H, C, E = bf(d["H"]), bf(d["C"]), bf(d["E"])
    off = torch.from_numpy(d["cl_off"]).to(dev)
    tok = torch.from_numpy(d["cl_tok"]).to(dev)
    Lt = torch.from_numpy(d["Lt"]).to(dev)
    mc = d["max_cl"]
    ws = spec.ClusterWorkspace(cfg.R, cfg.gamma, cfg.d, cfg.N_c, cfg.K_c, mc, cfg.V, device=dev)
    slot = spec.spec_cluster_index(off, tok, ws=ws, stream=stream)
    po = spec.spec_cluster_propose(H, C, E, off, tok, cfg.K_c, mc, cfg.T, ws=ws, stream=stream)
    vo = spec.spec_cluster_verify(slot, po[2], po[3], po[4], po[0], Lt, cfg.T, cfg.N_c, ws=ws, stream=stream)

    def step(i):
        spec.spec_cluster_propose(H, C, E, off, tok, cfg.K_c, mc, cfg.T, False, 1, i, *po, ws=ws, stream=stream)
        spec.spec_cluster_verify(slot, po[2], po[3], po[4], po[0], Lt, cfg.T, cfg.N_c, False, 1, i, None, *vo,
                                 ws=ws, stream=stream)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / n
    spec.spec_profile_reset()
    spec.spec_profile_enable(True)
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    spec.spec_profile_enable(False)
    kern = {}
    for name in spec.spec_profile_names():
        c, ms = spec.spec_profile_read(name)
        kern[name] = round(1000.0 * ms / c, 2)
    spec.spec_profile_reset()
    # algorithmic bytes: the LM-head rows of the clusters some row selected,
    # the centres and hidden rows once; verify streams the gamma + 1 target
    # rows twice (statistics, sweep)
    sel = po[2].cpu().numpy()
    used = np.unique(sel)
    sizes = np.diff(d["cl_off"])
    pb = float(sizes[used].sum()) * cfg.d * 2 + cfg.N_c * cfg.d * 2 + cfg.R * cfg.gamma * cfg.d * 2
    vb = 2.0 * cfg.R * (cfg.gamma + 1) * cfg.V * 4
    full_head = float(cfg.V) * cfg.d * 2
    ok = spec.spec_device_status(ws) == 0
    del H, C, E, Lt
    return {"workload": "gemma_e2b: R=%d, gamma=%d, d=%d, V=%d, N_c=%d, K_c=%d, bf16 H/C/E, equal clusters of %d, "
                        "sampled, T=%g" % (cfg.R, cfg.gamma, cfg.d, cfg.V, cfg.N_c, cfg.K_c, mc, cfg.T),
            "ms_per_step": round(1000.0 * el, 4), "kernels_us": kern,
            "clusters_expanded_distinct": int(used.size),
            "propose_algorithmic_bytes": pb, "full_lm_head_bytes": full_head,
            "propose_algorithmic_GBs": round(pb / (sum(v for k, v in kern.items() if k.startswith("cluster_")
                                                       and k not in ("cluster_sweep", "cluster_resolve")) * 1e-6)
                                             / 1e9, 1),
            "verify_algorithmic_bytes": vb,
            "mean_n_acc": round(float(vo[0].float().mean()), 3), "device_status_ok": ok}


def _load(spec, workloads, cfg, dev):
    """Device copies of a workload's inputs (W2 packed once, outside any
    timed region)."""
    import torch
    d = workloads.make(cfg)
    t = {"U": torch.from_numpy(d["U"]).to(dev), "Lt": torch.from_numpy(d["Lt"]).to(dev),
         "x0": torch.from_numpy(d["x0"]).to(dev)}
    if cfg.bf16:
        t["W1"] = torch.from_numpy(d["W1"].view(np.int16)).to(dev).view(torch.bfloat16)
        W2 = torch.from_numpy(d["W2"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        t["W1"], W2 = torch.from_numpy(d["W1"]).to(dev), torch.from_numpy(d["W2"]).to(dev)
    t["W2p"] = spec.spec_pack_w2(W2)
    if "c" in d:
        t["c"] = torch.from_numpy(d["c"]).to(dev)
    if "sps" in d:
        t["sps"] = torch.from_numpy(d["sps"]).to(dev)
    del d, W2
    return t


def _kernel_table(spec, run, n, cfg, K):
    """run(i) for i < n with the library's HIP events on: per-kernel average
    launch time, launches per step and algorithmic GB/s."""
    import torch
    spec.spec_profile_reset()
    spec.spec_profile_enable(True)
    for i in range(n):
        run(i)
    torch.cuda.synchronize()
    spec.spec_profile_enable(False)
    kernels = {}
    for name in spec.spec_profile_names():
        c, ms = spec.spec_profile_read(name)
        avg = 1000.0 * ms / c
        b = algorithmic_bytes(name, cfg, K)
        kernels[name] = {"launches_per_step": c / n, "avg_us": round(avg, 2),
                         "us_per_step": round(1000.0 * ms / n, 2),
                         "algorithmic_GBs": None if b != b else round(b / (avg * 1e-6) / 1e9, 1)}
    spec.spec_profile_reset()
    return kernels


def measure_config(spec, workloads, name, dev, stream, steps, warmup=3, min_warm_s=0.3, min_timed_s=0.5):
    """One more workload, timed with the headline's protocol (warm-up, then
    timed steps bracketed by device synchronisation; round = step index).
    The warm-up runs at least `warmup` steps and `min_warm_s` seconds, and
    the timed region at least `steps` steps and `min_timed_s` seconds: the
    clocks settle over some hundred milliseconds of back-to-back steps, and
    a short window after the host-side input generation reads high.
    c1: latency of one propose + verify step.  c3, c5: propose + verify of
    every position.  c4: the serving pipeline propose -> schedule(c) ->
    verify(l) with c* fused; verified draft tokens = K* of the schedule."""
    import torch
    cfg = workloads.CONFIGS["tiny" if name == "c1" else name]
    t = _load(spec, workloads, cfg, dev)
    R, g, V = cfg.R, cfg.gamma, cfg.V
    x = torch.empty((R, g), dtype=torch.int32, device=dev)
    pd_x = torch.empty((R, g), dtype=torch.float32, device=dev)
    pd_stats = torch.empty((R, g, 2), dtype=torch.float32, device=dev)
    n_acc = torch.empty(R, dtype=torch.int32, device=dev)
    y = torch.empty((R, g + 1), dtype=torch.int32, device=dev)
    pt_x = torch.empty((R, g), dtype=torch.float32, device=dev)
    c_star = torch.empty((R, g), dtype=torch.float32, device=dev)
    ws = spec.Workspace(R, g, cfg.r, V, B_max=max(cfg.sps_len, R), device=dev)
    sched = name == "c4"
    if sched:
        ell = torch.empty(R, dtype=torch.int32, device=dev)
        K_star = torch.empty(1, dtype=torch.int32, device=dev)
        theta = torch.empty(1, dtype=torch.float64, device=dev)

    def step(i):
        spec.spec_markov_propose(t["U"], t["W1"], t["W2p"], t["x0"], cfg.T, False, 1, i, x=x, pd_x=pd_x,
                                 pd_stats=pd_stats, ws=ws, stream=stream)
        if sched:
            spec.spec_schedule(t["c"], t["sps"], ell=ell, K_star=K_star, theta_star=theta, want_a=False, ws=ws,
                               stream=stream)
        spec.spec_verify(t["U"], t["W1"], t["W2p"], t["x0"], x, pd_stats, t["Lt"], cfg.T, False, 1, i,
                         ell=ell if sched else None, n_acc=n_acc, y=y, pt_x=pt_x, c_star=c_star, ws=ws,
                         stream=stream)

    n_warm = 0
    tw = time.perf_counter()
    while n_warm < warmup or time.perf_counter() - tw < min_warm_s:
        step(n_warm)
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # the timed step count: at least `steps`, and enough for min_timed_s at
    # the warm-up's rate
    per_step = (time.perf_counter() - tw) / n_warm
    n_table = steps  # the kernel table (HIP events around every launch) keeps the requested count
    steps = max(steps, int(min_timed_s / max(per_step, 1e-6)) + 1)
    t0 = time.perf_counter()
    for i in range(steps):
        step(n_warm + i)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    warmup = n_warm
    K = int(K_star.item()) if sched else R * g
    kernels = _kernel_table(spec, lambda i: step(warmup + i), n_table, cfg, K)
    sb = step_algorithmic_bytes(cfg, K) + (4.0 * R * g + 4.0 * cfg.sps_len if sched else 0.0)
    out = {"workload": "%s: R=%d, gamma=%d, V=%d, r=%d, %s weights, sampled, T=%g%s" % (
               cfg.name if name != "c1" else "c1 (tiny)", R, g, V, cfg.r, "bf16" if cfg.bf16 else "fp32", cfg.T,
               ", propose -> schedule(c) -> verify(l), c* fused" if sched else ", every position verified"),
           "steps": steps, "ms_per_step": round(1000.0 * el, 4),
           "verified_draft_tokens_per_step": K,
           "value": round(K / el, 1), "unit": "verified draft tokens/s",
           "step_algorithmic_bytes": sb,
           "hbm_roofline_frac_step": round(sb / (PEAK_HBM_GBS * 1e9) / el, 4),
           "kernels": kernels,
           "mean_n_acc": round(float(n_acc.float().mean()), 4),
           "device_status": spec.spec_device_status(ws)}
    if name == "c1":
        out["us_per_step"] = round(1e6 * el, 2)
    if sched:
        out["K_star"] = K
        out["candidates"] = R * g
    del t, ws
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + timed steps only (for rocprofv3), print the JSON line")
    ap.add_argument("--propose-path", choices=["auto", "per_position"], default="auto",
                    help="auto: the fused single-launch propose where it fits; per_position: two kernels "
                         "per draft position")
    ap.add_argument("--rounds", type=int, default=8,
                    help="rounds of the multi-round loop measured after the main steps (0 = skip)")
    ap.add_argument("--no-cluster", dest="cluster", action="store_false",
                    help="skip the clustered draft head measurement")
    ap.add_argument("--profile-cluster", action="store_true",
                    help="run only the clustered draft head's steps (for rocprofv3), print its JSON object")
    ap.add_argument("--configs", default="c1,c3,c4,c5",
                    help="other workloads timed after the headline (comma list; empty = none)")
    ap.add_argument("--calib-copy-mb", type=int, default=512,
                    help="size of the device-to-device copy timed as the achievable-bandwidth reference")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requests would shard across GPUs with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import draft_sampling_verify_amd as spec

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    spec.lib()
    if args.profile_cluster:
        print(json.dumps(cluster_bench(spec, workloads, torch.device("cuda:0"), torch.cuda.current_stream(),
                                       args.steps)), flush=True)
        return
    ppath = spec.SPEC_PATH_AUTO if args.propose_path == "auto" else spec.SPEC_PATH_NO_FUSED_PROPOSE
    cfg = workloads.CONFIGS[args.workload]
    d = workloads.make(cfg)
    dev = torch.device("cuda:0")
    U = torch.from_numpy(d["U"]).to(dev)
    Lt = torch.from_numpy(d["Lt"]).to(dev)
    if cfg.bf16:
        W1 = torch.from_numpy(d["W1"].view(np.int16)).to(dev).view(torch.bfloat16)
        W2 = torch.from_numpy(d["W2"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        W1, W2 = torch.from_numpy(d["W1"]).to(dev), torch.from_numpy(d["W2"]).to(dev)
    x0 = torch.from_numpy(d["x0"]).to(dev)
    W2p = spec.spec_pack_w2(W2)          # once per weight, outside the timed region
    del W2
    R, g, V = cfg.R, cfg.gamma, cfg.V
    x = torch.empty((R, g), dtype=torch.int32, device=dev)
    pd_x = torch.empty((R, g), dtype=torch.float32, device=dev)
    pd_stats = torch.empty((R, g, 2), dtype=torch.float32, device=dev)
    n_acc = torch.empty(R, dtype=torch.int32, device=dev)
    y = torch.empty((R, g + 1), dtype=torch.int32, device=dev)
    pt_x = torch.empty((R, g), dtype=torch.float32, device=dev)
    c_star = torch.empty((R, g), dtype=torch.float32, device=dev)
    ws = spec.Workspace(R, g, cfg.r, V, device=dev)
    stream = torch.cuda.current_stream()
    del d

    def step(i):
        spec.spec_markov_propose(U, W1, W2p, x0, cfg.T, False, 1, i, x=x, pd_x=pd_x, pd_stats=pd_stats,
                                 ws=ws, stream=stream, path=ppath)
        spec.spec_verify(U, W1, W2p, x0, x, pd_stats, Lt, cfg.T, False, 1, i, n_acc=n_acc, y=y, pt_x=pt_x,
                         c_star=c_star, ws=ws, stream=stream)

    # the GPU's round-0 outputs, for the oracle sample of the CPU baseline
    step(0)
    torch.cuda.synchronize()
    gx0, gn0, gy0 = x.cpu().numpy(), n_acc.cpu().numpy(), y.cpu().numpy()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, plain launches
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # same K steps again with HIP events around every kernel (on its stream)
    spec.spec_profile_reset()
    spec.spec_profile_enable(True)
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed_prof = time.perf_counter() - t1
    spec.spec_profile_enable(False)
    kernels = {}
    for name in spec.spec_profile_names():
        n, ms = spec.spec_profile_read(name)
        kernels[name] = {"launches_per_step": n / args.steps, "avg_us": 1000.0 * ms / n,
                         "us_per_step": 1000.0 * ms / args.steps}
    spec.spec_profile_reset()
    # achievable-bandwidth reference: a plain device copy of known size
    copy_gbs = None
    if args.calib_copy_mb > 0:
        nb = args.calib_copy_mb << 20
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 2.0 * nb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
    # the multi-round loop: n rounds of propose + verify (c* included), each
    # round anchored on the previous round's last emitted tokens, eager and
    # replayed from one captured HIP graph
    multi = None
    if args.rounds > 0 and not args.profile_only:
        n = args.rounds
        rb = dict(anchors=torch.empty((n + 1, R), dtype=torch.int32, device=dev),
                  x=torch.empty((n, R, g), dtype=torch.int32, device=dev),
                  n_acc=torch.empty((n, R), dtype=torch.int32, device=dev),
                  y=torch.empty((n, R, g + 1), dtype=torch.int32, device=dev),
                  c_star=torch.empty((n, R, g), dtype=torch.float32, device=dev))

        def rounds(i, strm):
            spec.spec_decode_rounds(U, W1, W2p, x0, Lt, cfg.T, n, False, 1, 1000 + i * n, ws=ws, stream=strm, **rb)

        reps = max(3, args.steps // (2 * n))
        rounds(0, stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            rounds(i, stream)
        torch.cuda.synchronize()
        eager_s = (time.perf_counter() - t0) / reps
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            rounds(0, side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            rounds(0, torch.cuda.current_stream())
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_s = (time.perf_counter() - t0) / reps
        emitted = float((rb["n_acc"].float() + 1.0).sum())
        multi = {"rounds": n, "repetitions": reps,
                 "ms_per_round_eager": round(1000.0 * eager_s / n, 4),
                 "ms_per_round_graph": round(1000.0 * graph_s / n, 4),
                 "verified_draft_tokens_per_s_graph": round(R * g * n / graph_s, 1),
                 "emitted_tokens_per_round": round(emitted / n, 2),
                 "emitted_tokens_per_s_graph": round(emitted / graph_s, 1)}
        del graph

    # the prefix scheduler at the scheduler-heavy shape (R = 512, gamma = 16,
    # sawtooth SPS over B = 1..8704), synchronous and production step
    sched = None
    if not args.profile_only:
        c4 = workloads.CONFIGS["c4"]
        cs = torch.from_numpy(workloads.confidences(c4)).to(dev)
        sps4 = torch.from_numpy(workloads.sawtooth_sps(c4)).to(dev)
        sws = spec.Workspace(c4.R, c4.gamma, 16, 1, B_max=sps4.numel(), device=dev)
        ring = torch.full((2,), -1, dtype=torch.int32, device=dev)
        so = spec.spec_schedule(cs, sps4, ws=sws, stream=stream)
        ao = spec.spec_schedule_async(cs, sps4, ring, ws=sws, stream=stream)
        times = {}
        for name, fn in (("sync", lambda: spec.spec_schedule(cs, sps4, *so, ws=sws, stream=stream)),
                         ("async", lambda: spec.spec_schedule_async(cs, sps4, ring, *ao, ws=sws, stream=stream))):
            for _ in range(3):
                fn()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for _ in range(50):
                fn()
            a1.record(stream)
            torch.cuda.synchronize()
            times[name] = a0.elapsed_time(a1) * 1e3 / 50
        sched = {"workload": "c4 shape: R=512, gamma=16 (8192 candidates), sawtooth SPS over B=1..8704",
                 "us_per_call_sync": round(times["sync"], 2), "us_per_call_async": round(times["async"], 2),
                 "K_star": int(so[2].item()), "K_used_async": int(ao[2].item())}
        del sws

    # the training-side loss over the same rows (teacher-forced on seeded
    # labels): draft row statistics, target row statistics, the sweep, the
    # terms and their weighted mean
    loss_info = None
    if not args.profile_only:
        yl = torch.from_numpy(workloads.loss_labels(cfg)).to(dev)
        ql = torch.from_numpy(workloads.confidence_logits(cfg)).to(dev)
        lo = spec.spec_draft_loss(U, W1, W2p, x0, yl, Lt, ql, cfg.T, ws=ws, stream=stream)
        for _ in range(3):
            spec.spec_draft_loss(U, W1, W2p, x0, yl, Lt, ql, cfg.T, loss=lo[0], terms=lo[1], dq=lo[2], ws=ws,
                                 stream=stream)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nl = max(10, args.steps // 4)
        a0.record(stream)
        for _ in range(nl):
            spec.spec_draft_loss(U, W1, W2p, x0, yl, Lt, ql, cfg.T, loss=lo[0], terms=lo[1], dq=lo[2], ws=ws,
                                 stream=stream)
        a1.record(stream)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) * 1e3 / nl
        lb = 2.0 * R * g * V * 4 + V * cfg.r * (2 if cfg.bf16 else 4)   # U, g target rows, W2 once
        loss_info = {"workload": "%s shape, uniform labels, q ~ N(0, 1.5^2), coefficients (0.1, 0.9, 1.0)" % cfg.name,
                     "us_per_call": round(us, 2), "positions_per_s": round(R * g / (us * 1e-6), 1),
                     "algorithmic_bytes": lb, "algorithmic_GBs": round(lb / (us * 1e-6) / 1e9, 1),
                     "loss": round(float(lo[0].item()), 6)}
        del yl, ql, lo

    # the clustered draft head (Gemma 4 E2B-like: V = 262144, d = 1536, 2048
    # centres, top 32 expanded) on its own workload: propose and verify
    cluster = None
    if not args.profile_only and args.cluster:
        cluster = cluster_bench(spec, workloads, dev, stream, max(10, args.steps // 4))

    acc = float(n_acc.float().mean())
    cmean = float(c_star.float().mean())
    flags = spec.spec_device_status(ws)

    K = R * g
    ms_step = 1000.0 * elapsed / args.steps
    value = K * args.steps / elapsed
    dom = max(kernels, key=lambda k: kernels[k]["us_per_step"])
    per_launch = algorithmic_bytes(dom, cfg, K)
    achieved = per_launch / (kernels[dom]["avg_us"] * 1e-6) / 1e9
    traffic = read_traffic(dom, cfg.name)
    step_bytes = step_algorithmic_bytes(cfg, K)
    for k, v in kernels.items():
        b = algorithmic_bytes(k, cfg, K)
        v["algorithmic_GBs"] = None if b != b else round(b / (v["avg_us"] * 1e-6) / 1e9, 1)
        v["avg_us"] = round(v["avg_us"], 2)
        v["us_per_step"] = round(v["us_per_step"], 2)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "%s: R=%d, gamma=%d, V=%d, r=%d, %s Markov weights, fp32 logits, "
                               "sampled, T=%g, all positions verified" %
                               (cfg.name, R, g, V, cfg.r, "bf16" if cfg.bf16 else "fp32", cfg.T),
                   "R": R, "gamma": g, "V": V, "r": cfg.r, "verified_per_step": K,
                   "propose": "fused" if "propose_fused" in kernels else "per_position"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": per_launch},
        "hbm_roofline_frac_step": round(step_bytes / (PEAK_HBM_GBS * 1e9) / (elapsed / args.steps), 4),
        "mfma": mfma_report(cfg, K, kernels),
        "device_copy_GBs": None if copy_gbs is None else round(copy_gbs, 1),
        "step_algorithmic_bytes": step_bytes,
        "ms_per_step_with_kernel_events": round(1000.0 * elapsed_prof / args.steps, 4),
        "kernels": kernels,
        "multi_round": multi,
        "scheduler": sched,
        "training_loss": loss_info,
        "cluster_head": cluster,
        "mean_n_acc": round(acc, 4),
        "mean_c_star": round(cmean, 4),
        "device_status": flags,
    }
    configs = {}
    if not args.profile_only and args.configs:
        del U, Lt, W1, W2p
        torch.cuda.empty_cache()
        for name in [c for c in args.configs.split(",") if c]:
            n = {"c1": 200, "c3": 20, "c4": 10, "c5": 20}.get(name, 20)
            print("bench: %s" % name, file=sys.stderr, flush=True)
            configs[name] = measure_config(spec, workloads, name, dev, stream, n)
    out["configs"] = configs
    if not args.no_cpu_baseline and not args.profile_only:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, gx0, gn0, gy0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
