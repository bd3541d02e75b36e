"""The oracle over many requests at once: requests are independent, so the
conditioned comparison of a full-size workload is split into request chunks
checked in separate host processes (each regenerates its own requests'
inputs from the seeded streams).  Processes are started fresh (spawn): they
never touch the GPU."""
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def host_procs() -> int:
    """Worker processes: the host's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def _check_chunk(args):
    cfg, reqs, gpu, greedy, ell, want_conf = args
    import oracle
    import workloads
    from parity_checks import check_propose, check_verify, PROB_TOL
    d = workloads.make(cfg, requests=list(reqs))
    out = {"propose": check_propose(d, gpu["x"], gpu["pd_x"], gpu["pd_stats"], greedy, free_running=True)}
    out["verify"] = check_verify(d, gpu["x"], ell, gpu["n_acc"], gpu["y"], gpu["pt_x"], gpu["c_star"], greedy)
    if want_conf:
        oc, _ = oracle.confidence(d["U"], d["W1"], d["W2"], d["x0"], gpu["x"], d["Lt"], np.float32(cfg.T))
        np.testing.assert_allclose(gpu["conf"], oc, rtol=0, atol=PROB_TOL)
    return out


def check_requests(cfg, reqs, gpu, greedy, ell=None, conf=None, chunk=None):
    """Conditioned GPU-vs-oracle comparison of the requests `reqs` (every one
    of them), in host processes.  gpu: numpy arrays over all R requests
    (x, pd_x, pd_stats, n_acc, y, pt_x, c_star); ell: verified lengths [R]
    or None; conf: spec_confidence's c* [R, gamma] or None.  Raises on the
    first disagreement; returns the summed counts."""
    reqs = list(reqs)
    n = host_procs()
    chunk = chunk or max(1, (len(reqs) + n - 1) // n)
    jobs = []
    for lo in range(0, len(reqs), chunk):
        sub = np.array(reqs[lo:lo + chunk])
        g = {k: np.ascontiguousarray(v[sub]) for k, v in gpu.items()}
        if conf is not None:
            g["conf"] = np.ascontiguousarray(conf[sub])
        jobs.append((cfg, sub.tolist(), g, greedy, None if ell is None else np.ascontiguousarray(ell[sub]),
                     conf is not None))
    ctx = multiprocessing.get_context("spawn")
    tot = {"propose": {}, "verify": {}}
    with ProcessPoolExecutor(min(n, len(jobs)), mp_context=ctx) as ex:
        for res in ex.map(_check_chunk, jobs):
            for part in ("propose", "verify"):
                for k, v in res[part].items():
                    tot[part][k] = tot[part].get(k, 0) + v
    tot["verify"]["n_acc_mean"] = float(np.mean(gpu["n_acc"][np.array(reqs)]))
    return tot
