"""GPU-side helpers of the parity tests (device copies, calls through the C
ABI); the comparison itself is in parity_checks (re-exported here)."""
import numpy as np
import torch

import draft_sampling_verify_amd as spec
from parity_checks import (MARGIN, PROB_TOL, check_propose, check_verify, check_verify_against,  # noqa: F401
                           draft_dist, near_boundary, target_dist)


def log(*a):
    print(*a, flush=True)


def to_dev(d):
    """numpy workload dict -> torch tensors on the GPU."""
    t = {}
    for k in ("U", "Lt"):
        t[k] = torch.from_numpy(np.ascontiguousarray(d[k])).cuda()
    for k in ("W1", "W2"):
        w = d[k]
        if w.dtype == np.uint16:
            t[k] = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            t[k] = torch.from_numpy(w).cuda()
    t["W2p"] = spec.spec_pack_w2(t["W2"])
    t["x0"] = torch.from_numpy(d["x0"]).cuda()
    if "c" in d:
        t["c"] = torch.from_numpy(d["c"]).cuda()
    if "sps" in d:
        t["sps"] = torch.from_numpy(d["sps"]).cuda()
    return t


def run_propose(t, cfg, greedy, seed=1, rnd=0, ws=None, path=0):
    x, pdx, pds = spec.spec_markov_propose(t["U"], t["W1"], t["W2p"], t["x0"], cfg.T, greedy, seed, rnd,
                                           ws=ws, path=path)
    torch.cuda.synchronize()
    return x, pdx, pds


def run_verify(t, cfg, x, pds, greedy, ell=None, seed=1, rnd=0, ws=None, path=0):
    n_acc, y, pt_x, c_star = spec.spec_verify(t["U"], t["W1"], t["W2p"], t["x0"], x, pds, t["Lt"], cfg.T,
                                              greedy, seed, rnd, ell=ell, ws=ws, path=path)
    torch.cuda.synchronize()
    return n_acc, y, pt_x, c_star


def np_(t):
    return None if t is None else t.detach().cpu().numpy()
