"""CPU oracle for the speculative-decoding output side -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps the plain C oracle in
``ref.c`` (double precision, single thread) with ctypes and numpy; it shares
no code with the HIP library and never imports it.

Parity status per function (what pins it is in ``tests/test_oracle_*.py``):
  philox / u24      pinned: published known-answer blocks + ATen's Philox engine
  bias / softmax    pinned: numpy matmul, scipy softmax, W2 = 0 reduction
  propose           pinned: numpy searchsorted on the whole softmax (one
                    inverse CDF over the row), chi-square at V = 16 and over
                    tokens spread across several 128-id granules, rows
                    without probability mass
  verify            pinned: chi-square of emitted tokens vs p_t, closed forms
                    for P(accept), E[n_acc], special cases
  confidence        pinned: V = 2 closed form, identical rows, TV identity
  schedule          pinned: exhaustive enumeration of allocations
  schedule_async    pinned: enumeration of fixed-size allocations (top-K is
                    the best), the two-step history ring, nesting in K
  draft_loss        pinned: scipy log-softmax cross-entropy, identical rows
                    (l1 = 0, c* = 1), l1 = 2(1 - c*) against confidence,
                    finite differences of dq, closed form at V = 2
  cluster_propose   pinned: numpy top-K and softmax over the expanded set,
                    full expansion with contiguous clusters = the plain
                    inverse CDF over the whole softmax, chi-square of draws
  cluster_verify    pinned: chi-square of emitted tokens vs p_t (lossless
                    with a sparse draft), P(accept) = c*, full expansion =
                    the Markov verify with U = H E^T and W2 = 0
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "ref.c")

F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile ref.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < max(os.path.getmtime(_SRC),
                                               os.path.getmtime(os.path.join(_HERE, "ref.h"))):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, u64, f32 = ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
        L.ref_philox4x32_10.argtypes = [P, P, P]
        L.ref_draw.argtypes = [u64, u64, i32, i32, P]
        L.ref_philox_words.argtypes = [u64, u64, u64, P]
        L.ref_u24.argtypes = [ctypes.c_uint32]
        L.ref_u24.restype = ctypes.c_double
        L.ref_bias.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32, P]
        L.ref_inverse_cdf.argtypes = [P, ctypes.c_int, ctypes.c_double, P]
        L.ref_inverse_cdf.restype = i32
        L.ref_argmax.argtypes = [P, ctypes.c_int, P]
        L.ref_argmax.restype = i32
        L.ref_markov_propose.argtypes = [P, P, P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, f32, ctypes.c_int, u64, u64,
                                         P, P, P, P, P, P]
        L.ref_verify.argtypes = [P, P, P, ctypes.c_int, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, f32, ctypes.c_int, u64, u64, P,
                                 P, P, P, P, P, P, P, P, P]
        L.ref_confidence.argtypes = [P, P, P, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, f32, P, P]
        L.ref_schedule.argtypes = [P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, P, P, P,
                                   P, P]
        L.ref_schedule_async.argtypes = [P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, P, P, P, P,
                                         P, P]
        L.ref_draft_loss.argtypes = [P, P, P, ctypes.c_int, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, f32, f32, f32, f32, P, P, P]
        L.ref_cluster_propose.argtypes = [P, P, P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, f32, ctypes.c_int, u64, u64,
                                          P, P, P, P, P, P]
        L.ref_cluster_verify.argtypes = [P, P, ctypes.c_int, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, f32, ctypes.c_int,
                                         u64, u64, P, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _weights(W1, W2):
    """Return (W1, W2, dtype code): float32 arrays, or bf16 given as uint16 bits."""
    if W1.dtype == np.uint16:
        return _c(W1, np.uint16), _c(W2, np.uint16), BF16
    return _c(W1, np.float32), _c(W2, np.float32), F32


def philox(ctr, key):
    out = np.zeros(4, np.uint32)
    lib().ref_philox4x32_10(_p(_c(ctr, np.uint32)), _p(_c(key, np.uint32)), _p(out))
    return out


def draw(seed, rnd, req, k):
    out = np.zeros(4, np.uint32)
    lib().ref_draw(seed, rnd, req, k, _p(out))
    return out


def u24(w):
    return lib().ref_u24(int(w))


def philox_words(seed, rnd, n):
    """[n, 4] uint32: the blocks at counters (i mod 2^16, i / 2^16, round)."""
    out = np.zeros((n, 4), np.uint32)
    lib().ref_philox_words(seed, rnd, n, _p(out))
    return out


def bias(W1, W2, xprev):
    W1, W2, dt = _weights(W1, W2)
    V, r = W2.shape
    out = np.zeros(V, np.float64)
    lib().ref_bias(_p(W1), _p(W2), dt, r, V, int(xprev), _p(out))
    return out


def inverse_cdf(w, u):
    w = _c(w, np.float64)
    m = np.zeros(1, np.float64)
    v = lib().ref_inverse_cdf(_p(w), w.size, float(u), _p(m))
    return int(v), float(m[0])


def argmax(z):
    z = _c(z, np.float64)
    m = np.zeros(1, np.float64)
    v = lib().ref_argmax(_p(z), z.size, _p(m))
    return int(v), float(m[0])


class OracleError(RuntimeError):
    pass


def markov_propose(U, W1, W2, x0, T, greedy, seed, rnd, req_ids=None, x_cond=None, allow_blank=False):
    """Returns dict with x [R,g], pd_x [R,g], pd_stats [R,g,2], margin [R,g]
    and blanked (True if a request had no valid chain: an anchor outside
    [0, V) or a row without probability mass; its entries are -1 / NaN).
    A blanked request raises OracleError unless allow_blank."""
    U = _c(U, np.float32)
    R, g, V = U.shape
    W1, W2, dt = _weights(W1, W2)
    r = W2.shape[1]
    x0 = _c(x0, np.int32)
    req_ids = _c(req_ids, np.int32)
    x_cond = _c(x_cond, np.int32)
    out = dict(x=np.zeros((R, g), np.int32), pd_x=np.zeros((R, g)),
               pd_stats=np.zeros((R, g, 2)), margin=np.zeros((R, g)))
    st = lib().ref_markov_propose(_p(U), _p(W1), _p(W2), dt, _p(x0), R, g, r, V, float(T),
                                  int(bool(greedy)), seed, rnd, _p(req_ids), _p(x_cond),
                                  _p(out["x"]), _p(out["pd_x"]), _p(out["pd_stats"]),
                                  _p(out["margin"]))
    if st == 1 and allow_blank:
        out["blanked"] = True
        return out
    if st != 0:
        raise OracleError("ref_markov_propose rejected its arguments" if st < 0 else
                          "ref_markov_propose: a request has no valid chain")
    out["blanked"] = False
    return out


def verify(U, W1, W2, x0, x, Lt, T, greedy, seed, rnd, ell=None, req_ids=None):
    """Returns dict with n_acc, y, pt_x, pd_x, c_star and per-position instrumentation."""
    U = _c(U, np.float32)
    R, g, V = U.shape
    Lt = _c(Lt, np.float32)
    assert Lt.shape == (R, g + 1, V)
    W1, W2, dt = _weights(W1, W2)
    r = W2.shape[1]
    x0, x = _c(x0, np.int32), _c(x, np.int32)
    ell, req_ids = _c(ell, np.int32), _c(req_ids, np.int32)
    o = dict(n_acc=np.zeros(R, np.int32), y=np.zeros((R, g + 1), np.int32),
             pt_x=np.zeros((R, g)), pd_x=np.zeros((R, g)), c_star=np.zeros((R, g)),
             acc=np.zeros((R, g), np.int32), acc_margin=np.zeros((R, g)),
             y_alt=np.zeros((R, g + 1), np.int32), y_margin=np.zeros((R, g + 1)))
    st = lib().ref_verify(_p(U), _p(W1), _p(W2), dt, _p(x0), _p(x), _p(Lt), _p(ell), R, g, r, V,
                          float(T), int(bool(greedy)), seed, rnd, _p(req_ids),
                          _p(o["n_acc"]), _p(o["y"]), _p(o["pt_x"]), _p(o["pd_x"]),
                          _p(o["c_star"]), _p(o["acc"]), _p(o["acc_margin"]), _p(o["y_alt"]),
                          _p(o["y_margin"]))
    if st != 0:
        raise OracleError("ref_verify rejected its arguments")
    return o


def confidence(U, W1, W2, x0, x, Lt, T):
    U = _c(U, np.float32)
    R, g, V = U.shape
    Lt = _c(Lt, np.float32)
    W1, W2, dt = _weights(W1, W2)
    r = W2.shape[1]
    x0, x = _c(x0, np.int32), _c(x, np.int32)
    c = np.zeros((R, g))
    a = np.zeros((R, g))
    st = lib().ref_confidence(_p(U), _p(W1), _p(W2), dt, _p(x0), _p(x), _p(Lt), R, g, r, V,
                              float(T), _p(c), _p(a))
    if st != 0:
        raise OracleError("ref_confidence rejected its arguments")
    return c, a


def _mats(*arrays):
    """float32 arrays, or bf16 given as uint16 bits (one dtype for all)."""
    if arrays[0].dtype == np.uint16:
        return [_c(a, np.uint16) for a in arrays] + [BF16]
    return [_c(a, np.float32) for a in arrays] + [F32]


def cluster_propose(H, C, E, cl_off, cl_tok, K_c, T, greedy=False, seed=1, rnd=0):
    """Clustered draft head (ref_cluster_propose).  H [R,g,d], C [N_c,d],
    E [V,d]; returns dict(x, pd_x, sel [R,g,K_c], pd_stats, cut, margin)."""
    H, C, E, dt = _mats(H, C, E)
    R, g, d = H.shape
    N_c, V = C.shape[0], E.shape[0]
    cl_off, cl_tok = _c(cl_off, np.int32), _c(cl_tok, np.int32)
    o = dict(x=np.zeros((R, g), np.int32), pd_x=np.zeros((R, g)), sel=np.zeros((R, g, K_c), np.int32),
             pd_stats=np.zeros((R, g, 2)), cut=np.zeros((R, g)), margin=np.zeros((R, g)))
    st = lib().ref_cluster_propose(_p(H), _p(C), _p(E), dt, _p(cl_off), _p(cl_tok), R, g, d, N_c, int(K_c), V,
                                   float(T), int(bool(greedy)), seed, rnd, _p(o["x"]), _p(o["pd_x"]),
                                   _p(o["sel"]), _p(o["pd_stats"]), _p(o["cut"]), _p(o["margin"]))
    if st != 0:
        raise OracleError("ref_cluster_propose rejected its arguments")
    return o


def cluster_verify(H, E, cl_off, cl_tok, sel, x, Lt, T, greedy=False, seed=1, rnd=0, ell=None, N_c=None):
    """Verification of clustered-head drafts (ref_cluster_verify), given the
    selection sel; returns the same dict as verify()."""
    H, E, dt = _mats(H, E)
    R, g, d = H.shape
    V = E.shape[0]
    cl_off, cl_tok = _c(cl_off, np.int32), _c(cl_tok, np.int32)
    N_c = cl_off.size - 1 if N_c is None else N_c
    sel, x = _c(sel, np.int32), _c(x, np.int32)
    K_c = sel.shape[-1]
    Lt = _c(Lt, np.float32)
    assert Lt.shape == (R, g + 1, V)
    ell = _c(ell, np.int32)
    o = dict(n_acc=np.zeros(R, np.int32), y=np.zeros((R, g + 1), np.int32),
             pt_x=np.zeros((R, g)), pd_x=np.zeros((R, g)), c_star=np.zeros((R, g)),
             acc=np.zeros((R, g), np.int32), acc_margin=np.zeros((R, g)),
             y_alt=np.zeros((R, g + 1), np.int32), y_margin=np.zeros((R, g + 1)))
    st = lib().ref_cluster_verify(_p(H), _p(E), dt, _p(cl_off), _p(cl_tok), _p(sel), _p(x), _p(Lt), _p(ell),
                                  R, g, d, N_c, K_c, V, float(T), int(bool(greedy)), seed, rnd,
                                  _p(o["n_acc"]), _p(o["y"]), _p(o["pt_x"]), _p(o["pd_x"]),
                                  _p(o["c_star"]), _p(o["acc"]), _p(o["acc_margin"]), _p(o["y_alt"]),
                                  _p(o["y_margin"]))
    if st != 0:
        raise OracleError("ref_cluster_verify rejected its arguments")
    return o


def draft_loss(U, W1, W2, x0, y, Lt, q, T, alphas=(0.1, 0.9, 1.0)):
    """Training-side loss (ref_draft_loss): returns dict(loss, terms [R,g,3]
    = (ce, l1, bce), dq [R,g])."""
    W1, W2, dt = _weights(W1, W2)
    U = _c(U, np.float32)
    R, g, V = U.shape
    r = W1.shape[1]
    x0 = _c(x0, np.int32)
    y = _c(y, np.int32)
    Lt = _c(Lt, np.float32)
    q = _c(q, np.float32)
    loss = np.zeros(1)
    terms = np.zeros((R, g, 3))
    dq = np.zeros((R, g))
    st = lib().ref_draft_loss(_p(U), _p(W1), _p(W2), dt, _p(x0), _p(y), _p(Lt), _p(q), R, g, r, V, float(T),
                              float(alphas[0]), float(alphas[1]), float(alphas[2]), _p(loss), _p(terms), _p(dq))
    if st != 0:
        raise OracleError("ref_draft_loss rejected its arguments")
    return dict(loss=float(loss[0]), terms=terms, dq=dq)


def schedule(c, sps):
    c = _c(c, np.float32)
    R, g = c.shape
    sps = _c(sps, np.float32)
    ell = np.zeros(R, np.int32)
    a = np.zeros((R, g))
    K = np.zeros(1, np.int32)
    th = np.zeros(1)
    tm = np.zeros(1)
    gap = np.zeros(1)
    st = lib().ref_schedule(_p(c), R, g, _p(sps), sps.size, _p(ell), _p(a), _p(K), _p(th),
                            _p(tm), _p(gap))
    if st != 0:
        raise OracleError("ref_schedule rejected its arguments")
    return dict(ell=ell, a=a, K_star=int(K[0]), theta_star=float(th[0]),
                theta_margin=float(tm[0]), a_gap=float(gap[0]))


def schedule_async(c, sps, K_hist):
    """The production scheduler step (ref_schedule_async): K from the ring
    K_hist = [K* two calls ago, K* one call ago] (negative: none yet),
    ranking by the current confidences.  Returns the outputs and the
    advanced ring."""
    c = _c(c, np.float32)
    R, g = c.shape
    sps = _c(sps, np.float32)
    hist = np.array(K_hist, np.int32)
    ell = np.zeros(R, np.int32)
    a = np.zeros((R, g))
    Ku = np.zeros(1, np.int32)
    K = np.zeros(1, np.int32)
    th = np.zeros(1)
    tm = np.zeros(1)
    st = lib().ref_schedule_async(_p(c), R, g, _p(sps), sps.size, _p(hist), _p(ell), _p(a), _p(Ku), _p(K),
                                  _p(th), _p(tm))
    if st != 0:
        raise OracleError("ref_schedule_async rejected its arguments")
    return dict(ell=ell, a=a, K_used=int(Ku[0]), K_star=int(K[0]), theta_star=float(th[0]),
                theta_margin=float(tm[0]), K_hist=hist)
