"""ctypes binding of libspec (include/spec.h): argument marshalling only.

Every function has the C entry point's name and takes torch tensors on the
GPU (PyTorch supplies device memory and the stream); outputs that are not
passed in are allocated with torch.empty.  All computation happens in the
HIP kernels of libspec.so; if the library is missing this module raises
instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspec.so")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EWORKSPACE, SPEC_ELAUNCH, SPEC_EDEVICE, SPEC_EUNSUPPORTED = range(7)
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_OP_PROPOSE, SPEC_OP_VERIFY, SPEC_OP_CONFIDENCE, SPEC_OP_SCHEDULE, SPEC_OP_ROUNDS, SPEC_OP_LOSS = range(6)
SPEC_DEV_BAD_TOKEN, SPEC_DEV_BAD_LENGTH, SPEC_DEV_BAD_CONFIDENCE, SPEC_DEV_WAIT_FAILED = 1, 2, 4, 8
SPEC_DEV_BAD_CLUSTER = 16
SPEC_PATH_AUTO, SPEC_PATH_NO_FUSED_PROPOSE, SPEC_PATH_NO_PIPELINED_SWEEP = 0, 1, 2


class SpecError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_str(status), status))


_lib = None

P, I, F, U64, SZ, D = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint64,
                       ctypes.c_size_t, ctypes.c_double)

_SIGS = {
    "spec_workspace_bytes": ([I, I, I, I, I, I], SZ),
    "spec_workspace_init": ([P, SZ, P], I),
    "spec_packed_w2_bytes": ([I, I, I], SZ),
    "spec_pack_w2": ([P, I, I, I, P, P], I),
    "spec_pack_w2_rv": ([P, I, I, I, P, P], I),
    "spec_device_status": ([P, P, I, P], I),
    "spec_markov_propose": ([P, P, P, I, P, I, I, I, I, F, I, U64, U64, P, P, P, P, SZ, P], I),
    "spec_markov_propose_noalloc": ([P, P, P, I, P, I, I, I, I, F, I, U64, U64, P, P, P, P, P], I),
    "spec_markov_propose_ex": ([P, P, P, I, P, I, I, I, I, F, I, U64, U64, P, P, P, I, P, SZ, P], I),
    "spec_verify": ([P, P, P, I, P, P, P, P, P, I, I, I, I, F, I, U64, U64, P, P, P, P, P, SZ, P], I),
    "spec_verify_ex": ([P, P, P, I, P, P, P, P, P, I, I, I, I, F, I, U64, U64, P, P, P, P, I, P, SZ, P], I),
    "spec_confidence": ([P, P, P, I, P, P, P, P, I, I, I, I, F, P, P, P, SZ, P], I),
    "spec_confidence_ex": ([P, P, P, I, P, P, P, P, I, I, I, I, F, P, P, I, P, SZ, P], I),
    "spec_schedule": ([P, I, I, P, I, P, P, P, P, P, SZ, P], I),
    "spec_schedule_async": ([P, I, I, P, I, P, P, P, P, P, P, P, SZ, P], I),
    "spec_draft_loss": ([P, P, P, I, P, P, P, P, I, I, I, I, F, F, F, F, P, P, P, P, SZ, P], I),
    "spec_cluster_workspace_bytes": ([I, I, I, I, I, I, I], SZ),
    "spec_cluster_index": ([P, P, I, I, P, P, SZ, P], I),
    "spec_cluster_propose": ([P, P, P, I, P, P, I, I, I, I, I, I, I, F, I, U64, U64, P, P, P, P, P, P, SZ, P], I),
    "spec_cluster_verify": ([P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, U64, U64, P, P, P, P, P, SZ, P], I),
    "spec_decode_rounds": ([P, P, P, I, P, P, I, I, I, I, F, I, U64, U64, I, P, P, P, P, P, P, SZ, P], I),
    "spec_decode_rounds_ex": ([P, P, P, I, P, P, I, I, I, I, F, I, U64, U64, I, P, P, P, P, P, I, P, SZ, P], I),
    "spec_status_str": ([I], ctypes.c_char_p),
    "spec_profile_enable": ([I], I),
    "spec_profile_reset": ([], I),
    "spec_profile_read": ([ctypes.c_char_p, P, P], I),
    "spec_profile_names": ([ctypes.c_char_p, I], I),
    "spec_philox_words": ([U64, U64, SZ, P, P], I),
}


def lib():
    """The loaded libspec.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libspec.so is not built (run draft_sampling_verify_amd.build.build()); "
                              "there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().spec_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != SPEC_OK:
        raise SpecError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError("%s must be %s %s, got %s %s" % (name, tuple(shape), dtype, tuple(t.shape), t.dtype))


def _draft_shapes(U, W1, W2p, x0):
    if U.dim() != 3 or U.dtype != torch.float32:
        raise ValueError("U must be float32 [R, gamma, V]")
    R, gamma, V = U.shape
    if W1.dim() != 2 or W1.shape[0] != V:
        raise ValueError("W1 must be [V, r]")
    r = W1.shape[1]
    nbytes = spec_packed_w2_bytes(_wdtype(W1), r, V)
    if W2p.dtype != torch.uint8 or W2p.dim() != 1 or W2p.numel() != nbytes:
        raise ValueError("W2p must be the uint8 tensor of %d bytes returned by spec_pack_w2" % nbytes)
    _need(x0, (R,), torch.int32, "x0")
    return R, gamma, V, r


def _wdtype(W):
    if W.dtype == torch.bfloat16:
        return SPEC_BF16
    if W.dtype == torch.float32:
        return SPEC_F32
    raise TypeError("weights must be torch.bfloat16 or torch.float32")


def spec_packed_w2_bytes(w_dtype, r, V) -> int:
    return int(lib().spec_packed_w2_bytes(w_dtype, r, V))


def spec_pack_w2(W2, out=None, stream=None):
    """Rearrange W2 [V, r] (bf16 or fp32) into the streamed layout; returns a
    uint8 tensor (do this once per weight)."""
    if W2.dim() != 2:
        raise ValueError("W2 must be [V, r]")
    V, r = W2.shape
    dt = _wdtype(W2)
    nbytes = spec_packed_w2_bytes(dt, r, V)
    if nbytes == 0:
        raise SpecError(SPEC_EINVAL, "spec_pack_w2")
    out = torch.empty(nbytes, dtype=torch.uint8, device=W2.device) if out is None else out
    _need(out, (nbytes,), torch.uint8, "out")
    _check(lib().spec_pack_w2(_ptr(W2), dt, r, V, _ptr(out), _stream(stream)), "spec_pack_w2")
    return out


def spec_pack_w2_rv(W2_rv, out=None, stream=None):
    """spec_pack_w2 for W2 held as the r x V matrix of B = W1[x] W2 (W2_rv
    [r, V]); returns the same packed tensor."""
    if W2_rv.dim() != 2:
        raise ValueError("W2_rv must be [r, V]")
    r, V = W2_rv.shape
    dt = _wdtype(W2_rv)
    nbytes = spec_packed_w2_bytes(dt, r, V)
    if nbytes == 0:
        raise SpecError(SPEC_EINVAL, "spec_pack_w2_rv")
    out = torch.empty(nbytes, dtype=torch.uint8, device=W2_rv.device) if out is None else out
    _need(out, (nbytes,), torch.uint8, "out")
    _check(lib().spec_pack_w2_rv(_ptr(W2_rv), dt, r, V, _ptr(out), _stream(stream)), "spec_pack_w2_rv")
    return out


def spec_workspace_bytes(op, R, gamma, r, V, B_max=0) -> int:
    return int(lib().spec_workspace_bytes(op, R, gamma, r, V, B_max))


class Workspace:
    """A device workspace (uint8 tensor) large enough for the given sizes of
    every operation, with its status word zeroed."""

    def __init__(self, R, gamma, r, V, B_max=0, device=None):
        need = max(spec_workspace_bytes(op, R, gamma, r, V, max(B_max, R))
                   for op in (SPEC_OP_PROPOSE, SPEC_OP_VERIFY, SPEC_OP_CONFIDENCE, SPEC_OP_ROUNDS, SPEC_OP_LOSS))
        if need == 0:
            raise SpecError(SPEC_EINVAL, "Workspace")
        self.tensor = torch.empty(need, dtype=torch.uint8, device=device or "cuda")
        spec_workspace_init(self)

    @property
    def nbytes(self):
        return self.tensor.numel()

    def ptr(self):
        return ctypes.c_void_p(self.tensor.data_ptr())


def _ws(ws, R, gamma, r, V, device):
    if ws is None:
        ws = Workspace(R, gamma, r, V, device=device)
    return ws


def spec_workspace_init(ws: Workspace, stream=None):
    _check(lib().spec_workspace_init(ws.ptr(), ws.nbytes, _stream(stream)), "spec_workspace_init")


def spec_device_status(ws: Workspace, stream=None, clear=False) -> int:
    flags = ctypes.c_int(0)
    st = lib().spec_device_status(ws.ptr(), _stream(stream), int(bool(clear)), ctypes.byref(flags))
    if st not in (SPEC_OK, SPEC_EDEVICE):
        raise SpecError(st, "spec_device_status")
    return flags.value


def spec_markov_propose(U, W1, W2p, x0, T, greedy=False, seed=1, round=0, x=None, pd_x=None,
                        pd_stats=None, ws=None, stream=None, path=SPEC_PATH_AUTO):
    """path != 0 calls spec_markov_propose_ex with those SPEC_PATH_* bits."""
    R, gamma, V, r = _draft_shapes(U, W1, W2p, x0)
    dev = U.device
    _need(x, (R, gamma), torch.int32, "x")
    _need(pd_x, (R, gamma), torch.float32, "pd_x")
    _need(pd_stats, (R, gamma, 2), torch.float32, "pd_stats")
    x = torch.empty((R, gamma), dtype=torch.int32, device=dev) if x is None else x
    pd_x = torch.empty((R, gamma), dtype=torch.float32, device=dev) if pd_x is None else pd_x
    pd_stats = torch.empty((R, gamma, 2), dtype=torch.float32, device=dev) if pd_stats is None else pd_stats
    ws = _ws(ws, R, gamma, r, V, dev)
    args = (_ptr(U), _ptr(W1), _ptr(W2p), _wdtype(W1), _ptr(x0), R, gamma, r, V, float(T), int(bool(greedy)),
            int(seed), int(round), _ptr(x), _ptr(pd_x), _ptr(pd_stats))
    if path:
        st = lib().spec_markov_propose_ex(*args, int(path), ws.ptr(), ws.nbytes, _stream(stream))
    else:
        st = lib().spec_markov_propose(*args, ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "spec_markov_propose")
    return x, pd_x, pd_stats


SPEC_NOALLOC_BYTES = 8 << 20


def spec_markov_propose_noalloc(U, W1, W2p, x0, T, greedy=False, seed=1, round=0, x=None, pd_x=None,
                                pd_stats=None, flags=None, stream=None):
    """spec_markov_propose with the library's static workspace (no device
    allocation inside the call; pass preallocated outputs to allocate
    nothing at all).  Returns (x, pd_x, pd_stats, flags [1] int32 device)."""
    R, gamma, V, r = _draft_shapes(U, W1, W2p, x0)
    dev = U.device
    _need(x, (R, gamma), torch.int32, "x")
    _need(pd_x, (R, gamma), torch.float32, "pd_x")
    _need(pd_stats, (R, gamma, 2), torch.float32, "pd_stats")
    _need(flags, (1,), torch.int32, "flags")
    x = torch.empty((R, gamma), dtype=torch.int32, device=dev) if x is None else x
    pd_x = torch.empty((R, gamma), dtype=torch.float32, device=dev) if pd_x is None else pd_x
    pd_stats = torch.empty((R, gamma, 2), dtype=torch.float32, device=dev) if pd_stats is None else pd_stats
    flags = torch.empty(1, dtype=torch.int32, device=dev) if flags is None else flags
    st = lib().spec_markov_propose_noalloc(_ptr(U), _ptr(W1), _ptr(W2p), _wdtype(W1), _ptr(x0), R, gamma, r, V,
                                           float(T), int(bool(greedy)), int(seed), int(round), _ptr(x), _ptr(pd_x),
                                           _ptr(pd_stats), _ptr(flags), _stream(stream))
    _check(st, "spec_markov_propose_noalloc")
    return x, pd_x, pd_stats, flags


def spec_verify(U, W1, W2p, x0, x, pd_stats, Lt, T, greedy=False, seed=1, round=0, ell=None,
                n_acc=None, y=None, pt_x=None, c_star=None, want_pt_x=True, want_c_star=True,
                ws=None, stream=None, path=SPEC_PATH_AUTO):
    """path != 0 calls spec_verify_ex with those SPEC_PATH_* bits."""
    R, gamma, V, r = _draft_shapes(U, W1, W2p, x0)
    dev = U.device
    _need(x, (R, gamma), torch.int32, "x")
    _need(pd_stats, (R, gamma, 2), torch.float32, "pd_stats")
    _need(Lt, (R, gamma + 1, V), torch.float32, "Lt")
    _need(ell, (R,), torch.int32, "ell")
    _need(n_acc, (R,), torch.int32, "n_acc")
    _need(y, (R, gamma + 1), torch.int32, "y")
    _need(pt_x, (R, gamma), torch.float32, "pt_x")
    _need(c_star, (R, gamma), torch.float32, "c_star")
    n_acc = torch.empty(R, dtype=torch.int32, device=dev) if n_acc is None else n_acc
    y = torch.empty((R, gamma + 1), dtype=torch.int32, device=dev) if y is None else y
    if pt_x is None and want_pt_x:
        pt_x = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    if c_star is None and want_c_star:
        c_star = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    ws = _ws(ws, R, gamma, r, V, dev)
    args = (_ptr(U), _ptr(W1), _ptr(W2p), _wdtype(W1), _ptr(x0), _ptr(x), _ptr(pd_stats), _ptr(Lt), _ptr(ell), R,
            gamma, r, V, float(T), int(bool(greedy)), int(seed), int(round), _ptr(n_acc), _ptr(y), _ptr(pt_x),
            _ptr(c_star))
    if path:
        st = lib().spec_verify_ex(*args, int(path), ws.ptr(), ws.nbytes, _stream(stream))
    else:
        st = lib().spec_verify(*args, ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "spec_verify")
    return n_acc, y, pt_x, c_star


def spec_decode_rounds(U, W1, W2p, x0, Lt, T, n_rounds, greedy=False, seed=1, round0=0, want_c_star=False,
                       anchors=None, x=None, n_acc=None, y=None, c_star=None, ws=None, stream=None,
                       path=SPEC_PATH_AUTO):
    """n_rounds propose + verify rounds on the device, each round's anchors
    being the previous round's last emitted tokens.  Returns (anchors
    [n+1, R], x [n, R, gamma], n_acc [n, R], y [n, R, gamma+1], c_star or
    None)."""
    R, gamma, V, r = _draft_shapes(U, W1, W2p, x0)
    dev = U.device
    n = int(n_rounds)
    _need(Lt, (R, gamma + 1, V), torch.float32, "Lt")
    _need(anchors, (n + 1, R), torch.int32, "anchors")
    _need(x, (n, R, gamma), torch.int32, "x")
    _need(n_acc, (n, R), torch.int32, "n_acc")
    _need(y, (n, R, gamma + 1), torch.int32, "y")
    _need(c_star, (n, R, gamma), torch.float32, "c_star")
    anchors = torch.empty((n + 1, R), dtype=torch.int32, device=dev) if anchors is None else anchors
    x = torch.empty((n, R, gamma), dtype=torch.int32, device=dev) if x is None else x
    n_acc = torch.empty((n, R), dtype=torch.int32, device=dev) if n_acc is None else n_acc
    y = torch.empty((n, R, gamma + 1), dtype=torch.int32, device=dev) if y is None else y
    if c_star is None and want_c_star:
        c_star = torch.empty((n, R, gamma), dtype=torch.float32, device=dev)
    ws = _ws(ws, R, gamma, r, V, dev)
    args = (_ptr(U), _ptr(W1), _ptr(W2p), _wdtype(W1), _ptr(x0), _ptr(Lt), R, gamma, r, V, float(T),
            int(bool(greedy)), int(seed), int(round0), n, _ptr(anchors), _ptr(x), _ptr(n_acc), _ptr(y), _ptr(c_star))
    if path:
        st = lib().spec_decode_rounds_ex(*args, int(path), ws.ptr(), ws.nbytes, _stream(stream))
    else:
        st = lib().spec_decode_rounds(*args, ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "spec_decode_rounds")
    return anchors, x, n_acc, y, c_star


def spec_confidence(U, W1, W2p, x0, x, Lt, T, pd_stats=None, c_star=None, a_star=None, want_a_star=True,
                    ws=None, stream=None, path=SPEC_PATH_AUTO):
    R, gamma, V, r = _draft_shapes(U, W1, W2p, x0)
    dev = U.device
    _need(x, (R, gamma), torch.int32, "x")
    _need(pd_stats, (R, gamma, 2), torch.float32, "pd_stats")
    _need(Lt, (R, gamma + 1, V), torch.float32, "Lt")
    _need(c_star, (R, gamma), torch.float32, "c_star")
    _need(a_star, (R, gamma), torch.float64, "a_star")
    c_star = torch.empty((R, gamma), dtype=torch.float32, device=dev) if c_star is None else c_star
    if a_star is None and want_a_star:
        a_star = torch.empty((R, gamma), dtype=torch.float64, device=dev)
    ws = _ws(ws, R, gamma, r, V, dev)
    args = (_ptr(U), _ptr(W1), _ptr(W2p), _wdtype(W1), _ptr(x0), _ptr(x), _ptr(pd_stats), _ptr(Lt), R, gamma, r, V,
            float(T), _ptr(c_star), _ptr(a_star))
    if path:
        st = lib().spec_confidence_ex(*args, int(path), ws.ptr(), ws.nbytes, _stream(stream))
    else:
        st = lib().spec_confidence(*args, ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "spec_confidence")
    return c_star, a_star


def spec_draft_loss(U, W1, W2p, x0, y, Lt, q, T, alphas=(0.1, 0.9, 1.0), loss=None, terms=None, dq=None,
                    want_terms=True, want_dq=True, ws=None, stream=None):
    """Training-side loss over the drafted positions, teacher-forced on the
    labels y.  Returns (loss [1] fp64, terms [R,gamma,3] fp32 or None,
    dq [R,gamma] fp32 or None)."""
    R, gamma, V, r = _draft_shapes(U, W1, W2p, x0)
    dev = U.device
    _need(y, (R, gamma), torch.int32, "y")
    _need(Lt, (R, gamma + 1, V), torch.float32, "Lt")
    _need(q, (R, gamma), torch.float32, "q")
    _need(loss, (1,), torch.float64, "loss")
    _need(terms, (R, gamma, 3), torch.float32, "terms")
    _need(dq, (R, gamma), torch.float32, "dq")
    loss = torch.empty(1, dtype=torch.float64, device=dev) if loss is None else loss
    if terms is None and want_terms:
        terms = torch.empty((R, gamma, 3), dtype=torch.float32, device=dev)
    if dq is None and want_dq:
        dq = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    ws = _ws(ws, R, gamma, r, V, dev)
    st = lib().spec_draft_loss(_ptr(U), _ptr(W1), _ptr(W2p), _wdtype(W1), _ptr(x0), _ptr(y), _ptr(Lt), _ptr(q), R,
                               gamma, r, V, float(T), float(alphas[0]), float(alphas[1]), float(alphas[2]),
                               _ptr(loss), _ptr(terms), _ptr(dq), ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "spec_draft_loss")
    return loss, terms, dq


# ------------------------------------------------------- clustered draft head

def spec_cluster_workspace_bytes(R, gamma, d, N_c, K_c, max_cl, V) -> int:
    return int(lib().spec_cluster_workspace_bytes(R, gamma, d, N_c, K_c, max_cl, V))


class ClusterWorkspace(Workspace):
    """A device workspace for spec_cluster_propose / spec_cluster_verify at
    these sizes, with its status word zeroed."""

    def __init__(self, R, gamma, d, N_c, K_c, max_cl, V, device=None):
        need = spec_cluster_workspace_bytes(R, gamma, d, N_c, K_c, max_cl, V)
        if need == 0:
            raise SpecError(SPEC_EINVAL, "ClusterWorkspace")
        self.tensor = torch.empty(need, dtype=torch.uint8, device=device or "cuda")
        spec_workspace_init(self)


def spec_cluster_index(cl_off, cl_tok, tok_slot=None, ws=None, stream=None):
    """tok_slot [V] int32 = (cluster << 16) | place of every token."""
    N_c, V = cl_off.numel() - 1, cl_tok.numel()
    _need(cl_off, (N_c + 1,), torch.int32, "cl_off")
    _need(cl_tok, (V,), torch.int32, "cl_tok")
    _need(tok_slot, (V,), torch.int32, "tok_slot")
    tok_slot = torch.empty(V, dtype=torch.int32, device=cl_tok.device) if tok_slot is None else tok_slot
    if ws is None:
        ws = ClusterWorkspace(1, 1, 16, 1, 1, 1, 1, device=cl_tok.device)
    st = lib().spec_cluster_index(_ptr(cl_off), _ptr(cl_tok), N_c, V, _ptr(tok_slot), ws.ptr(), ws.nbytes,
                                  _stream(stream))
    _check(st, "spec_cluster_index")
    return tok_slot


def spec_cluster_propose(H, C, E, cl_off, cl_tok, K_c, max_cl, T, greedy=False, seed=1, round=0, x=None,
                         pd_x=None, sel=None, zf=None, pd_stats=None, ws=None, stream=None):
    """Clustered draft head.  H [R,gamma,d], C [N_c,d], E [V,d] bf16.
    Returns (x, pd_x, sel, zf, pd_stats)."""
    if H.dim() != 3:
        raise ValueError("H must be [R, gamma, d]")
    R, gamma, d = H.shape
    N_c, V = C.shape[0], E.shape[0]
    for name, t, shape in (("C", C, (N_c, d)), ("E", E, (V, d))):
        _need(t, shape, H.dtype, name)
    _need(cl_off, (N_c + 1,), torch.int32, "cl_off")
    _need(cl_tok, (V,), torch.int32, "cl_tok")
    dev = H.device
    out = dict(x=(x, (R, gamma), torch.int32), pd_x=(pd_x, (R, gamma), torch.float32),
               sel=(sel, (R, gamma, K_c), torch.int32), zf=(zf, (R, gamma, K_c, max_cl), torch.float32),
               pd_stats=(pd_stats, (R, gamma, 2), torch.float32))
    res = {}
    for name, (t, shape, dt) in out.items():
        _need(t, shape, dt, name)
        res[name] = torch.empty(shape, dtype=dt, device=dev) if t is None else t
    if ws is None:
        ws = ClusterWorkspace(R, gamma, d, N_c, K_c, max_cl, V, device=dev)
    st = lib().spec_cluster_propose(_ptr(H), _ptr(C), _ptr(E), _wdtype(H), _ptr(cl_off), _ptr(cl_tok), R, gamma, d,
                                    N_c, int(K_c), int(max_cl), V, float(T), int(bool(greedy)), seed, round,
                                    _ptr(res["x"]), _ptr(res["pd_x"]), _ptr(res["sel"]), _ptr(res["zf"]),
                                    _ptr(res["pd_stats"]), ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "spec_cluster_propose")
    return res["x"], res["pd_x"], res["sel"], res["zf"], res["pd_stats"]


def spec_cluster_verify(tok_slot, sel, zf, pd_stats, x, Lt, T, N_c, greedy=False, seed=1, round=0, ell=None,
                        n_acc=None, y=None, pt_x=None, c_star=None, ws=None, stream=None, d=16):
    """Verify clustered-head drafts.  Returns (n_acc, y, pt_x, c_star)."""
    R, gamma, K_c, max_cl = zf.shape
    V = tok_slot.numel()
    dev = zf.device
    _need(tok_slot, (V,), torch.int32, "tok_slot")
    _need(sel, (R, gamma, K_c), torch.int32, "sel")
    _need(pd_stats, (R, gamma, 2), torch.float32, "pd_stats")
    _need(x, (R, gamma), torch.int32, "x")
    _need(Lt, (R, gamma + 1, V), torch.float32, "Lt")
    _need(ell, (R,), torch.int32, "ell")
    n_acc = torch.empty(R, dtype=torch.int32, device=dev) if n_acc is None else n_acc
    y = torch.empty((R, gamma + 1), dtype=torch.int32, device=dev) if y is None else y
    pt_x = torch.empty((R, gamma), dtype=torch.float32, device=dev) if pt_x is None else pt_x
    c_star = torch.empty((R, gamma), dtype=torch.float32, device=dev) if c_star is None else c_star
    if ws is None:
        ws = ClusterWorkspace(R, gamma, d, N_c, K_c, max_cl, V, device=dev)
    st = lib().spec_cluster_verify(_ptr(tok_slot), _ptr(sel), _ptr(zf), _ptr(pd_stats), _ptr(x), _ptr(Lt),
                                   _ptr(ell), R, gamma, int(N_c), K_c, max_cl, V, float(T), int(bool(greedy)), seed,
                                   round, _ptr(n_acc), _ptr(y), _ptr(pt_x), _ptr(c_star), ws.ptr(), ws.nbytes,
                                   _stream(stream))
    _check(st, "spec_cluster_verify")
    return n_acc, y, pt_x, c_star


def spec_schedule(c, sps, ell=None, a=None, K_star=None, theta_star=None, want_a=True, ws=None,
                  stream=None):
    if c.dim() != 2 or c.dtype != torch.float32:
        raise ValueError("c must be float32 [R, gamma]")
    R, gamma = c.shape
    if sps.dim() != 1 or sps.dtype != torch.float32:
        raise ValueError("sps must be float32 [B_max]")
    dev = c.device
    _need(ell, (R,), torch.int32, "ell")
    _need(a, (R, gamma), torch.float64, "a")
    ell = torch.empty(R, dtype=torch.int32, device=dev) if ell is None else ell
    if a is None and want_a:
        a = torch.empty((R, gamma), dtype=torch.float64, device=dev)
    K_star = torch.empty(1, dtype=torch.int32, device=dev) if K_star is None else K_star
    theta_star = torch.empty(1, dtype=torch.float64, device=dev) if theta_star is None else theta_star
    if ws is None:
        ws = Workspace(R, gamma, 16, 1, B_max=sps.numel(), device=dev)
    st = lib().spec_schedule(_ptr(c), R, gamma, _ptr(sps), sps.numel(), _ptr(ell), _ptr(a), _ptr(K_star),
                             _ptr(theta_star), ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "spec_schedule")
    return ell, a, K_star, theta_star


def spec_schedule_async(c, sps, K_hist, ell=None, a=None, K_used=None, K_star=None, theta_star=None, want_a=True,
                        ws=None, stream=None):
    """The production scheduler step.  K_hist: int32 [2] device tensor (the
    K* of the previous two calls, oldest first, -1 = none), updated in place.
    Returns (ell, a, K_used, K_star, theta_star)."""
    if c.dim() != 2 or c.dtype != torch.float32:
        raise ValueError("c must be float32 [R, gamma]")
    R, gamma = c.shape
    if sps.dim() != 1 or sps.dtype != torch.float32:
        raise ValueError("sps must be float32 [B_max]")
    dev = c.device
    _need(K_hist, (2,), torch.int32, "K_hist")
    _need(ell, (R,), torch.int32, "ell")
    _need(a, (R, gamma), torch.float64, "a")
    ell = torch.empty(R, dtype=torch.int32, device=dev) if ell is None else ell
    if a is None and want_a:
        a = torch.empty((R, gamma), dtype=torch.float64, device=dev)
    K_used = torch.empty(1, dtype=torch.int32, device=dev) if K_used is None else K_used
    K_star = torch.empty(1, dtype=torch.int32, device=dev) if K_star is None else K_star
    theta_star = torch.empty(1, dtype=torch.float64, device=dev) if theta_star is None else theta_star
    if ws is None:
        ws = Workspace(R, gamma, 16, 1, B_max=sps.numel(), device=dev)
    st = lib().spec_schedule_async(_ptr(c), R, gamma, _ptr(sps), sps.numel(), _ptr(K_hist), _ptr(ell), _ptr(a),
                                   _ptr(K_used), _ptr(K_star), _ptr(theta_star), ws.ptr(), ws.nbytes,
                                   _stream(stream))
    _check(st, "spec_schedule_async")
    return ell, a, K_used, K_star, theta_star


# ---- kernel timing (include/spec_debug.h)

def spec_profile_enable(on=True):
    _check(lib().spec_profile_enable(int(bool(on))), "spec_profile_enable")


def spec_profile_reset():
    _check(lib().spec_profile_reset(), "spec_profile_reset")


def spec_profile_read(kernel: str):
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(lib().spec_profile_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)), "spec_profile_read")
    return n.value, ms.value


def spec_profile_names():
    need = lib().spec_profile_names(None, 0)
    buf = ctypes.create_string_buffer(need + 1)
    lib().spec_profile_names(buf, need + 1)
    return [s for s in buf.value.decode().split(",") if s]


def spec_philox_words(seed, rnd, n, out=None, stream=None):
    """[n, 4] int32 tensor (uint32 bits): the kernels' Philox4x32-10 blocks
    at counters (i mod 2^16, i / 2^16, round) with key = seed."""
    out = torch.empty((n, 4), dtype=torch.int32, device="cuda") if out is None else out
    _need(out, (n, 4), torch.int32, "out")
    _check(lib().spec_philox_words(int(seed), int(rnd), int(n), _ptr(out), _stream(stream)), "spec_philox_words")
    return out

