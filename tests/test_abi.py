"""C-ABI checks that need no GPU: libspec.so loads, exports every entry
point that include/spec.h declares, and rejects bad arguments with the
documented status before enqueuing anything."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "spec_debug.h")]


@pytest.fixture(scope="module")
def L():
    import draft_sampling_verify_amd as d
    if not os.path.exists(d.LIB_PATH):
        from draft_sampling_verify_amd import build
        build.build()
    return d.lib()


def declared_symbols(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(spec_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_four_operations():
    names = declared_symbols()
    for n in ("spec_markov_propose", "spec_verify", "spec_confidence", "spec_schedule",
              "spec_workspace_bytes", "spec_status_str", "spec_device_status"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    import draft_sampling_verify_amd as d
    out = subprocess.run(["nm", "-D", "--defined-only", d.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(spec_\w+)$", out, flags=re.M))
    missing = [n for n in declared_symbols() if n not in exported]
    assert not missing, missing
    for n in declared_symbols():
        assert hasattr(L, n)


def test_status_strings(L):
    import draft_sampling_verify_amd as d
    assert d.spec_status_str(0) == "ok"
    for s in range(1, 7):
        assert d.spec_status_str(s) not in ("ok", "unknown status")
    assert d.spec_status_str(99) == "unknown status"


def test_workspace_bytes(L):
    import draft_sampling_verify_amd as d
    small = d.spec_workspace_bytes(d.SPEC_OP_VERIFY, 4, 4, 16, 1024)
    big = d.spec_workspace_bytes(d.SPEC_OP_VERIFY, 512, 16, 256, 129280)
    assert 0 < small < big
    assert d.spec_workspace_bytes(d.SPEC_OP_PROPOSE, 32, 7, 256, 129280) >= 32 * 1010 * 12
    assert d.spec_workspace_bytes(d.SPEC_OP_CONFIDENCE, 4, 4, 16, 1024) > 0
    assert d.spec_workspace_bytes(d.SPEC_OP_SCHEDULE, 512, 16, 0, 0, 8704) > 0
    # rejected sizes report 0
    assert d.spec_workspace_bytes(d.SPEC_OP_VERIFY, 4, 4, 17, 1024) == 0     # r % 16
    assert d.spec_workspace_bytes(d.SPEC_OP_VERIFY, 4, 0, 16, 1024) == 0     # gamma
    assert d.spec_workspace_bytes(d.SPEC_OP_SCHEDULE, 600, 16, 0, 0, 9000) == 0  # > 8192 entries
    assert d.spec_workspace_bytes(d.SPEC_OP_SCHEDULE, 8, 2, 0, 0, 7) == 0    # B_max < R
    assert d.spec_workspace_bytes(7, 4, 4, 16, 1024) == 0


FAKE = ctypes.c_void_p(4096)  # aligned, never dereferenced: validation fails first


def test_empty_batch_returns_before_any_device_call(L):
    """R = 0 is valid for every entry point but the scheduler: the size
    queries stay finite and the calls return SPEC_OK from host code alone
    (null data pointers; nothing is enqueued)."""
    import draft_sampling_verify_amd as d
    for op in (d.SPEC_OP_PROPOSE, d.SPEC_OP_VERIFY, d.SPEC_OP_CONFIDENCE, d.SPEC_OP_ROUNDS):
        assert d.spec_workspace_bytes(op, 0, 4, 16, 1024) > 0
    assert d.spec_workspace_bytes(d.SPEC_OP_SCHEDULE, 0, 4, 0, 0, 8) == 0
    assert d.spec_cluster_workspace_bytes(0, 2, 16, 6, 2, 20, 60) > 0
    big = 1 << 30
    assert L.spec_markov_propose(None, FAKE, FAKE, 1, None, 0, 4, 16, 1024, 1.0, 0, 1, 0, None, None, None,
                                 FAKE, big, None) == d.SPEC_OK
    assert L.spec_verify(None, FAKE, FAKE, 1, None, None, None, None, None, 0, 4, 16, 1024, 1.0, 0, 1, 0,
                         None, None, None, None, FAKE, big, None) == d.SPEC_OK
    assert L.spec_cluster_propose(None, None, None, 1, None, None, 0, 2, 16, 6, 2, 20, 60, 1.0, 0, 1, 0,
                                  None, None, None, None, None, FAKE, big, None) == d.SPEC_OK
    assert L.spec_cluster_verify(None, None, None, None, None, None, None, 0, 2, 6, 2, 20, 60, 1.0, 0, 1, 0,
                                 None, None, None, None, FAKE, big, None) == d.SPEC_OK


def _propose(L, **kw):
    a = dict(U=FAKE, W1=FAKE, W2=FAKE, dt=1, x0=FAKE, R=4, g=4, r=16, V=1024, T=1.0, greedy=0,
             seed=1, rnd=0, x=FAKE, pdx=FAKE, pds=FAKE, ws=FAKE, wsb=1 << 30, s=None)
    a.update(kw)
    return L.spec_markov_propose(*a.values())


def test_propose_validation(L):
    import draft_sampling_verify_amd as d
    assert _propose(L, dt=5) == d.SPEC_EDTYPE
    assert _propose(L, R=-1) == d.SPEC_EINVAL
    assert _propose(L, g=0) == d.SPEC_EINVAL
    assert _propose(L, r=8) == d.SPEC_EINVAL
    assert _propose(L, r=24) == d.SPEC_EINVAL
    assert _propose(L, V=0) == d.SPEC_EINVAL
    assert _propose(L, T=0.0) == d.SPEC_EINVAL
    assert _propose(L, T=float("nan")) == d.SPEC_EINVAL
    assert _propose(L, T=float("inf")) == d.SPEC_EINVAL
    assert _propose(L, U=None) == d.SPEC_EINVAL
    assert _propose(L, x=None) == d.SPEC_EINVAL
    assert _propose(L, U=ctypes.c_void_p(4100)) == d.SPEC_EINVAL           # misaligned
    assert _propose(L, g=65) == d.SPEC_EUNSUPPORTED
    assert _propose(L, r=528) == d.SPEC_EUNSUPPORTED
    assert _propose(L, dt=0, r=272) == d.SPEC_EUNSUPPORTED               # fp32 weights: r <= 256
    assert _propose(L, V=(1 << 24) + 1) == d.SPEC_EUNSUPPORTED
    assert _propose(L, ws=None) == d.SPEC_EWORKSPACE
    assert _propose(L, wsb=100) == d.SPEC_EWORKSPACE
    # empty batch: nothing to enqueue
    assert _propose(L, R=0, U=None, W1=None, W2=None, x0=None, x=None, pdx=None, pds=None) == d.SPEC_OK


def test_path_flags(L):
    """The _ex entry points take the kernel path per call: unknown bits are
    rejected before anything is enqueued; known bits pass validation (an
    empty batch then returns at once).  No process-wide switch exists."""
    import draft_sampling_verify_amd as d
    F = FAKE
    for name in ("spec_set_propose_fused", "spec_set_verify_lds"):
        assert not hasattr(L, name) or name not in declared_symbols()
    base = [F, F, F, 1, F, 4, 4, 16, 1024, 1.0, 0, 1, 0, F, F, F]
    assert L.spec_markov_propose_ex(*base, 4, F, 1 << 30, None) == d.SPEC_EINVAL
    assert L.spec_markov_propose_ex(*base, -1, F, 1 << 30, None) == d.SPEC_EINVAL
    empty = [None, F, F, 1, None, 0, 4, 16, 1024, 1.0, 0, 1, 0, None, None, None]
    for path in (d.SPEC_PATH_AUTO, d.SPEC_PATH_NO_FUSED_PROPOSE, d.SPEC_PATH_NO_PIPELINED_SWEEP, 3):
        assert L.spec_markov_propose_ex(*empty, path, F, 1 << 30, None) == d.SPEC_OK
    vargs = [F, F, F, 1, F, F, F, F, None, 4, 4, 16, 1024, 1.0, 0, 1, 0, F, F, None, None]
    assert L.spec_verify_ex(*vargs, 8, F, 1 << 30, None) == d.SPEC_EINVAL
    cargs = [F, F, F, 1, F, F, None, F, 4, 4, 16, 1024, 1.0, F, None]
    assert L.spec_confidence_ex(*cargs, 16, F, 1 << 30, None) == d.SPEC_EINVAL
    need = d.spec_workspace_bytes(d.SPEC_OP_ROUNDS, 4, 4, 16, 1024)
    rargs = [F, F, F, 1, F, F, 4, 4, 16, 1024, 1.0, 0, 1, 0, 3, F, F, F, F, None]
    assert L.spec_decode_rounds_ex(*rargs, 32, F, need, None) == d.SPEC_EINVAL


def test_pack_validation(L):
    import draft_sampling_verify_amd as d
    assert L.spec_packed_w2_bytes(1, 256, 129280) == 129280 * 256 * 2
    assert L.spec_packed_w2_bytes(1, 16, 1001) == 32 * 32 * 16 * 2      # padded to 32-id blocks
    assert L.spec_packed_w2_bytes(0, 16, 5) == 32 * 16 * 4
    assert L.spec_packed_w2_bytes(1, 24, 100) == 0
    assert L.spec_packed_w2_bytes(3, 16, 100) == 0
    assert L.spec_pack_w2(FAKE, 1, 16, 100, None, None) == d.SPEC_EINVAL
    assert L.spec_pack_w2(FAKE, 1, 16, 100, ctypes.c_void_p(4100), None) == d.SPEC_EINVAL
    assert L.spec_pack_w2(FAKE, 4, 16, 100, FAKE, None) == d.SPEC_EDTYPE
    assert L.spec_pack_w2(FAKE, 1, 16, 0, FAKE, None) == d.SPEC_EINVAL
    assert L.spec_pack_w2_rv(FAKE, 1, 16, 100, None, None) == d.SPEC_EINVAL
    assert L.spec_pack_w2_rv(FAKE, 1, 24, 100, FAKE, None) == d.SPEC_EINVAL
    assert L.spec_pack_w2_rv(FAKE, 4, 16, 100, FAKE, None) == d.SPEC_EDTYPE


def test_verify_confidence_schedule_validation(L):
    import draft_sampling_verify_amd as d
    F = FAKE
    args = [F, F, F, 1, F, F, F, F, None, 4, 4, 16, 1024, 1.0, 0, 1, 0, F, F, None, None, F, 1 << 30, None]
    assert L.spec_verify(*args[:6], None, *args[7:]) == d.SPEC_EINVAL      # pd_stats required
    a2 = list(args); a2[7] = ctypes.c_void_p(4104)
    assert L.spec_verify(*a2) == d.SPEC_EINVAL                             # Lt misaligned
    a3 = list(args); a3[22] = 64
    assert L.spec_verify(*a3) == d.SPEC_EWORKSPACE
    cargs = [F, F, F, 1, F, F, None, F, 4, 4, 16, 1024, 1.0, None, None, F, 1 << 30, None]
    assert L.spec_confidence(*cargs) == d.SPEC_EINVAL                      # c_star required
    sargs = [F, 4, 4, F, 20, F, None, F, F, F, 1 << 20, None]
    s2 = list(sargs); s2[4] = 3
    assert L.spec_schedule(*s2) == d.SPEC_EINVAL                           # B_max < R
    s3 = list(sargs); s3[1] = 4096; s3[4] = 100000
    assert L.spec_schedule(*s3) == d.SPEC_EUNSUPPORTED                     # R*gamma > 8192
    s4 = list(sargs); s4[9] = None
    assert L.spec_schedule(*s4) == d.SPEC_EWORKSPACE
    s5 = list(sargs); s5[5] = None
    assert L.spec_schedule(*s5) == d.SPEC_EINVAL                           # ell required


def test_decode_rounds_validation(L):
    import draft_sampling_verify_amd as d
    F = FAKE
    need = d.spec_workspace_bytes(d.SPEC_OP_ROUNDS, 4, 4, 16, 1024)
    assert need > max(d.spec_workspace_bytes(d.SPEC_OP_PROPOSE, 4, 4, 16, 1024),
                      d.spec_workspace_bytes(d.SPEC_OP_VERIFY, 4, 4, 16, 1024))
    args = [F, F, F, 1, F, F, 4, 4, 16, 1024, 1.0, 0, 1, 0, 3, F, F, F, F, None, F, need, None]
    a0 = list(args); a0[14] = 0
    assert L.spec_decode_rounds(*a0) == d.SPEC_EINVAL                       # n_rounds
    a1 = list(args); a1[21] = need - 1
    assert L.spec_decode_rounds(*a1) == d.SPEC_EWORKSPACE
    a2 = list(args); a2[15] = None
    assert L.spec_decode_rounds(*a2) == d.SPEC_EINVAL                       # anchors required
    a3 = list(args); a3[5] = ctypes.c_void_p(4100)
    assert L.spec_decode_rounds(*a3) == d.SPEC_EINVAL                       # Lt misaligned


def test_binding_rejects_bad_shapes_without_a_gpu():
    import torch
    import draft_sampling_verify_amd as d
    U = torch.zeros(2, 3, 8)
    W = torch.zeros(7, 16)   # V mismatch
    with pytest.raises(ValueError):
        d.spec_markov_propose(U, W, W, torch.zeros(2, dtype=torch.int32), 1.0)
