"""Seeded synthetic inputs for the speculative-decoding output side.

This module is the only code shared by the HIP library's callers (tests,
bench) and the CPU oracle: it draws random numbers and lays them out, and
holds none of the method's arithmetic.

Every array is a pure function of (config index, tensor tag, request index),
drawn with numpy's PCG64 from ``SeedSequence([config, tag, request])``, so
any subset of requests can be regenerated on its own (the oracle checks
sampled requests at the large sizes) and generation runs in a thread pool.

Workloads (sizes and distributions of the five measured configurations;
"N(m, s)" means standard deviation s):

  tiny    R=4,   gamma=4,  V=1024,   r=16,  fp32 weights, U~N(0,2),
          Lt = U_ext + N(0,0.5), W~N(0,0.05), T=1
  c2      R=32,  gamma=7,  V=129280, r=256, bf16 weights, U~N(0,3),
          Lt = U_ext + N(0,1), W~N(0,0.02), T=1
  c3      R=256, gamma=7,  V=129280, r=256, as c2 with per-request noise
          sigma_r ~ U[0.3, 2]
  c4      R=512, gamma=16, V=129280, r=256, as c2, plus confidences
          c = sigmoid(N(1.5,1)) and a sawtooth SPS table for B = 1..8704
  c5      R=64,  gamma=8,  V=262144, r=256, bf16, U~N(0,3) plus +8 at 32
          distinct random ids of every row (bonus row included),
          Lt = U_ext + N(0,0.7), T=0.7

U_ext has gamma+1 rows per request: the gamma base rows of U and one more
row drawn the same way for the bonus position.  bf16 weights are produced
from fp32 draws by round-to-nearest-even and returned as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor tags of the seed sequences
(_TAG_U, _TAG_NOISE, _TAG_W1, _TAG_W2, _TAG_X0, _TAG_SIGMA, _TAG_C, _TAG_SPS, _TAG_PEAK, _TAG_Y, _TAG_Q,
 _TAG_CL_PERM, _TAG_CL_SIZE, _TAG_CL_MU, _TAG_CL_EPS, _TAG_CL_H, _TAG_CL_HT) = range(17)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int            # seed of every stream of this workload
    R: int
    gamma: int
    V: int
    r: int
    bf16: bool
    T: float
    u_std: float
    w_std: float
    noise_std: float      # target noise std (ignored when sigma_range is set)
    sigma_range: tuple | None = None   # per-request noise std ~ U[lo, hi]
    peaks: int = 0        # planted peaks per row
    peak_height: float = 0.0
    confidences: bool = False          # draw c = sigmoid(N(1.5, 1))
    sps_len: int = 0                   # sawtooth SPS table length (0 = none)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", 1, 4, 4, 1024, 16, False, 1.0, 2.0, 0.05, 0.5,
                   confidences=True, sps_len=20),
    "c2": Config("c2", 2, 32, 7, 129280, 256, True, 1.0, 3.0, 0.02, 1.0),
    "c3": Config("c3", 3, 256, 7, 129280, 256, True, 1.0, 3.0, 0.02, 1.0,
                 sigma_range=(0.3, 2.0)),
    "c4": Config("c4", 4, 512, 16, 129280, 256, True, 1.0, 3.0, 0.02, 1.0,
                 confidences=True, sps_len=512 * 17),
    "c5": Config("c5", 5, 64, 8, 262144, 256, True, 0.7, 3.0, 0.02, 0.7,
                 peaks=32, peak_height=8.0),
}


def _rng(cfg: Config, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.index, tag, idx])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    if not np.isfinite(a).all():
        raise ValueError("to_bf16_bits expects finite values")
    # finite inputs cannot overflow 32 bits here (largest is 0xFF7FFFFF + 0x8000)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


_WCHUNK = 4096   # vocabulary rows per weight stream


def _weight(cfg: Config, tag: int) -> np.ndarray:
    out = np.empty((cfg.V, cfg.r), np.uint16 if cfg.bf16 else np.float32)

    def fill(c):
        lo, hi = c * _WCHUNK, min(cfg.V, (c + 1) * _WCHUNK)
        w = _rng(cfg, tag, c).standard_normal((hi - lo, cfg.r), dtype=np.float32)
        w *= np.float32(cfg.w_std)
        out[lo:hi] = to_bf16_bits(w) if cfg.bf16 else w

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range((cfg.V + _WCHUNK - 1) // _WCHUNK)))
    return out


def weights(cfg: Config):
    """W1 [V, r] and W2 [V, r] (fp32, or bf16 bits as uint16)."""
    return _weight(cfg, _TAG_W1), _weight(cfg, _TAG_W2)


def anchors(cfg: Config) -> np.ndarray:
    return _rng(cfg, _TAG_X0).integers(0, cfg.V, size=cfg.R, dtype=np.int64).astype(np.int32)


def sigmas(cfg: Config) -> np.ndarray:
    if cfg.sigma_range is None:
        return np.full(cfg.R, cfg.noise_std, np.float32)
    lo, hi = cfg.sigma_range
    return _rng(cfg, _TAG_SIGMA).uniform(lo, hi, size=cfg.R).astype(np.float32)


def confidences(cfg: Config) -> np.ndarray:
    """c_{r,k} = sigmoid(N(1.5, 1)) as float32 [R, gamma]."""
    n = _rng(cfg, _TAG_C).normal(1.5, 1.0, size=(cfg.R, cfg.gamma))
    return (1.0 / (1.0 + np.exp(-n))).astype(np.float32)


def loss_labels(cfg: Config) -> np.ndarray:
    """Training labels y [R, gamma] int32, uniform over the vocabulary."""
    return _rng(cfg, _TAG_Y).integers(0, cfg.V, size=(cfg.R, cfg.gamma), dtype=np.int64).astype(np.int32)


def confidence_logits(cfg: Config) -> np.ndarray:
    """Confidence-head logits q [R, gamma] = N(0, 1.5^2) as float32."""
    return _rng(cfg, _TAG_Q).normal(0.0, 1.5, size=(cfg.R, cfg.gamma)).astype(np.float32)


def sawtooth_sps(cfg: Config, length: int | None = None) -> np.ndarray:
    """Decreasing sawtooth SPS(B), B = 1..length: flat within each 64-token
    step apart from a slight slope, a drop at every multiple of 64, and a
    +-8% jitter drawn once per step."""
    n = cfg.sps_len if length is None else length
    B = np.arange(1, n + 1, dtype=np.float64)
    step = np.ceil(B / 64.0)
    eps = _rng(cfg, _TAG_SPS).uniform(-1.0, 1.0, size=int(step.max()) + 1)
    sps = 1000.0 * (1.0 + 0.08 * eps[step.astype(np.int64)]) / (20.0 + 0.25 * step + 0.001 * B)
    return sps.astype(np.float32)


def _request_rows(cfg: Config, req: int, sigma: float):
    """(U_ext [gamma+1, V], Lt [gamma+1, V]) of one request."""
    g1 = cfg.gamma + 1
    u = _rng(cfg, _TAG_U, req).standard_normal((g1, cfg.V), dtype=np.float32)
    u *= np.float32(cfg.u_std)
    if cfg.peaks:
        pr = _rng(cfg, _TAG_PEAK, req)
        for k in range(g1):
            ids = pr.choice(cfg.V, size=cfg.peaks, replace=False)
            u[k, ids] += np.float32(cfg.peak_height)
    noise = _rng(cfg, _TAG_NOISE, req).standard_normal((g1, cfg.V), dtype=np.float32)
    noise *= np.float32(sigma)
    return u, u + noise


def request_rows(cfg: Config, requests, threads: int | None = None):
    """(U [n, gamma, V], Lt [n, gamma+1, V]) float32 of the listed requests,
    in that order: the per-request part of make(), so that large inputs can
    be built a slice of requests at a time."""
    req = np.asarray(list(requests), dtype=np.int32)
    n = req.size
    U = np.empty((n, cfg.gamma, cfg.V), np.float32)
    Lt = np.empty((n, cfg.gamma + 1, cfg.V), np.float32)
    sig = sigmas(cfg)

    def fill(i):
        u, lt = _request_rows(cfg, int(req[i]), float(sig[req[i]]))
        U[i] = u[: cfg.gamma]
        Lt[i] = lt

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(fill, range(n)))
    return U, Lt


def make(cfg: Config | str, requests=None, threads: int | None = None) -> dict:
    """Build the inputs of a workload.

    requests: None for all R requests, else an iterable of request indices;
    the returned per-request arrays then hold only those rows, in that order,
    and 'req_ids' names them (the Philox request index of each row).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    req = np.arange(cfg.R, dtype=np.int32) if requests is None else \
        np.asarray(list(requests), dtype=np.int32)
    U, Lt = request_rows(cfg, req, threads)
    W1, W2 = weights(cfg)
    out = dict(cfg=cfg, req_ids=req, U=U, Lt=Lt, W1=W1, W2=W2,
               x0=anchors(cfg)[req], T=np.float32(cfg.T))
    if cfg.confidences:
        out["c"] = confidences(cfg)[req]
    if cfg.sps_len:
        out["sps"] = sawtooth_sps(cfg)
    return out


# ------------------------------------------------------ clustered draft head
#
# Inputs of the clustered head: the vocabulary is split into N_c clusters by
# a seeded permutation (equal sizes, or sizes 1 + multinomial); each token's
# LM-head row is its cluster's mean plus noise, E_v = mu_c + eps_v (coherent
# clusters, as an embedding clustered by k-means would give), rounded to
# bf16; the centres C_c are the means of their clusters' bf16 rows, rounded
# to bf16; hidden rows H ~ N(0, h_std); the target's logits are those of a
# perturbed hidden state through the same rows, Lt = (H + N(0, t_std)) E^T
# (the bonus row from its own draw), fp32.


@dataclasses.dataclass(frozen=True)
class ClusterConfig:
    name: str
    index: int
    R: int
    gamma: int
    d: int
    V: int
    N_c: int
    K_c: int
    T: float
    equal: bool = True     # equal cluster sizes (V % N_c == 0), else 1 + multinomial
    mu_std: float = 0.07
    eps_std: float = 0.03
    h_std: float = 1.0
    t_std: float = 0.5

    def replace(self, **kw) -> "ClusterConfig":
        return dataclasses.replace(self, **kw)


CLUSTER_CONFIGS = {
    # Gemma 4 E2B-like drafter head: 262144-token vocabulary, hidden 1536,
    # 2048 centres, the top 32 expanded; 4 requests of 8 drafted tokens
    "gemma_e2b": ClusterConfig("gemma_e2b", 60, 4, 8, 1536, 262144, 2048, 32, 1.0, t_std=0.1),
    "cl_tiny": ClusterConfig("cl_tiny", 61, 3, 2, 16, 60, 6, 2, 1.0, equal=False, mu_std=0.5, eps_std=0.3),
    "cl_ragged": ClusterConfig("cl_ragged", 62, 5, 3, 48, 1001, 40, 5, 0.8, equal=False, mu_std=0.4,
                               eps_std=0.2),
    "cl_mid": ClusterConfig("cl_mid", 63, 4, 4, 256, 20000, 160, 8, 1.0, equal=False, mu_std=0.15,
                            eps_std=0.08),
    "cl_rows": ClusterConfig("cl_rows", 64, 40, 2, 64, 4096, 64, 8, 1.0, mu_std=0.3, eps_std=0.15),
    # long expansions: 16 clusters of 1000 tokens (16000 per row), and the
    # largest the interface takes, 16 x 4096 = 65536 tokens per row
    "cl_wide": ClusterConfig("cl_wide", 65, 3, 2, 32, 40000, 40, 16, 1.0, mu_std=0.3, eps_std=0.15),
    "cl_max": ClusterConfig("cl_max", 66, 3, 2, 32, 262144, 64, 16, 1.0, mu_std=0.3, eps_std=0.15),
}


def _crng(cfg: ClusterConfig, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.index, tag, idx])))


def make_cluster(cfg: ClusterConfig | str) -> dict:
    """H [R,gamma,d], C [N_c,d], E [V,d] (bf16 bits, uint16), cl_off [N_c+1],
    cl_tok [V] (int32), Lt [R,gamma+1,V] fp32, and max_cl."""
    if isinstance(cfg, str):
        cfg = CLUSTER_CONFIGS[cfg]
    V, N_c, d = cfg.V, cfg.N_c, cfg.d
    perm = _crng(cfg, _TAG_CL_PERM).permutation(V).astype(np.int32)
    if cfg.equal:
        sizes = np.full(N_c, V // N_c, np.int64)
    else:
        sizes = 1 + _crng(cfg, _TAG_CL_SIZE).multinomial(V - N_c, np.full(N_c, 1.0 / N_c))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    clus = np.empty(V, np.int64)
    clus[perm] = np.repeat(np.arange(N_c), sizes)           # cluster of each token
    mu = _crng(cfg, _TAG_CL_MU).standard_normal((N_c, d), dtype=np.float32) * np.float32(cfg.mu_std)
    E = np.empty((V, d), np.uint16)

    def fill(c):
        lo, hi = c * _WCHUNK, min(V, (c + 1) * _WCHUNK)
        e = _crng(cfg, _TAG_CL_EPS, c).standard_normal((hi - lo, d), dtype=np.float32)
        e *= np.float32(cfg.eps_std)
        e += mu[clus[lo:hi]]
        E[lo:hi] = to_bf16_bits(e)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range((V + _WCHUNK - 1) // _WCHUNK)))
    Ef = bf16_bits_to_f32(E)
    # cluster c's rows are Ef[perm[off[c]:off[c+1]]]
    sums = np.add.reduceat(Ef[perm], off[:-1], axis=0)
    C = to_bf16_bits((sums / sizes[:, None].astype(np.float32)).astype(np.float32))
    H = to_bf16_bits(_crng(cfg, _TAG_CL_H).standard_normal((cfg.R, cfg.gamma, d), dtype=np.float32)
                     * np.float32(cfg.h_std))
    Hf = bf16_bits_to_f32(H)
    ht = _crng(cfg, _TAG_CL_HT).standard_normal((cfg.R, cfg.gamma + 1, d), dtype=np.float32)
    ht[:, : cfg.gamma] = Hf + np.float32(cfg.t_std) * ht[:, : cfg.gamma]
    ht[:, cfg.gamma] *= np.float32(cfg.h_std)
    Lt = (ht.reshape(-1, d) @ Ef.T).reshape(cfg.R, cfg.gamma + 1, V).astype(np.float32)
    return dict(cfg=cfg, H=H, C=C, E=E, cl_off=off, cl_tok=perm, Lt=Lt, max_cl=int(sizes.max()))

