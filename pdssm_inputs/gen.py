"""Seeded generators for the five PD-SSM workloads (see ``configs.py``).

Draw order for a workload with seed ``s``.  ``SeedSequence(s)`` seeds the
parameter generator (numpy PCG64), which draws, in this order:

1. dictionary   ``integers(0, N, (H, K, N))``; rule ``identity0`` then
                overwrites k = 0 with the identity map
2. W_sel        ``standard_normal((H, K, d)) * sqrt(1/d)``
3. W_d          ``standard_normal((H, N, d)) * sqrt(1/d)``
4. W_b          ``standard_normal((H, N, d)) * sqrt(1/d)``
5. C            ``standard_normal((H, N)) * sqrt(1/N)``
6. sinusoid parameters (amplitude, log-period, phase; each (B, H, d, 3)),
   for the sinusoid rule only.

u is then drawn per row sequence -- (b, h) in row-major order for per-head
inputs, b for a shared input -- each from its own child generator
``SeedSequence(s).spawn(n_sequences)[i]``: ``standard_normal((L, d))`` scaled,
plus the deterministic part, followed by that sequence's redraw rounds.  The
sequences are independent, so they may be generated on several threads with
identical results.

Values are formed in fp64 and rounded to fp32 (round to nearest even); for
``dtype == "bf16"`` u, W_sel, W_d and W_b are further rounded from fp32 to
bf16 (round to nearest even) and carried as fp32 arrays holding bf16 values,
so that every consumer reads exactly the same numbers.

Redraw rule.  An input row is one u vector that owns a set of scores: u[b,h,t]
for per-head inputs, u[b,t] (all H heads at once) for a shared input.  A row is
accepted when, for every head that reads it, the two largest of the K linear
forms W_sel[h] @ u (evaluated in fp64 on the rounded values) differ by at least
``GAP``.  Rejected rows get a fresh random component (drawn for all rejected
rows of a sequence at once, in ascending step order) and are tested again, up to
``MAX_ROUNDS`` rounds.  This is input conditioning only: nothing here decides a
selection that a consumer is compared against.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

from .configs import Config

GAP = 1e-3
MAX_ROUNDS = 10_000


# --------------------------------------------------------------------------
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 encoding of fp32 values, round to nearest even.  Inputs
    must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 array holding the bf16 (RNE) rounding of ``x``."""
    bits = bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    return bf16_round(x32) if dtype == "bf16" else x32


def top2_margin(scores: np.ndarray) -> np.ndarray:
    """Difference between the largest and second-largest entry along the last
    axis (0 when they tie)."""
    if scores.shape[-1] < 2:
        return np.full(scores.shape[:-1], np.inf)
    part = np.partition(scores, -2, axis=-1)
    return part[..., -1] - part[..., -2]


# --------------------------------------------------------------------------
# generated bundle
# --------------------------------------------------------------------------

@dataclass
class Inputs:
    cfg: Config
    u: np.ndarray          # f32 [B,H,L,d] or [B,L,d]
    W_sel: np.ndarray      # f32 [H,K,d]
    W_d: np.ndarray        # f32 [H,N,d]
    W_b: np.ndarray        # f32 [H,N,d]
    b_d: np.ndarray        # f32 [H,N]
    dict_idx: np.ndarray   # i32 [H,K,N]
    C: np.ndarray          # f32 [H,N]
    h0: np.ndarray         # f32 [B,H,N]
    Bu: np.ndarray         # f32 [B,H,L,N]
    rounds: int = 0
    redrawn_rows: int = 0
    info: dict = field(default_factory=dict)


def _dictionary(rng, cfg: Config) -> np.ndarray:
    dic = rng.integers(0, cfg.N, size=(cfg.H, cfg.K, cfg.N)).astype(np.int32)
    if cfg.dict_rule == "identity0":
        dic[:, 0, :] = np.arange(cfg.N, dtype=np.int32)
    elif cfg.dict_rule != "uniform":
        raise ValueError(f"unknown dictionary rule {cfg.dict_rule!r}")
    return dic


def _u_rule(rng, cfg: Config):
    """Return (base, noise scale).  ``base`` is the deterministic part of u:
    None (zero), the string "impulse" (e_0 at t = 0), or a callable
    (b, h) -> [L, d] fp64 for the sinusoid rule, whose parameters are drawn
    here from the parameter generator."""
    if cfg.u_rule == "normal":
        return None, 1.0
    if cfg.u_rule == "impulse":
        return "impulse", 1e-3
    if cfg.u_rule == "sinusoid":
        if cfg.u_shared:
            raise ValueError("sinusoid rule is defined for per-head inputs")
        pshape = (cfg.B, cfg.H, cfg.d, 3)
        amp = rng.uniform(0.5, 1.5, pshape)
        omega = 2.0 * math.pi / np.exp(rng.uniform(math.log(8.0), math.log(4096.0), pshape))
        phase = rng.uniform(0.0, 2.0 * math.pi, pshape)
        return (lambda b, h: _sinusoids(cfg.L, amp[b, h], omega[b, h], phase[b, h])), math.sqrt(0.1)
    raise ValueError(f"unknown input rule {cfg.u_rule!r}")


def _sinusoids(L, amp, omega, phase, block=128):
    """[L, d] with entry (t, c) = sum_m amp[c,m] sin(omega[c,m] t + phase[c,m]),
    in fp64 by angle addition over blocks of ``block`` steps:
    sin(A + omega tau) = sin(A) cos(omega tau) + cos(A) sin(omega tau) with
    A = omega t0 + phase.  Agrees with direct evaluation to a few fp64 ulps."""
    tau = np.arange(block, dtype=np.float64)[:, None, None]
    s_tau, c_tau = np.sin(omega * tau), np.cos(omega * tau)   # [blk, d, 3]
    out = np.empty((L, amp.shape[0]))
    for t0 in range(0, L, block):
        n = min(block, L - t0)
        A = omega * t0 + phase
        out[t0:t0 + n] = (amp * np.sin(A) * c_tau[:n] + amp * np.cos(A) * s_tau[:n]).sum(-1)
    return out


def _sequence(cfg, rng, base, scale, W64, Wb64):
    """Draw one row sequence of u ([L, d]) from its own generator and apply the
    redraw rule to it; return (u_rows f32 [L, d], Bu [H_read, L, N], rounds,
    redrawn).  ``W64`` holds the score forms of the heads that read these rows
    ([n_heads, K, d], fp64); ``Wb64`` the matching driving matrices."""
    z = rng.standard_normal((cfg.L, cfg.d))
    z *= scale
    if isinstance(base, str):                      # impulse: e_0 at step 0
        z[0, 0] += 1.0
    elif base is not None:
        z += base
    u = _store(z, cfg.dtype)
    del z
    rounds = redrawn = 0
    if cfg.K >= 2:
        Wflat = W64.reshape(-1, cfg.d).T           # [d, n_heads*K]

        def margins(rows_u):
            s = rows_u.astype(np.float64) @ Wflat
            return top2_margin(s.reshape(rows_u.shape[0], -1, cfg.K)).min(axis=1)

        bad = np.flatnonzero(margins(u) < GAP)
        while bad.size:
            rounds += 1
            if rounds > MAX_ROUNDS:
                raise RuntimeError(
                    f"{cfg.name}: {bad.size} rows still below the score margin "
                    f"after {MAX_ROUNDS} redraw rounds")
            redrawn += bad.size
            z = rng.standard_normal((bad.size, cfg.d))
            z *= scale
            if isinstance(base, str):
                z[bad == 0, 0] += 1.0
            elif base is not None:
                z += base[bad]
            u[bad] = _store(z, cfg.dtype)
            bad = bad[margins(u[bad]) < GAP]
    u64 = u.astype(np.float64)
    Bu = np.stack([(u64 @ Wb.T).astype(np.float32) for Wb in Wb64])
    return u, Bu, rounds, redrawn


def generate(cfg: Config, *, threads: int | None = None) -> Inputs:
    """Draw one workload.  Deterministic in ``cfg`` (seed included) and
    independent of ``threads``."""
    ss = np.random.SeedSequence(cfg.seed)
    rng = np.random.default_rng(ss)
    dic = _dictionary(rng, cfg)
    W_sel = _store(rng.standard_normal((cfg.H, cfg.K, cfg.d)) * math.sqrt(1.0 / cfg.d), cfg.dtype)
    W_d = _store(rng.standard_normal((cfg.H, cfg.N, cfg.d)) * math.sqrt(1.0 / cfg.d), cfg.dtype)
    W_b = _store(rng.standard_normal((cfg.H, cfg.N, cfg.d)) * math.sqrt(1.0 / cfg.d), cfg.dtype)
    C = _store(rng.standard_normal((cfg.H, cfg.N)) * math.sqrt(1.0 / cfg.N), "f32")
    b_d = np.full((cfg.H, cfg.N), cfg.b_d, dtype=np.float32)
    h0 = np.zeros((cfg.B, cfg.H, cfg.N), dtype=np.float32)
    base, scale = _u_rule(rng, cfg)

    W64 = W_sel.astype(np.float64)
    Wb64 = W_b.astype(np.float64)
    if cfg.u_shared:
        seqs = [(b, None) for b in range(cfg.B)]
        u = np.empty((cfg.B, cfg.L, cfg.d), dtype=np.float32)
    else:
        seqs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
        u = np.empty((cfg.B, cfg.H, cfg.L, cfg.d), dtype=np.float32)
    Bu = np.empty((cfg.B, cfg.H, cfg.L, cfg.N), dtype=np.float32)
    children = ss.spawn(len(seqs))

    def one(i):
        b, h = seqs[i]
        r = np.random.default_rng(children[i])
        if h is None:
            bs = base if (base is None or isinstance(base, str)) else base[b]
            uu, bu, nr, nd = _sequence(cfg, r, bs, scale, W64, Wb64)
            u[b] = uu
            Bu[b] = bu
        else:
            bs = base if (base is None or isinstance(base, str)) else base(b, h)
            uu, bu, nr, nd = _sequence(cfg, r, bs, scale, W64[h:h + 1], Wb64[h:h + 1])
            u[b, h] = uu
            Bu[b, h] = bu[0]
        return nr, nd

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads > 1 and len(seqs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            res = list(ex.map(one, range(len(seqs))))
    else:
        res = [one(i) for i in range(len(seqs))]
    return Inputs(cfg=cfg, u=u, W_sel=W_sel, W_d=W_d, W_b=W_b, b_d=b_d,
                  dict_idx=dic, C=C, h0=h0, Bu=Bu,
                  rounds=max(r[0] for r in res), redrawn_rows=sum(r[1] for r in res))


def upstream_grads(B, H, L, N, seed):
    """Seeded dLoss/dy [B,H,L] and dLoss/dh_L [B,H,N] (standard normal, fp32)
    for the gradient pass through the scan."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x6272]))
    g_y = rng.standard_normal((B, H, L)).astype(np.float32)
    g_hL = rng.standard_normal((B, H, N)).astype(np.float32)
    return g_y, g_hL


def dense_dictionary(H, K, N, seed):
    """Seeded dense dictionary matrices M [H,K,N,N] (standard normal, fp32;
    M[h,k,i,j] is row i, column j) for the soft-selection comparison path."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x736F6674]))
    return rng.standard_normal((H, K, N, N)).astype(np.float32)
