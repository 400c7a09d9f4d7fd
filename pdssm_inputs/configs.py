"""The five synthetic workloads, as data.

Shapes: B batch, H heads, L steps, N state size, K dictionary size, d input
width, ``chunk`` the scan chunk length.  ``dtype`` is the storage type of u and
of the three projection matrices (W_sel, W_d, W_b); the state, D, Bu, C and
outputs are always fp32.

Recipes (all normal draws use the variance convention N(mean, variance)):

* ``u_rule``
    - ``normal``    u ~ N(0, 1)
    - ``sinusoid``  u[b,h,t,c] = sum_{m<3} a_m sin(2 pi t / P_m + phi_m) + eps,
                    a_m ~ U(0.5, 1.5), P_m log-uniform in [8, 4096],
                    phi_m ~ U[0, 2 pi) drawn per (b, h, c); eps ~ N(0, 0.1)
                    (a time-series stand-in for the long multivariate
                    classification / forecasting workloads of the Flash
                    PD-SSM experiments, "time-series modelling")
    - ``impulse``   u_t = 1e-3 z_t, plus e_0 (channel 0) at t = 0, z ~ N(0, 1)
                    (a stand-in for the 128 000-step impulse-response
                    benchmark of the Phase Gradient Flow paper, abstract)
* ``dict_rule``
    - ``identity0`` P^(0) = I; for k > 0 each column's one sits in a row
                    drawn uniformly from [0, N)
    - ``uniform``   every k drawn that way
* W_sel, W_d, W_b ~ N(0, 1/d) each; C ~ N(0, 1/N); b_d constant; h0 = 0.
* ``u_shared``: u is one [B, L, d] tensor read by every head (the LM-layer
  shape: K = 32 ~ sqrt(768), matching the dictionary-size scaling of the
  Flash PD-SSM "architecture integration" paragraph); otherwise u is
  [B, H, L, d], one input row per head and step.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    L: int
    N: int
    K: int
    d: int
    chunk: int
    dtype: str          # "f32" or "bf16"
    u_shared: bool
    b_d: float
    u_rule: str
    dict_rule: str
    seed: int

    @property
    def state_updates(self) -> int:
        return self.B * self.H * self.L * self.N

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    c.name: c
    for c in (
        Config("tiny", B=1, H=1, L=256, N=8, K=4, d=16, chunk=64, dtype="f32",
               u_shared=False, b_d=2.0, u_rule="normal", dict_rule="identity0",
               seed=1),
        Config("base", B=4, H=8, L=4096, N=16, K=8, d=64, chunk=128,
               dtype="f32", u_shared=False, b_d=2.0, u_rule="normal",
               dict_rule="identity0", seed=2),
        Config("timeseries", B=8, H=16, L=16384, N=32, K=16, d=128, chunk=256,
               dtype="bf16", u_shared=False, b_d=3.0, u_rule="sinusoid",
               dict_rule="uniform", seed=3),
        Config("impulse", B=1, H=32, L=131072, N=16, K=8, d=64, chunk=512,
               dtype="f32", u_shared=False, b_d=4.0, u_rule="impulse",
               dict_rule="identity0", seed=4),
        Config("lm_layer", B=16, H=24, L=2048, N=64, K=32, d=768, chunk=128,
               dtype="bf16", u_shared=True, b_d=2.0, u_rule="normal",
               dict_rule="uniform", seed=5),
    )
}

# Order in which the workloads are listed (smallest first).
ORDER = ("tiny", "base", "timeseries", "impulse", "lm_layer")


def get_config(name: str, **overrides) -> Config:
    """Return a named workload, optionally with fields replaced (for reduced
    parity sizes: e.g. ``get_config("impulse", L=3000)``)."""
    c = CONFIGS[name]
    return c.with_(**overrides) if overrides else c


# Launch chunk of a pass where it differs from the workload's own.  The
# passes on the LM-layer shape run the selection (and drive) GEMMs and then
# the chunked scan, which is fastest at 96 steps per chunk: three workgroups
# of 53 KB of LDS share a CU there, two at 128.  The base shape (32 sequences of
# 4096 steps) at 128 makes 1024 chunk tasks, more than one round of the 768
# workgroups the chip holds, each paying the per-task set-up; at 256 the 512
# tasks run in one round.  The results do not depend on the chunk beyond
# rounding.
LAUNCH_CHUNK = {("fold", "lm_layer"): 96, ("multi", "lm_layer"): 96, ("fwd", "base"): 256, ("fwd", "lm_layer"): 96, ("scan", "lm_layer"): 96}


def launch_chunk(pass_name: str, cfg: Config) -> int:
    """Chunk at which the benchmark runs `pass_name` on workload `cfg`."""
    return LAUNCH_CHUNK.get((pass_name, cfg.name), cfg.chunk)
