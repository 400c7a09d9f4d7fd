"""Seeded synthetic inputs for the hard-selection PD-SSM forward pass.

This module is shared by the tests, the benchmark and the oracle's checks.  It
draws random numbers and lays them out; it does not evaluate the method (no
selection, no transition, no scan).  Two input-preparation steps do touch the
parameters, and both are described where they happen:

* the top-2 score-margin rule, which redraws any input row whose two largest
  linear scores are closer than ``GAP`` (so that an argmax is well posed in any
  reasonable floating-point precision);
* the driving term ``Bu = W_b u``, which the forward pass receives as an input.

``upstream_grads`` draws the loss gradients (dLoss/dy, dLoss/dh_L) that the
gradient pass through the scan takes as inputs; ``dense_dictionary`` draws
the dense dictionary matrices of the soft-selection comparison path.

Workloads follow the pages' experiment descriptions only loosely (they print no
inputs); the recipes are synthetic stand-ins, see ``configs.py``.
"""

from .configs import CONFIGS, Config, get_config, launch_chunk  # noqa: F401
from .gen import (  # noqa: F401
    GAP,
    Inputs,
    bf16_bits,
    bf16_round,
    dense_dictionary,
    generate,
    top2_margin,
    upstream_grads,
)
