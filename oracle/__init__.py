"""fp64 CPU oracle for the hard-selection PD-SSM forward pass and the
gradient through its scan for fixed selections.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path."""

from .pdssm_oracle import (  # noqa: F401
    dict_hardmax,
    drive,
    forward,
    forward_wb,
    forward_wb_multi,
    forward_inputs,
    impulse_sensitivity,
    pd_apply,
    pd_compose,
    scan,
    scan_multi,
    scan_pidx,
    scan_states,
    scan_vjp,
    scores,
    select,
    sigmoid,
    soft_select,
    three_phase,
    transition_matrix,
)
