"""The allocation-free fused entry point (pdssm_fwd_noalloc), for callers that
cannot allocate device memory: its look-back scratch is the library's own
per-device array.  Its results must equal those of pdssm_fwd with a caller
workspace on the same inputs (the same kernels run on both), for two calls in
a row, the second on a smaller problem (the array keeps the first call's
contents, which the second must not see), and every selection must match the
oracle."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config
from tests._gpu import assert_within, host, lib, torch_mod, upload

pytestmark = pytest.mark.gpu


def _pair(name, kw):
    inp = generate(get_config(name, **kw))
    ref = oracle.forward_inputs(inp)
    return inp, ref, upload(inp)


def _run_both(P, inp, dev, chunk):
    torch = torch_mod()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (dev["u"], dev["W_sel"], dev["dict_idx"], dev["W_d"], dev["b_d"], dev["Bu"], dev["C"], dev["h0"])
    na = P.pdssm_fwd_noalloc(*args, chunk=chunk, want_k=True, want_D=True, status=st)
    torch.cuda.synchronize()
    wk = P.pdssm_fwd(*args, chunk=chunk, want_k=True, want_D=True)
    return na, wk, int(host(st)[0])


@pytest.mark.parametrize("first,second", [
    (("impulse", dict(H=8, L=20000)), ("impulse", dict(H=2, L=3000))),
    (("timeseries", dict(B=2, H=4, L=4096)), ("base", dict(B=1, H=3, L=700))),
])
def test_noalloc_matches_workspace_entry(first, second):
    P = lib()
    for (name, kw) in (first, second):
        inp, ref, dev = _pair(name, kw)
        print(f"[gpu] pdssm_fwd_noalloc {name} {kw}", flush=True)
        na, wk, status = _run_both(P, inp, dev, inp.cfg.chunk)
        assert status == 0
        for key in ("k_star", "D", "y", "h_L"):
            assert np.array_equal(host(na[key]), host(wk[key])), f"{name}: {key} differs from pdssm_fwd"
        assert np.array_equal(host(na["k_star"]), ref["k_star"])
        assert_within(host(na["y"]), ref["y"], f"{name} y")
        assert_within(host(na["h_L"]), ref["h_L"], f"{name} h_L")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """A call whose look-back scratch would exceed the array is refused
    before anything is enqueued (here 32 MiB: 256 chunks of 256 sequences)."""
    P = lib()
    import ctypes
    d = P.make_dims(8, 32, 131072, 16, 8, 64)
    assert P.fwd_workspace_bytes(d, 512) > P.PDSSM_NOALLOC_SCRATCH_BYTES
    A = 0x7f0000000000
    big = 1 << 30
    rc = P.lib.pdssm_fwd_noalloc(ctypes.byref(d), 512, A, A + big, A + 2 * big, A + 3 * big, A + 4 * big,
                                 A + 5 * big, A + 6 * big, None, None, None, A + 7 * big, A + 8 * big, None, None)
    assert rc == P.PDSSM_EUNSUPPORTED
    assert b"scratch" in P.lib.pdssm_last_error()
