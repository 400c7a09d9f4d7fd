"""The Python binding checks every tensor's shape and dtype against the call's
dims before anything reaches the library (the C ABI cannot see allocation
sizes, so a short or mistyped tensor would be read or written past its end on
the device).  Host tensors suffice: shape and dtype are checked before device
placement, so a correct call on host tensors stops at the device check and a
wrong one stops earlier, naming the argument."""

import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def P():
    from tests._libutil import ensure_built
    ensure_built()
    import structured_sparse_state_pdssm_amd as P
    return P


B, H, L, N, K, d = 2, 3, 40, 16, 8, 64
f32, i32, bf16 = torch.float32, torch.int32, torch.bfloat16


def z(*shape, dt=f32):
    return torch.zeros(shape, dtype=dt)


def fwd_args():
    return dict(u=z(B, H, L, d), W_sel=z(H, K, d), dict_idx=z(H, K, N, dt=i32), W_d=z(H, N, d),
                b_d=z(H, N), Bu=z(B, H, L, N), C=z(H, N), h0=z(B, H, N))


def scan_args():
    return dict(k_star=z(B, H, L, dt=i32), dict_idx=z(H, K, N, dt=i32), D=z(B, H, L, N),
                Bu=z(B, H, L, N), C=z(H, N), h0=z(B, H, N))


def _device_error(fn, **kw):
    with pytest.raises(ValueError, match="device tensor"):
        fn(**kw)


def test_correct_host_call_stops_at_device_check(P):
    _device_error(P.pdssm_fwd, **fwd_args())
    _device_error(P.pdssm_scan_fwd, **scan_args())


@pytest.mark.parametrize("name,bad", [
    ("dict_idx", z(H, K, N + 1, dt=i32)),
    ("b_d", z(H, N - 1)),
    ("Bu", z(B, H, L - 1, N)),
    ("C", z(H + 1, N)),
    ("h0", z(B, H, 2 * N)),
])
def test_fwd_wrong_input_shape(P, name, bad):
    kw = fwd_args()
    kw[name] = bad
    with pytest.raises(ValueError, match=f"{name} must have shape"):
        P.pdssm_fwd(**kw)


@pytest.mark.parametrize("name,bad", [
    ("y", z(B, H, L - 4)),
    ("h_L", z(B, H, N - 1)),
    ("k_star", z(B, H, L + 1, dt=i32)),
    ("D", z(B, H, L, N // 2)),
])
def test_fwd_undersized_output(P, name, bad):
    kw = fwd_args()
    with pytest.raises(ValueError, match=f"{name} must have shape"):
        P.pdssm_fwd(**kw, want_k=True, want_D=True, out={name: bad})


@pytest.mark.parametrize("name,bad", [
    ("dict_idx", z(H, K, N, dt=torch.int64)),
    ("Bu", z(B, H, L, N, dt=bf16)),
    ("C", z(H, N, dt=torch.float64)),
])
def test_fwd_wrong_dtype(P, name, bad):
    kw = fwd_args()
    kw[name] = bad
    with pytest.raises(TypeError, match=name):
        P.pdssm_fwd(**kw)


def test_fwd_wrong_output_dtype(P):
    with pytest.raises(TypeError, match="k_star"):
        P.pdssm_fwd(**fwd_args(), want_k=True, out={"k_star": z(B, H, L)})
    with pytest.raises(TypeError, match="y"):
        P.pdssm_fwd(**fwd_args(), out={"y": z(B, H, L, dt=bf16)})


@pytest.mark.parametrize("name,bad", [
    ("D", z(B, H, L, N - 1)),
    ("Bu", z(B, H, L + 3, N)),
    ("C", z(H, 2, N)),
    ("h0", z(1, H, N)),
])
def test_scan_wrong_shape(P, name, bad):
    kw = scan_args()
    kw[name] = bad
    with pytest.raises(ValueError, match=f"{name} must have shape"):
        P.pdssm_scan_fwd(**kw)


def test_scan_undersized_outputs(P):
    with pytest.raises(ValueError, match="y must have shape"):
        P.pdssm_scan_fwd(**scan_args(), out={"y": z(B, H, L - 1)})
    with pytest.raises(ValueError, match="h_L must have shape"):
        P.pdssm_scan_fwd(**scan_args(), out={"h_L": z(B, H - 1, N)})


def test_fold_and_multi_shapes(P):
    kw = fwd_args()
    del kw["Bu"]
    _device_error(P.pdssm_fwd_wb, W_b=z(H, N, d), **kw)
    with pytest.raises(ValueError, match="W_b must have shape"):
        P.pdssm_fwd_wb(W_b=z(H, N, d - 8), **kw)
    with pytest.raises(TypeError, match="W_b"):
        P.pdssm_fwd_wb(W_b=z(H, N, d, dt=bf16), **kw)
    kw["C"] = z(H, 2, N)
    _device_error(P.pdssm_fwd_wb_multi, W_b=z(H, N, d), **kw)
    with pytest.raises(ValueError, match="y must have shape"):
        P.pdssm_fwd_wb_multi(W_b=z(H, N, d), out={"y": z(B, H, L)}, **kw)
    sk = scan_args()
    sk["C"] = z(H, 3, N)
    with pytest.raises(ValueError, match="y must have shape"):
        P.pdssm_scan_fwd_multi(**sk, out={"y": z(B, H, L, 2)})


def test_select_shapes(P):
    kw = dict(u=z(B, L, d), W_sel=z(H, K, d), W_d=z(H, N, d), b_d=z(H, N))   # shared u
    _device_error(P.pdssm_select, **kw)
    with pytest.raises(ValueError, match="D must have shape"):
        P.pdssm_select(**kw, out={"D": z(B, H, L, N + 1)})
    with pytest.raises(ValueError, match="P_idx must have shape"):
        P.pdssm_select(**kw, dict_idx=z(H, K, N, dt=i32), want_P=True, out={"P_idx": z(B, H, L, N - 1, dt=i32)})
    with pytest.raises(ValueError, match="inconsistent"):
        P.pdssm_select(u=z(B, L, d + 8), W_sel=z(H, K, d), W_d=z(H, N, d), b_d=z(H, N))


def test_states_bwd_sens_soft_pidx_shapes(P):
    sk = scan_args()
    with pytest.raises(ValueError, match="H_all must have shape"):
        P.pdssm_scan_states(**sk, out={"H_all": z(B, H, L, N - 1)})
    bk = dict(k_star=sk["k_star"], dict_idx=sk["dict_idx"], D=sk["D"], C=sk["C"], H_all=z(B, H, L, N),
              g_y=z(B, H, L))
    _device_error(P.pdssm_scan_bwd, **bk)
    with pytest.raises(ValueError, match="g_y must have shape"):
        P.pdssm_scan_bwd(**{**bk, "g_y": z(B, H, L + 1)})
    with pytest.raises(ValueError, match="g_C must have shape"):
        P.pdssm_scan_bwd(**bk, out={"g_C": z(H, N - 1)})
    with pytest.raises(ValueError, match="dY must have shape"):
        P.pdssm_impulse_sens(sk["k_star"], sk["dict_idx"], sk["D"], z(H, N, d), z(H, N, d), sk["C"],
                             out=z(B, H, L, d - 1))
    with pytest.raises(ValueError, match="M must have shape"):
        P.pdssm_soft_select(z(B, H, L, d), z(H, K, d), z(H, K, N, N + 1), z(H, N, d), z(H, N))
    with pytest.raises(ValueError, match="Bu must have shape"):
        P.pdssm_scan_fwd_pidx(z(B, H, L, N, dt=i32), z(B, H, L, N), z(B, H, L - 1, N), z(H, N))


def test_workspace_checked(P):
    with pytest.raises(TypeError, match="workspace"):
        P.pdssm_workspace_status(torch.zeros(256, dtype=torch.float32))
    with pytest.raises(ValueError, match="device tensor"):
        P.pdssm_workspace_status(torch.zeros(256, dtype=torch.uint8))
