"""Parity of the soft-selection comparison path (HIP through the C ABI) with
the fp64 oracle: ``pdssm_soft_select`` against ``soft_select``,
``pdssm_scan_fwd_pidx`` against ``scan_pidx``, ``pdssm_dict_hardmax`` against
``dict_hardmax``.

Where the top two rows of a mixture column are closer than ``TIE`` both rows
are correct choices (fp32 against fp64 rounding decides): the GPU's row must
then be one of them, and the scan is compared on the GPU's own choices.
Bar: M_t within 1e-5 (1 + |ref|), D within 2e-6, y and h_L within
1e-4 (1 + |ref|)."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import dense_dictionary, generate, get_config
from tests._gpu import assert_within, host, lib, proj_dev, to_dev, torch_mod

pytestmark = pytest.mark.gpu

TIE = 1e-4

CASES = {
    "impulse": ("impulse", dict(H=3, L=700)),
    "tiny": ("tiny", dict(L=250)),
    "bf16_d128": ("timeseries", dict(B=1, H=2, L=300, N=16, K=8)),
    "n5": ("base", dict(B=2, H=2, L=333, N=5, K=3, d=32)),
}

_cache = {}


def _case(key):
    if key not in _cache:
        name, kw = CASES[key]
        inp = generate(get_config(name, **kw))
        c = inp.cfg
        M = dense_dictionary(c.H, c.K, c.N, c.seed)
        ref = oracle.soft_select(inp.u, inp.W_sel, M, inp.W_d, inp.b_d, c.u_shared)
        _cache[key] = (inp, M, ref)
    return _cache[key]


def _gpu_soft(inp, M):
    P = lib()
    bf = inp.cfg.dtype == "bf16"
    return P.pdssm_soft_select(proj_dev(inp.u, bf), proj_dev(inp.W_sel, bf), to_dev(M), proj_dev(inp.W_d, bf),
                               to_dev(inp.b_d))


def _check_selection(out, ref, what):
    assert_within(host(out["M_t"]), ref["M_t"], f"{what} M_t", tol=1e-5)
    assert np.max(np.abs(host(out["D"]) - ref["D"])) <= 2e-6, f"{what} D"
    got = host(out["P_idx"])
    sure = ref["gap"] >= TIE
    assert np.array_equal(got[sure], ref["P_idx"][sure]), f"{what}: P_idx differs where the choice is clear"
    # near ties: the GPU's row must be within TIE of the column maximum
    Mt = ref["M_t"]
    top = Mt.max(axis=-2)
    picked = np.take_along_axis(Mt, got[..., None, :].astype(np.int64), axis=-2)[..., 0, :]
    assert np.all(top - picked <= TIE), f"{what}: a near-tie choice is not one of the top rows"
    return got


@pytest.mark.parametrize("key", list(CASES))
def test_soft_select_parity(key):
    inp, M, ref = _case(key)
    print(f"[gpu] pdssm_soft_select {key}", flush=True)
    _check_selection(_gpu_soft(inp, M), ref, key)


@pytest.mark.parametrize("key", list(CASES))
def test_soft_forward_parity(key):
    """Selection then the scan on per-step maps, against the oracle's scan on
    the same maps and diagonals."""
    inp, M, ref = _case(key)
    P = lib()
    print(f"[gpu] soft forward {key}", flush=True)
    out = _gpu_soft(inp, M)
    pidx = _check_selection(out, ref, key)
    D32 = host(out["D"])
    y, hL = P.pdssm_scan_fwd_pidx(out["P_idx"], out["D"], to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0),
                                  chunk=128)
    yr, hr = oracle.scan_pidx(pidx, D32.astype(np.float64), inp.Bu, inp.C, inp.h0)
    assert_within(host(y), yr, f"{key} y")
    assert_within(host(hL), hr, f"{key} h_L")


@pytest.mark.parametrize("chunk", [1, 3, 16, 100, 128, 256, 512])
@pytest.mark.parametrize("N", [16, 5, 20])
def test_scan_pidx_chunk_independence(chunk, N):
    """N <= 16 with chunks up to 512: maps streamed through registers (the
    step-major scan); N = 20: one on-chip table entry per step (it fits up to
    548 steps: 512 takes 61.7 KB of the 64 KiB)."""
    rng = np.random.default_rng(chunk + 1000 * N)
    B, H, L = 2, 3, 600
    pidx = rng.integers(0, N, (B, H, L, N)).astype(np.int32)
    D = rng.uniform(0.2, 1.0, (B, H, L, N)).astype(np.float32)
    Bu = rng.standard_normal((B, H, L, N)).astype(np.float32)
    C = rng.standard_normal((H, N)).astype(np.float32)
    h0 = rng.standard_normal((B, H, N)).astype(np.float32)
    P = lib()
    print(f"[gpu] pdssm_scan_fwd_pidx N={N} chunk={chunk}", flush=True)
    y, hL = P.pdssm_scan_fwd_pidx(to_dev(pidx), to_dev(D), to_dev(Bu), to_dev(C), to_dev(h0), chunk=chunk)
    yr, hr = oracle.scan_pidx(pidx, D.astype(np.float64), Bu, C, h0)
    assert_within(host(y), yr, f"chunk {chunk} y")
    assert_within(host(hL), hr, f"chunk {chunk} h_L")


@pytest.mark.parametrize("N,chunk", [(16, 1024), (20, 549), (20, 1024)])
def test_scan_pidx_rejects_a_chunk_too_long_for_its_table(N, chunk):
    """The header's limits: N = 16 above 512 steps, N = 20 above 548."""
    P = lib()
    z = np.zeros((1, 1, 2048, N), dtype=np.float32)
    with pytest.raises(P.PdssmError) as e:
        P.pdssm_scan_fwd_pidx(to_dev(z.astype(np.int32)), to_dev(z), to_dev(z), to_dev(np.zeros((1, N), np.float32)),
                              chunk=chunk)
    assert e.value.status == P.PDSSM_EUNSUPPORTED


def test_scan_pidx_deterministic():
    rng = np.random.default_rng(3)
    B, H, L, N = 1, 4, 2000, 16
    args = (to_dev(rng.integers(0, N, (B, H, L, N)).astype(np.int32)),
            to_dev(rng.uniform(0.2, 1.0, (B, H, L, N)).astype(np.float32)),
            to_dev(rng.standard_normal((B, H, L, N)).astype(np.float32)),
            to_dev(rng.standard_normal((H, N)).astype(np.float32)))
    P = lib()
    a = P.pdssm_scan_fwd_pidx(*args, chunk=512)
    b = P.pdssm_scan_fwd_pidx(*args, chunk=512)
    assert np.array_equal(host(a[0]), host(b[0])) and np.array_equal(host(a[1]), host(b[1]))


def test_dict_hardmax_parity():
    P = lib()
    M = dense_dictionary(5, 7, 13, 11)
    got = host(P.pdssm_dict_hardmax(to_dev(M)))
    assert np.array_equal(got, oracle.dict_hardmax(M))


def test_soft_select_deterministic():
    inp, M, _ = _case("impulse")
    a, b = _gpu_soft(inp, M), _gpu_soft(inp, M)
    for n in ("M_t", "P_idx", "D"):
        assert np.array_equal(host(a[n]), host(b[n])), n


@pytest.mark.slow
def test_soft_full_impulse_sampled_heads():
    """Full impulse shape in the bench's configuration (chunk 512): the whole
    soft forward on the GPU, two heads compared with the oracle over all
    131072 steps (selection element by element, then the scan on the GPU's
    own maps)."""
    torch = torch_mod()
    P = lib()
    inp = generate(get_config("impulse"))
    c = inp.cfg
    M = dense_dictionary(c.H, c.K, c.N, c.seed)
    print("[gpu] soft forward impulse full size", flush=True)
    out = _gpu_soft(inp, M)
    y, hL = P.pdssm_scan_fwd_pidx(out["P_idx"], out["D"], to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0),
                                  chunk=c.chunk)
    torch.cuda.synchronize()
    for h in (0, 17):
        sl = slice(h, h + 1)
        ref = oracle.soft_select(inp.u[:, sl], inp.W_sel[sl], M[sl], inp.W_d[sl], inp.b_d[sl])
        got = {k: out[k][:, sl] for k in ("M_t", "P_idx", "D")}
        pidx = _check_selection(got, ref, f"head {h}")
        yr, hr = oracle.scan_pidx(pidx, host(out["D"][:, sl]).astype(np.float64), inp.Bu[:, sl], inp.C[sl],
                                  inp.h0[:, sl])
        assert_within(host(y[:, sl]), yr, f"head {h} y")
        assert_within(host(hL[:, sl]), hr, f"head {h} h_L")
