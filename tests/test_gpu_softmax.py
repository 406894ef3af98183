"""GPU parity of row_softmax (HIP, through the C ABI) against the FP64 oracle.

Outputs are NaN-prefilled (the softmax study's coverage check, section 3.4).
Tolerances: max-abs 1e-6, rows sum to 1 within 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import online_softmax_causal_amd as osc
import workloads
from tests import tolerances

pytestmark = pytest.mark.gpu


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_gpu(x, x_off=0, y_off=0):
    """Run on device copies placed x_off / y_off floats past a 256-byte boundary."""
    d = dev()
    M, N = x.shape
    xb = torch.empty(M * N + x_off + 4, dtype=torch.float32, device=d)
    yb = torch.full((M * N + y_off + 4,), float("nan"), dtype=torch.float32, device=d)
    xd = xb[x_off:x_off + M * N]
    xd.copy_(x.reshape(-1).to(d))
    yd = yb[y_off:y_off + M * N]
    osc.row_softmax(xd, yd, M, N)
    torch.cuda.synchronize()
    return yd.view(M, N)


def check(name, y, y_ref):
    yn = y.cpu().double().numpy() if hasattr(y, "cpu") else y
    assert np.isfinite(yn).all(), "%s: non-finite output" % name
    err = np.abs(yn - y_ref).max()
    rs = np.abs(yn.sum(axis=1) - 1.0).max()
    print("%s: max|dy| %.3e  max|rowsum-1| %.3e" % (name, err, rs), flush=True)
    assert err <= tolerances.SOFTMAX_Y, name
    assert rs <= tolerances.SOFTMAX_ROWSUM, name


NS = [1, 2, 3, 4, 5, 63, 64, 65, 255, 257, 1023, 2045, 2046, 2048, 2051, 4093, 4096,
      4099, 16381, 32768, 65533, 65536, 70001]


@pytest.mark.parametrize("N", NS)
def test_row_lengths(N):
    M = 7 if N > 10000 else 37
    x = workloads.softmax_inputs(M, N, seed=200 + N)
    print("running row_softmax M%d N%d" % (M, N), flush=True)
    check("M%d N%d" % (M, N), run_gpu(x), oracle.row_softmax(x))


@pytest.mark.parametrize("M,N,x_off", [(2, (1 << 24) + 3, 1), (3, 1000003, 0)])
def test_very_long_rows(M, N, x_off):
    """Rows of millions of elements (the streaming kernel), one of them with
    misaligned row starts: every element against the oracle."""
    x = workloads.softmax_inputs(M, N, seed=400 + M, last=None) * 4
    print("running row_softmax very long M%d N%d x_off %d" % (M, N, x_off), flush=True)
    check("long M%d N%d" % (M, N), run_gpu(x, x_off, 0), oracle.row_softmax(x))


@pytest.mark.parametrize("x_off,y_off", [(1, 1), (2, 2), (3, 3), (1, 3), (0, 2), (3, 0)])
@pytest.mark.parametrize("N", [6, 257, 3001, 9000])
def test_misaligned_rows(N, x_off, y_off):
    """Row starts at every 16-byte phase, with x and y in equal or different phases."""
    M = 9
    x = workloads.softmax_inputs(M, N, seed=300 + N + x_off, last=None) * 5
    print("running row_softmax misaligned M%d N%d x_off %d y_off %d" % (M, N, x_off, y_off), flush=True)
    check("misaligned N%d %d/%d" % (N, x_off, y_off), run_gpu(x, x_off, y_off), oracle.row_softmax(x))


def test_special_inputs():
    """Softmax study section 3.3: all-zero rows, a constant added to a row, huge spreads."""
    N = 513
    x = torch.zeros(6, N)
    x[1] = 1000.0                      # constant row: uniform
    x[2] = workloads.softmax_inputs(1, N, seed=5, last=None)[0] * 30
    x[3] = x[2] + 250.0                # same row shifted: same output
    x[4, 7] = 1e4                      # one dominant element
    x[5] = -3e4
    x[5, 100] = 3e4
    print("running row_softmax special inputs", flush=True)
    y = run_gpu(x).cpu().double().numpy()
    check("special", y, oracle.row_softmax(x))
    np.testing.assert_allclose(y[0], 1.0 / N, rtol=1e-6)
    np.testing.assert_allclose(y[1], 1.0 / N, rtol=1e-6)
    assert np.abs(y[2] - y[3]).max() <= 2e-6


@pytest.mark.parametrize("wname", ["R1", "R2"])
def test_configs(wname):
    w = workloads.SOFTMAX[wname]
    x = workloads.softmax_inputs(w.M, w.N, seed=w.seed, last=w.last)
    print("running", w.describe(), flush=True)
    y = run_gpu(x)
    if w.M * w.N <= 4 << 20:
        check(wname, y, oracle.row_softmax(x))
    else:
        rows = sorted({0, 1, w.M // 2, w.M - 2, w.M - 1} | set(range(3, w.M, w.M // 61)))
        yr = y[rows].cpu().double().numpy()
        check(wname + " sampled", yr, oracle.row_softmax_rows(x, rows))
        assert torch.isfinite(y).all().item()
        rs = (y.double().sum(dim=1) - 1.0).abs().max().item()
        assert rs <= tolerances.SOFTMAX_ROWSUM


def test_softmax_deterministic():
    x = workloads.softmax_inputs(64, 5000, seed=17)
    a = run_gpu(x).cpu()
    b = run_gpu(x).cpu()
    assert torch.equal(a, b)
