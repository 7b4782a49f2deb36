"""The hardware fact the beacon maintenance kernel's error bound rests on.

The kernel forms its chunk-start dots with v_mfma_f32_32x32x16_bf16 and bounds
their error by assuming every MFMA result lies within 8u (u = 2^-24) of the
sum of the magnitudes it adds (the accumulator input and the 16 products).
Adversarial fragments -- magnitudes spread over 2^40, signs mixed, zeros,
cancellation -- are run through one MFMA, and every one of the 1024 outputs
per launch is compared with the exact sum (products of bf16 values are exact
in double; math.fsum sums them exactly rounded)."""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "probes", "libmfma_rounding.so")
U = 2.0 ** -24
BOUND_U = 8.0


def bf16_values(rng, n, emin, emax):
    e = rng.integers(emin, emax + 1, n)
    m = rng.integers(0, 128, n)
    v = rng.choice([-1.0, 1.0], n) * (1 + m / 128.0) * np.exp2(e)
    v[rng.random(n) < 0.1] = 0.0
    return v.astype(np.float32)          # exactly representable in bf16


def test_mfma_result_within_the_assumed_bound():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    assert os.path.exists(LIB), "build the probes first (__graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    lib.mfma_rounding_run.argtypes = [ctypes.c_void_p] * 5
    print("[case] MFMA rounding bound, 24 adversarial launches", flush=True)
    rng = np.random.default_rng(20261203)
    worst = 0.0
    for trial in range(24):
        lo, hi = [(-20, 20), (-4, 4), (-10, 10)][trial % 3]
        A = bf16_values(rng, 32 * 16, lo, hi).reshape(32, 16)
        B = bf16_values(rng, 16 * 32, lo, hi).reshape(16, 32)
        C = bf16_values(rng, 32 * 32, lo + 4, hi + 4).reshape(32, 32)
        if trial % 4 == 3:      # cancellation: an accumulator that the products nearly cancel
            C = (-(A.astype(np.float64) @ B.astype(np.float64))).astype(np.float32)
        ab = (A.view(np.uint32) >> 16).astype(np.uint16)
        bb = (B.view(np.uint32) >> 16).astype(np.uint16)
        a = np.zeros((64, 8), np.uint16)
        b = np.zeros((64, 8), np.uint16)
        c = np.zeros((64, 16), np.float32)
        rows = np.zeros((64, 16), np.int64)
        for lane in range(64):
            r, k0, hh = lane % 32, 8 * (lane // 32), lane // 32
            a[lane] = ab[r, k0:k0 + 8]          # A[row][k] of lane half hh
            b[lane] = bb[k0:k0 + 8, r]          # B[k][col]
            for i in range(16):
                rows[lane, i] = 8 * (i >> 2) + 4 * hh + (i & 3)
                c[lane, i] = C[rows[lane, i], r]
        ta, tb, tc = (torch.from_numpy(x).cuda() for x in (a, b, c))
        td = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
        assert lib.mfma_rounding_run(ta.data_ptr(), tb.data_ptr(), tc.data_ptr(), td.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        d = td.cpu().numpy()
        A64, B64 = A.astype(np.float64), B.astype(np.float64)
        for lane in range(64):
            col = lane % 32
            for i in range(16):
                row = int(rows[lane, i])
                terms = [float(C[row, col])] + list(A64[row, :] * B64[:, col])
                exact = math.fsum(terms)
                mag = math.fsum(abs(t) for t in terms)
                err = abs(float(d[lane, i]) - exact)
                assert err <= BOUND_U * U * mag + 1e-300, (trial, row, col, err, mag)
                if mag > 0:
                    worst = max(worst, err / (U * mag))
    print(f"[case] MFMA rounding: worst error {worst:.2f}u of the magnitudes added "
          f"(bound {BOUND_U:.0f}u)", flush=True)
