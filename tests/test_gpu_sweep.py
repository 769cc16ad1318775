"""A fixed sweep of small random shapes (seeded): every combination of
padded/unpadded d, head-gradient tile (320/192/128 wide), ragged vocabulary
and chunk tails, single-chunk and many-chunk calls, duplicate ids, masked
rows, both input dtypes, against the oracle.  A second seeded set reaches
hidden sizes up to 3000 (the 256x320 tiles of both gradient GEMMs)."""
import numpy as np
import pytest

from tests.gpu_util import GRAD_TOL, LOSS_TOL
from tests.test_gpu_parity import _check, _small

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 600))
        d = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 700)), 4 * int(rng.integers(1, 160))]))
        K = int(rng.integers(1, 129))
        V = int(rng.integers(K, 6000))
        chunk = int(rng.integers(1, T + 64))
        tau = float(np.round(rng.uniform(0.3, 3.0), 2))
        dtype = "f32" if i % 4 == 3 else "bf16"
        out.append((T, d, V, K, chunk, tau, dtype, i))
    return out


@pytest.mark.parametrize("T,d,V,K,chunk,tau,dtype,i", _cases())
def test_random_shapes(T, d, V, K, chunk, tau, dtype, i):
    masked = tuple(range(0, T, 7)) if T > 3 else ()
    x = _small(T, d, V, K, dtype, seed=100 + i, tau=tau, masked=masked,
               dup_row=(T // 2 if K >= 2 else None))
    tight = dtype == "f32"
    _check(x, f"sweep {i}: T={T} d={d} V={V} K={K} chunk={chunk} tau={tau} {dtype}", chunk=chunk,
           loss_tol=1e-5 if tight else LOSS_TOL, grad_tol=1e-4 if tight else GRAD_TOL)


def _cases_large_d(n=60, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 700))
        d = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 700)), 4 * int(rng.integers(1, 160)),
                            int(rng.integers(700, 3000))]))
        K = int(rng.integers(1, 129))
        V = int(rng.integers(K, 9000))
        chunk = int(rng.integers(1, T + 64))
        tau = float(np.round(rng.uniform(0.3, 3.0), 2))
        dtype = "f32" if i % 5 == 4 else "bf16"
        out.append((T, d, V, K, chunk, tau, dtype, i))
    return out


@pytest.mark.parametrize("T,d,V,K,chunk,tau,dtype,i", _cases_large_d())
def test_random_shapes_large_d(T, d, V, K, chunk, tau, dtype, i):
    masked = tuple(range(0, T, 5)) if T > 3 else ()
    x = _small(T, d, V, K, dtype, seed=5000 + i, tau=tau, masked=masked,
               dup_row=(T // 3 if K >= 2 else None))
    tight = dtype == "f32"
    _check(x, f"sweep-d {i}: T={T} d={d} V={V} K={K} chunk={chunk} tau={tau} {dtype}", chunk=chunk,
           loss_tol=1e-5 if tight else LOSS_TOL, grad_tol=1e-4 if tight else GRAD_TOL)
