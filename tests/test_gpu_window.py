"""Band radii at and past the sequence length, up to 2^31 - 1.

Under the band of the Hinglish notes' "Worked example Local Attention Window"
(|i - j| <= window), a radius of N - 1 or more allows every pair of a length-N
sequence. The kernels add the radius to row indices in 32-bit integers, so the
library clamps it to N - 1 before any launch; these cases check every entry
point that takes a mask (fa_fwd, fa_bwd, fa_fwd_keymajor, fa_fwd_standard)
against the oracle, which keeps the radius in 64 bits, on ragged lengths (not
multiples of any tile) at both head dimensions.
"""
import pytest
import torch

from tests.test_gpu_bwd import run_case as bwd_case
from tests.test_gpu_fwd import run_case as fwd_case, BF16
from tests.test_gpu_keymajor import run_km
from tests.test_gpu_standard import run_std

pytestmark = pytest.mark.gpu

I32_MAX = 2 ** 31 - 1
CASES = [(N, d, w) for N in (300, 1000) for d in (64, 128) for w in (N - 1, N, I32_MAX)]


@pytest.mark.parametrize("N,d,window", CASES, ids=[f"N{N}-d{d}-w{w}" for N, d, w in CASES])
def test_forward_wide_band(N, d, window):
    fwd_case((1, 2, N, d), BF16, "local", window, seed=N + d)


@pytest.mark.parametrize("N,d,window", CASES, ids=[f"N{N}-d{d}-w{w}" for N, d, w in CASES])
def test_backward_wide_band(N, d, window):
    bwd_case((1, 2, N, d), BF16, "local", window, seed=N + d + 1)


@pytest.mark.parametrize("N,d,window", CASES, ids=[f"N{N}-d{d}-w{w}" for N, d, w in CASES])
def test_keymajor_wide_band(N, d, window):
    run_km((1, 2, N, d), "local", window, 64, seed=N + d + 2)


@pytest.mark.parametrize("N,d,window", CASES, ids=[f"N{N}-d{d}-w{w}" for N, d, w in CASES])
def test_standard_wide_band(N, d, window):
    run_std((1, 2, N, d), "local", window, seed=N + d + 3)


def test_radius_past_int32_from_python():
    """A radius above 2^31 - 1 from Python allows the same pairs (it is passed
    as 2^31 - 1, never wrapped to a negative or small value)."""
    fwd_case((1, 1, 300, 128), BF16, "local", 2 ** 40, seed=5)
