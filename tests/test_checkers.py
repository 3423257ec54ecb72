"""The GPU tests' checkers, on the CPU: each must reject the mistake it is
there to catch."""
import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("fmt,dtype", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_rounded_once_catches_double_rounding(fmt, dtype):
    """Rounding through binary32 (binary64 -> binary32 -> 16 bits, nearest even
    both times) is off by one ulp where the binary32 value lands on a 16-bit
    halfway point; the once-rounding check must flag it, and accept the
    correctly rounded values."""
    from test_gpu_layouts import _rounded_once
    rng = np.random.default_rng(97)
    exact = rng.standard_normal((256, 4096)) * 3
    twice = torch.from_numpy(exact.astype(np.float32)).to(dtype)
    once = torch.from_numpy(oracle.round_bits(exact, fmt).view(np.int16)).view(dtype)
    _rounded_once(once, exact, fmt, "once")
    with pytest.raises(AssertionError, match="not rounded once"):
        _rounded_once(twice, exact, fmt, "twice")
