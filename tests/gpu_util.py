"""Helpers for the GPU parity tests: tolerance checks, device inputs, reading
the cache's bytes through ll_cache_layout."""

import math
import sys

import numpy as np
import pytest

from sink_short_window_amd import ll, synth

# Output tolerances (bf16 activations with fp32 accumulation; fp32 path).
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 5e-3
F32_MAX_ABS = 1e-4
# Diagnostic gates: relative L2 error and LSE error.  A correct bf16 kernel
# sits near 2-3e-3 relative L2; dropping or doubling a key run gives 0.3-1.
REL_L2 = 1e-2
LSE_ABS_BF16 = 1e-2
LSE_ABS_F32 = 1e-4


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    ll.load()    # raises if the library is missing: no fallback


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x32, dtype):
    return synth.to_torch(x32, dtype, "cuda")


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_out(got, want, dtype, what=""):
    """Compare a GPU output (torch) with the oracle (float64 numpy)."""
    g = host(got)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - want)
    mx, mean = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-30))
    say(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} rel_l2={rel:.3e}")
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"{what}: max abs {mx}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx}"
        assert mean <= BF16_MEAN_ABS, f"{what}: mean abs {mean}"
        assert rel <= REL_L2, f"{what}: rel L2 {rel}"
    return mx, mean, rel


def check_lse(got, want, dtype, what=""):
    g = host(got)
    err = float(np.abs(g - want).max())
    say(f"  {what} lse: max_abs={err:.3e}")
    assert err <= (LSE_ABS_F32 if dtype == "f32" else LSE_ABS_BF16), f"{what}: lse err {err}"


def cache_rows(cache, layer, which, segment):
    """A cached tensor as a host array [H][rows][cols] (exact values)."""
    t = cache.rows(layer, which, segment)
    return t.cpu().numpy() if t.dtype.is_floating_point is False else host(t)


def act_code(dtype):
    return ll.LL_F32 if dtype == "f32" else ll.LL_BF16
