"""Shared helpers of the GPU parity tests (comparison, conversions, tolerances)."""

from __future__ import annotations

import numpy as np
import torch

# Tolerances of the attention outputs against the fp64 oracle: bf16 inputs and
# bf16 probabilities in the P.V product with fp32 accumulation.
O_ATOL = 2e-2
O_RTOL = 2e-2
LSE_ATOL = 5e-3


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (bf16/fp32) tensor to a float64 NumPy array on the host."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run on a host without a GPU")
    return torch.device("cuda:0")


def banner(msg: str) -> None:
    """Name the case before each GPU step (a fault can end the process)."""
    print(f"[case] {msg}", flush=True)


def assert_attention_close(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray,
                           lse_ref: np.ndarray, what: str = "") -> None:
    """O within atol=rtol=2e-2, finite LSE within 5e-3, -inf exactly where the oracle has it."""
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    np.testing.assert_allclose(o_gpu, o_ref, atol=O_ATOL, rtol=O_RTOL, err_msg=what)
    fin = np.isfinite(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse_gpu), np.isneginf(lse_ref), err_msg=what)
    np.testing.assert_allclose(lse_gpu[fin], lse_ref[fin], atol=LSE_ATOL, rtol=0, err_msg=what)
