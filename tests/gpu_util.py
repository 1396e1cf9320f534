"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import math

import numpy as np
import torch

from oracle import mla_oracle as O

LN2 = math.log(2.0)
TOL = {"bf16": 2e-2, "fp8": 6e-2}


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def lse_to_nats(lse: np.ndarray, base: str) -> np.ndarray:
    return lse * LN2 if base == "2" else lse


def assert_partial_close(got_out, got_lse, ref_out, ref_lse, base: str, tol: float, what: str = ""):
    """Max-abs check of out and lse (lse compared in nats after rebase);
    neutral rows must be exactly (+0, -inf)."""
    go, gl = to_np(got_out), to_np(got_lse)
    ro, rl = np.asarray(ref_out, np.float64), np.asarray(ref_lse, np.float64)
    assert go.shape == ro.shape and gl.shape == rl.shape, (what, go.shape, ro.shape)
    assert not np.isnan(go).any(), f"{what}: NaN in out (unwritten or poisoned row)"
    assert not np.isnan(gl).any(), f"{what}: NaN in lse"
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), f"{what}: -inf pattern differs"
    if empty.any():
        assert np.all(go[empty] == 0.0), f"{what}: neutral rows must be exactly 0"
        assert np.all(np.signbit(go[empty]) == False), f"{what}: neutral rows must be +0"  # noqa: E712
    fin = ~empty
    err_o = np.abs(go - ro).max() if go.size else 0.0
    assert err_o <= tol, f"{what}: out max-abs error {err_o:.3e} > {tol}"
    if fin.any():
        err_l = np.abs(lse_to_nats(gl[fin], base) - lse_to_nats(rl[fin], base)).max()
        assert err_l <= tol, f"{what}: lse max-abs error {err_l:.3e} (nats) > {tol}"
    return err_o


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (RNE) via float32, for comparing bf16 outputs."""
    from workloads import f32_to_bf16_bits
    return O.decode_bf16(f32_to_bf16_bits(np.asarray(x, np.float32)))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)
