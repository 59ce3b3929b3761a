"""Helpers shared by the GPU parity tests."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import pipeline as OP
from oracle.pipeline import to64

# relative gap the oracle must show at a top-k cut before index sets are
# compared bit for bit (a smaller one makes the case invalid, not passed)
MARGIN = 1e-2


def device() -> torch.device:
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def announce(name: str, **kw) -> None:
    """Name the case before any GPU work, so a fault can be traced to it."""
    args = " ".join(f"{k}={v}" for k, v in kw.items())
    print(f"[gpu-case] {name} {args}", file=sys.stderr, flush=True)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 7)


def assert_cache_close(got: torch.Tensor, want: np.ndarray, dtype: str, ref_norm=None):
    """Re-rotated keys: bf16 within one ulp, >= 99.9% bit-equal; fp32 within
    fp32 rounding of the row scale."""
    g = to64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    if dtype == "bf16":
        diff = np.abs(g - want)
        # The oracle rotates twice in fp64 (R(p_new) R(p_old)^T), which leaves an
        # absolute error of a few 2^-53 of the row's magnitude.  bf16 represents
        # such tiny values, so where the exact result is 0 (a zero element of a
        # unit with delta 0, rotated by the identity) the oracle may hold ~1e-17:
        # that error, bounded by 2^-45 of the row's largest element, is allowed
        # on top of the one ulp.
        floor = 2.0 ** -45 * np.abs(want).max(axis=-1, keepdims=True)
        bad = diff > bf16_ulp(want) * 1.0001 + floor
        if bad.any():
            where = np.argwhere(bad)[:8]
            shown = ", ".join(f"{tuple(int(i) for i in ix)}: got {g[tuple(ix)]!r} want "
                              f"{want[tuple(ix)]!r}" for ix in where)
            raise AssertionError(f"{int(bad.sum())} of {bad.size} elements beyond one bf16 ulp "
                                 f"(worst {float(np.max(diff / bf16_ulp(want))):.4g} ulp); {shown}")
        assert np.mean(g == want) >= 0.999, float(np.mean(g == want))
    else:
        scale = np.abs(want).max(axis=-1, keepdims=True) if ref_norm is None else ref_norm
        assert np.all(np.abs(g - want) <= 4e-7 * scale + 1e-30)


def assert_rel(got, want, rel: float, atol: float = 0.0, what: str = ""):
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    err = np.abs(g - w)
    bound = rel * np.abs(w) + atol
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside rel {rel} (worst {float(np.max(err - bound)):.3g})"


def check_against_oracle(w, got: dict, want: dict, planted=None):
    for g, m in enumerate(want["margin"]):
        assert m >= MARGIN, f"oracle margin {m:.3g} at the cut of group {g}: invalid case"
    if planted is not None:
        for g in range(len(planted)):
            assert np.array_equal(want["idx"][g], planted[g]), "oracle misses the planted set"
    idx = got["idx"].cpu().numpy().astype(np.int64)
    assert np.array_equal(idx, want["idx"]), "kept index sets differ"
    assert_rel(got["unit_score"], want["unit_score"], 2e-3, 0.0, "unit_score")
    if "k_rep" in got:   # kept where later steps read them
        assert_cache_close(got["k_rep"], want["k_rep"], w.dtype)
    if not w.decode:
        return
    if w.align:
        assert_cache_close(got["k_gather"], want["k_gather"], w.dtype)
    else:
        assert np.array_equal(OP.to64(got["k_gather"]), want["k_gather"]), "gathered keys"
    assert np.array_equal(OP.to64(got["v_gather"]), want["v_gather"]), "gathered values"
    assert_rel(got["o"], want["o"], 0.0, 5e-3, "decode output")
    assert_rel(got["lse"], want["lse"], 0.0, 2e-3, "lse")
