"""Helpers shared by the GPU tests: host arrays -> device tensors, and the tolerances.

Tolerances (max-abs, from the accuracy target of this decode path):
  * bf16 cache: O <= 1e-2, LSE <= 1e-3.
  * FP8 / NVFP4 cache: O <= 2e-2 against the oracle run on the dequantised cache; LSE
    keeps 1e-3, since dequantisation to bf16 is exact and only the accumulation differs.
Budget behind them: P is rounded to bf16 before the PV product (relative 2^-9 per
weight), and fp32 accumulation over <= 64k tokens adds ~1e-5 to the LSE.  The final O is
then rounded to bf16; check_o adds that rounding (half an ulp, <= 2^-8 |O|) to the
tolerance, since a row that sees only a few tokens can have |O| above 2.5.  The fp32
partials are compared without it.
"""

import sys

import numpy as np
import torch

TOL_O_BF16 = 1e-2
TOL_LSE = 1e-3
TOL_O_QUANT = 2e-2


def bf16_dev(bits: np.ndarray, dev="cuda:0") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def u8_dev(a: np.ndarray, dev="cuda:0") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def i32_dev(a: np.ndarray, dev="cuda:0") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Err(float):
    """A max-abs error that also remembers where it happened (shown when a test fails)."""

    def __new__(cls, v, where=""):
        o = super().__new__(cls, v)
        o.where = where
        return o

    def __repr__(self):
        return f"{float(self):.3e} {self.where}"


def max_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |got - want| where both are finite, +inf if the -inf / finite pattern differs."""
    gi, wi = np.isneginf(got), np.isneginf(want)
    if got.shape != want.shape:
        return Err(float("inf"), f"shape {got.shape} vs {want.shape}")
    if not np.array_equal(gi, wi):
        return Err(float("inf"), f"-inf pattern differs at {np.argwhere(gi != wi)[:4].tolist()}")
    if np.isnan(got).any():
        return Err(float("inf"), f"NaN at {np.argwhere(np.isnan(got))[:4].tolist()}")
    m = ~wi
    if not m.any():
        return Err(0.0)
    d = np.where(m, np.abs(got - np.where(m, want, 0)), 0)
    i = np.unravel_index(int(np.argmax(d)), d.shape)
    return Err(float(d[i]), f"at {tuple(int(x) for x in i)} got {got[i]:.6g} want {want[i]:.6g}")


def check(what: str, got: np.ndarray, want: np.ndarray, tol: float):
    """Assert max |got - want| <= tol, and print the margin (it shows in the test log)."""
    e = max_err(got, want)
    say(f"  {what}: max|d|={float(e):.3e} tol={tol:.0e} ({float(e) / tol:.2f} of tol)")
    assert e <= tol, (what, e)
    return e


def check_o(what: str, got: np.ndarray, want: np.ndarray, tol: float):
    """Check a final output O, which the kernels round to bf16 (nearest even): its
    rounding alone moves a value by up to half a bf16 ulp, at most 2^-8 |O|, which passes
    the fixed tolerances once |O| > 2.5 (a row that sees a few tokens takes the values of
    those tokens, up to about 4.5 here).  Asserts |got - want| <= tol + 2^-8 |want| and
    prints the margin."""
    e = max_err(got, want)
    if np.isfinite(float(e)) and got.size:
        m = ~np.isneginf(want)
        d = np.where(m, np.abs(got - np.where(m, want, 0)) - 2.0 ** -8 * np.abs(np.where(m, want, 0)), -np.inf)
        i = np.unravel_index(int(np.argmax(d)), d.shape)
        e = Err(max(float(d[i]), 0.0), f"at {tuple(int(x) for x in i)} got {got[i]:.6g} want {want[i]:.6g}")
    say(f"  {what}: max(|d| - 2^-8|O|)={float(e):.3e} tol={tol:.0e} ({float(e) / tol:.2f} of tol)")
    assert e <= tol, (what, e)
    return e


def paged_device_inputs(w, dev="cuda:0"):
    return dict(q=bf16_dev(w.q, dev), qpe=bf16_dev(w.qpe, dev), cache=u8_dev(w.cache, dev),
                bt=i32_dev(w.block_tables, dev), sl=i32_dev(w.seq_lens, dev))
