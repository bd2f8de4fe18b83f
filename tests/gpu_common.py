"""Helpers for the GPU parity tests: device copies, calls through the binding
(which calls the C ABI), and the oracle comparison."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import q4_swiglu_mlp_amd as Z

DEV = torch.device("cuda:0")


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def unscale(y: torch.Tensor, out_shift: int) -> np.ndarray:
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64) * 2.0 ** out_shift


def prefill(wg, wu, wd, hidden, inter, x, a, b, **kw):
    y = Z.zinc_mlp_q4k_prefill(dev(wg), dev(wu), dev(wd), hidden, inter, dev(x), a, b, **kw)
    return unscale(y, b)


def decode(wg, wu, wd, hidden, inter, x, a, b, **kw):
    y = Z.zinc_mlp_q4k_decode(dev(wg), dev(wu), dev(wd), hidden, inter, dev(x), a, b, **kw)
    return unscale(y, b)


def assert_parity(y_test: np.ndarray, y_ref: np.ndarray, what: str = "") -> dict:
    m = O.parity_metrics(y_test, y_ref)
    print(f"[parity] {what}: max|err|/rms={m['max_err_over_rms']:.3e} mean rel={m['mean_rel_err']:.3e}", flush=True)
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_err_over_rms"] <= O.MAX_ERR_OVER_RMS, f"{what}: {m}"
    assert m["mean_rel_err"] <= O.MEAN_REL_ERR, f"{what}: {m}"
    return m


def shifts_for(y_ref: np.ndarray, h_ref: np.ndarray) -> tuple[int, int]:
    """Smallest power-of-two exponents keeping |h|, |y| at most 2^13 (4x below 2^15)."""
    def need(v):
        mx = float(np.abs(v).max())
        return max(0, int(np.ceil(np.log2(mx / 2 ** 13)))) if mx > 0 else 0
    return need(h_ref), need(y_ref)
