"""GPU parity of the MLP block entry points (pre-MLP RMS norm, MLP, residual
and per-layer scale) against the oracle, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import q4_swiglu_mlp_amd as Z
import q4k_synth as S
from tests.gpu_common import assert_parity, dev, shifts_for, unscale

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _inputs(seed, H, I, M, workload=None):
    rng = np.random.default_rng(seed)
    if workload is not None:
        w = S.WORKLOADS[workload]
        wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
        x = S.workload_x(w, M=M)
    else:
        wg, wu, wd = S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, H, I)
        x = S.gen_x(rng, M, H)
    gamma = rng.uniform(0.5, 1.5, H).astype(np.float16)
    return wg, wu, wd, x, gamma


def _balanced(x, gamma, wg, wu, wd, H, I):
    """A per-layer scale that makes the residual and the scaled MLP output
    equally large (so both are checked), and the shifts for that output."""
    xn = O.rms_norm(x, gamma, EPS)
    ym, h = O.mlp(xn, wg, wu, wd, H, I)
    s = float(2.0 ** np.round(np.log2(np.sqrt(np.mean(x.astype(np.float64) ** 2)) / np.sqrt(np.mean(ym ** 2)))))
    y_ref = x.astype(np.float64) + s * ym
    a, _ = shifts_for(ym, h)
    _, b = shifts_for(y_ref, h)
    return s, a, b, y_ref


def _run(fn, wg, wu, wd, H, I, x, gamma, s, a, b, **kw):
    y = fn(dev(wg), dev(wu), dev(wd), H, I, dev(x), dev(gamma), EPS, s, a, b, **kw)
    return unscale(y, b)


@pytest.mark.parametrize("M", [1, 65, 256])
def test_prefill_block_matches_oracle(M):
    wg, wu, wd, x, gamma = _inputs(90 + M, 4096, 11008, M, workload="prefill_m256")
    H, I = 4096, 11008
    s, a, b, y_ref = _balanced(x, gamma, wg, wu, wd, H, I)
    y = _run(Z.zinc_mlp_q4k_prefill_block, wg, wu, wd, H, I, x, gamma, s, a, b)
    assert_parity(y, y_ref, f"prefill block M={M}, scale {s}")


@pytest.mark.parametrize("M", [1, 3, 4, 8])
def test_decode_block_matches_oracle(M):
    H, I = 256, 768
    wg, wu, wd, x, gamma = _inputs(95 + M, H, I, M)
    s, a, b, y_ref = _balanced(x, gamma, wg, wu, wd, H, I)
    yd = _run(Z.zinc_mlp_q4k_decode_block, wg, wu, wd, H, I, x, gamma, s, a, b)
    yp = _run(Z.zinc_mlp_q4k_prefill_block, wg, wu, wd, H, I, x, gamma, s, a, b)
    assert_parity(yd, y_ref, f"decode block M={M}")
    assert_parity(yp, y_ref, f"prefill block M={M}")


def test_decode_block_workload_m1():
    w = S.WORKLOADS["decode_m1"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.workload_x(w)
    gamma = np.random.default_rng(97).uniform(0.5, 1.5, w.hidden).astype(np.float16)
    s, a, b, y_ref = _balanced(x, gamma, wg, wu, wd, w.hidden, w.inter)
    y = _run(Z.zinc_mlp_q4k_decode_block, wg, wu, wd, w.hidden, w.inter, x, gamma, s, a, b)
    assert_parity(y, y_ref, "decode block 4096/11008 M=1")


@pytest.mark.parametrize("which", ["prefill", "decode"])
def test_block_in_place_and_zero_scale(which):
    fn = Z.zinc_mlp_q4k_prefill_block if which == "prefill" else Z.zinc_mlp_q4k_decode_block
    H, I, M = 512, 1024, (100 if which == "prefill" else 4)
    wg, wu, wd, x, gamma = _inputs(98, H, I, M)
    s, a, b, _ = _balanced(x, gamma, wg, wu, wd, H, I)
    gw = [dev(v) for v in (wg, wu, wd)]
    gx, gg = dev(x), dev(gamma)
    y_out = fn(*gw, H, I, gx, gg, EPS, s, a, b)
    # y aliasing x: the residual update in place gives the same bits
    gx2 = gx.clone()
    fn(*gw, H, I, gx2, gg, EPS, s, a, b, y=gx2)
    torch.cuda.synchronize()
    assert torch.equal(gx2, y_out)
    # zero scale: y is the residual exactly (no shift)
    y0 = fn(*gw, H, I, gx, gg, EPS, 0.0, a, 0)
    torch.cuda.synchronize()
    assert torch.equal(y0, gx)
