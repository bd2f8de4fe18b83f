"""GPU parity of the Q5_K / Q5_1 paths: the bit-exact decoders, and the
batched-expert call with its down projections in those formats, against the
oracle through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import q4_swiglu_mlp_amd as Z
import q4k_synth as S
from tests.gpu_common import assert_parity, dev, shifts_for, unscale

pytestmark = pytest.mark.gpu

FMTS = ["q5_k", "q5_1"]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(3, 256), (17, 768), (64, 2048)])
def test_q5_decoder_bit_exact(fmt, rows, cols):
    blob = S.gen_down_blob(np.random.default_rng(rows + cols), fmt, rows, cols)
    w = Z.zinc_q5_dequant_f32(fmt, dev(blob), rows, cols).cpu().numpy()
    ref = O.DOWN_DECODERS[fmt](blob, rows, cols).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def _inputs(fmt, E, H, I, M, k, seed):
    rng = np.random.default_rng(seed)
    wg = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wd = np.stack([S.gen_down_blob(rng, fmt, H, I) for _ in range(E)])
    x = S.gen_x(rng, M, H)
    ids, p = S.gen_routing(rng, M, E, k)
    return wg, wu, wd, x, ids, p


def _moe(fmt, wg, wu, wd, E, H, I, x, ids, p, a, b):
    y = Z.zinc_moe_experts_fmt(dev(wg), dev(wu), dev(wd), fmt, E, H, I, dev(x), dev(ids), dev(p), a, b)
    return unscale(y, b)


def _shift(y_ref):
    return max(0, int(np.ceil(np.log2(np.abs(y_ref).max() / 2 ** 13))))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("E,H,I,M,k,seed", [
    (4, 256, 256, 40, 2, 31),      # one 64-row panel chunks
    (16, 256, 768, 300, 4, 32),    # 192-row chunks at every panel offset, and 128-row chunks
    (8, 512, 1536, 90, 3, 33),     # chunks crossing a 256-row group
])
def test_moe_q5_down_matches_oracle(fmt, E, H, I, M, k, seed):
    wg, wu, wd, x, ids, p = _inputs(fmt, E, H, I, M, k, seed)
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I, fmt)
    assert bad == 0
    y = _moe(fmt, wg, wu, wd, E, H, I, x, ids, p, 0, _shift(y_ref))
    assert_parity(y, y_ref, f"moe {fmt} down E={E} H={H} I={I} M={M} k={k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_q5_top1_matches_dense_oracle(fmt):
    E, H, I, M = 4, 512, 512, 70
    wg, wu, wd, x, _, _ = _inputs(fmt, E, H, I, M, 1, 34)
    ids = np.full((M, 1), 2, np.int32)
    p = np.ones((M, 1), np.float32)
    y_ref, h_ref = O.mlp(x, wg[2], wu[2], wd[2], H, I, fmt)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(_moe(fmt, wg, wu, wd, E, H, I, x, ids, p, a, b), y_ref, f"moe {fmt} top-1 vs dense")


@pytest.mark.parametrize("fmt", FMTS)
def test_moe_q5_workload_size(fmt):
    # the E=64 top-8 2048 -> 768 M=512 shape with the down projections in fmt
    w = S.WORKLOADS["moe_e64"]
    rng = np.random.default_rng([w.seed, 50])
    wg, wu, _ = S.expert_weights(w.seed, w.n_experts, w.hidden, w.inter)
    wd = np.stack([S.gen_down_blob(rng, fmt, w.hidden, w.inter) for _ in range(w.n_experts)])
    x = S.workload_x(w)
    ids, p = S.workload_routing(w)
    y_ref, _ = O.moe(x, wg, wu, wd, ids, p, w.hidden, w.inter, fmt)
    y = _moe(fmt, wg, wu, wd, w.n_experts, w.hidden, w.inter, x, ids, p, w.inter_shift, _shift(y_ref))
    assert_parity(y, y_ref, f"moe {fmt} down E=64 top-8 M=512")


def test_moe_fmt_q4k_is_the_q4k_call():
    E, H, I, M, k = 8, 256, 512, 60, 2
    wg, wu, wd, x, ids, p = _inputs("q4_k", E, H, I, M, k, 35)
    y1 = Z.zinc_moe_experts_fmt(dev(wg), dev(wu), dev(wd), "q4_k", E, H, I, dev(x), dev(ids), dev(p), 0, 10)
    y2 = Z.zinc_moe_q4k_experts(dev(wg), dev(wu), dev(wd), E, H, I, dev(x), dev(ids), dev(p), 0, 10)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
