"""GPU parity of the MoE router (zinc_moe_route_topk) against the oracle:
expert ids bit-exact (both sides rank the same fp32 logits), mixing weights
within fp32 rounding of the float64 softmax, and the router's device buffers
fed straight into the batched-expert call."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import q4_swiglu_mlp_amd as Z
import q4k_synth as S
from tests.gpu_common import assert_parity, dev, unscale

pytestmark = pytest.mark.gpu

# fp32 softmax of at most 64 values: exp within a few ulp, one division, a
# 64-term sum -> a few 1e-7 relative; weights below 1e-30 are compared absolutely
P_RTOL, P_ATOL = 2e-6, 1e-30


def _route_gpu(logits: np.ndarray, k: int):
    ids, p = Z.zinc_moe_route_topk(dev(logits), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), p.cpu().numpy().astype(np.float64)


def _check(logits, k, what):
    ids_ref, p_ref = O.route_topk(logits, k)
    ids, p = _route_gpu(logits, k)
    print(f"[router] {what}: M={logits.shape[0]} E={logits.shape[1]} k={k}", flush=True)
    assert np.array_equal(ids, ids_ref), what
    nan_ref = np.isnan(p_ref)
    assert np.array_equal(np.isnan(p), nan_ref), what
    assert np.allclose(p[~nan_ref], p_ref[~nan_ref], rtol=P_RTOL, atol=P_ATOL), what


@pytest.mark.parametrize("M,E,k", [(1, 1, 1), (7, 7, 3), (100, 64, 8), (513, 65, 8), (64, 128, 64),
                                   (33, 257, 16), (10, 1024, 64), (1000, 64, 8), (5, 1000, 1)])
def test_router_matches_oracle(M, E, k):
    rng = np.random.default_rng(1000 + M + E + k)
    _check(S.gen_router_logits(rng, M, E, scale=2.0), k, "normal logits")


def test_router_ties_infinities_and_nans():
    rng = np.random.default_rng(77)
    L = rng.integers(-2, 3, size=(300, 70)).astype(np.float32)    # many equal logits
    L[5, :] = 0.0                                                    # all equal
    L[6, ::3] = -np.inf
    L[7, [1, 9, 40]] = np.nan                                        # skipped while numbers remain
    L[8, :] = np.nan                                                 # all NaN: lowest indices, NaN weights
    L[9, :66] = np.nan                                               # fewer numbers than k
    L[10, :] = -np.inf                                               # all -inf: NaN weights
    L[11, 3] = 1e30                                                  # one dominant logit
    _check(L, 8, "ties / inf / NaN")


def test_router_workload_size():
    w = S.WORKLOADS["moe_e64"]
    _check(S.workload_router_logits(w), w.top_k, "E=64 top-8 M=512")


def test_router_zero_tokens_writes_nothing():
    logits = torch.zeros((0, 64), dtype=torch.float32, device="cuda:0")
    ids = torch.full((1, 8), -7, dtype=torch.int32, device="cuda:0")
    p = torch.full((1, 8), 3.0, dtype=torch.float32, device="cuda:0")
    # the outputs are [0, 8] views at the start of the guard buffers
    Z.zinc_moe_route_topk(logits, 8, expert_ids=ids[:0], expert_weights=p[:0])
    torch.cuda.synchronize()
    assert torch.all(ids == -7) and torch.all(p == 3.0)


def test_router_feeds_expert_call():
    # logits -> GPU router -> ids/p on the device -> batched experts, against
    # the oracle's router and MoE
    E, H, I, M, k = 16, 256, 512, 200, 4
    rng = np.random.default_rng(78)
    wg = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wd = np.stack([S.gen_q4k_blob(rng, H, I) for _ in range(E)])
    x = S.gen_x(rng, M, H)
    logits = S.gen_router_logits(rng, M, E)
    ids_ref, p_ref = O.route_topk(logits, k)
    y_ref, bad = O.moe(x, wg, wu, wd, ids_ref, p_ref.astype(np.float32), H, I)
    assert bad == 0
    b = max(0, int(np.ceil(np.log2(np.abs(y_ref).max() / 2 ** 13))))
    gids, gp = Z.zinc_moe_route_topk(dev(logits), k)
    y = Z.zinc_moe_q4k_experts(dev(wg), dev(wu), dev(wd), E, H, I, dev(x), gids, gp, 0, b)
    assert np.array_equal(gids.cpu().numpy(), ids_ref)
    assert_parity(unscale(y, b), y_ref, "router -> experts")
