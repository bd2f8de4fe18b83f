"""Every entry point replayed from a captured HIP graph gives the eager
call's bits, replay after replay, with other eager work in between."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import q4_swiglu_mlp_amd as Z
import q4k_synth as S
from tests.gpu_common import dev

pytestmark = pytest.mark.gpu


def _replays_match(call, y, replays=3):
    """call() enqueues the entry point on the current stream writing y."""
    call()
    torch.cuda.synchronize()
    want = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                      # warm the path on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    scratch = torch.randn(1 << 20, device="cuda:0")
    for r in range(replays):
        y.zero_()
        (scratch * 2.0).sum().item()     # unrelated eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {r} differs from the eager call"


def _dense(seed, H, I, M):
    rng = np.random.default_rng(seed)
    return ([dev(S.gen_q4k_blob(rng, I, H)), dev(S.gen_q4k_blob(rng, I, H)), dev(S.gen_q4k_blob(rng, H, I))],
            dev(S.gen_x(rng, M, H)))


@pytest.mark.parametrize("M", [1, 4, 100])
def test_graph_dense(M):
    H, I = 512, 1280
    w, x = _dense(60 + M, H, I, M)
    y = torch.empty((M, H), dtype=torch.float16, device="cuda:0")
    if M <= 8:
        ws = torch.empty(Z.decode_workspace_size(M, H, I), dtype=torch.uint8, device="cuda:0")
        _replays_match(lambda: Z.zinc_mlp_q4k_decode(*w, H, I, x, 2, 10, y=y, workspace=ws), y)
    ws = torch.empty(Z.prefill_workspace_size(M, H, I), dtype=torch.uint8, device="cuda:0")
    _replays_match(lambda: Z.zinc_mlp_q4k_prefill(*w, H, I, x, 2, 10, y=y, workspace=ws), y)


def test_graph_block_and_staged():
    H, I, M = 512, 1280, 70
    w, x = _dense(64, H, I, M)
    g = dev(np.random.default_rng(65).uniform(0.5, 1.5, H).astype(np.float16))
    y = torch.empty((M, H), dtype=torch.float16, device="cuda:0")
    ws = torch.empty(int(Z.lib.zinc_mlp_q4k_prefill_block_workspace_size(M, H, I)), dtype=torch.uint8,
                     device="cuda:0")
    _replays_match(lambda: Z.zinc_mlp_q4k_prefill_block(*w, H, I, x, g, 1e-5, 2.0 ** -8, 2, 10, y=y, workspace=ws), y)
    ws2 = torch.empty(Z.prefill_staged_workspace_size(M, H, I), dtype=torch.uint8, device="cuda:0")
    _replays_match(lambda: Z.zinc_mlp_q4k_prefill_staged(*w, H, I, x, 2, 10, y=y, workspace=ws2), y)


@pytest.mark.parametrize("fmt", ["q4_k", "q5_1"])
def test_graph_router_and_experts(fmt):
    E, H, I, M, k = 8, 256, 512, 60, 2
    rng = np.random.default_rng(66)
    wg = dev(np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)]))
    wu = dev(np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)]))
    wd = dev(np.stack([S.gen_down_blob(rng, fmt, H, I) for _ in range(E)]))
    x = dev(S.gen_x(rng, M, H))
    logits = dev(S.gen_router_logits(rng, M, E))
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda:0")
    p = torch.empty((M, k), dtype=torch.float32, device="cuda:0")
    y = torch.empty((M, H), dtype=torch.float16, device="cuda:0")
    ws = torch.empty(Z.moe_workspace_size(M, k, E, H, I), dtype=torch.uint8, device="cuda:0")

    def layer():
        Z.zinc_moe_route_topk(logits, k, expert_ids=ids, expert_weights=p)
        Z.zinc_moe_experts_fmt(wg, wu, wd, fmt, E, H, I, x, ids, p, 0, 10, y=y, workspace=ws)

    _replays_match(layer, y)
