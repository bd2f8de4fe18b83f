"""Calls enqueued on a side stream: the binding allocates the call's
temporaries (y and the workspace) on that stream, so memory the call still
uses is not handed to work on the default stream while the side stream runs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import q4_swiglu_mlp_amd as Z
import q4k_synth as S
from tests.gpu_common import dev

pytestmark = pytest.mark.gpu


def _slow_work(s, n=4096, reps=12):
    # keeps the side stream busy for a while before the library's kernels run
    with torch.cuda.stream(s):
        a = torch.randn((n, n), device="cuda:0")
        for _ in range(reps):
            a = a @ a
            a = a / a.norm()
    return a


@pytest.mark.parametrize("entry", ["prefill", "decode", "moe"])
def test_side_stream_temporaries_survive_default_stream_allocations(entry):
    rng = np.random.default_rng(90)
    H, I = 1024, 2816
    M = 200 if entry != "decode" else 4
    if entry == "moe":
        E, k = 8, 2
        wg = dev(np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)]))
        wu = dev(np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)]))
        wd = dev(np.stack([S.gen_q4k_blob(rng, H, I) for _ in range(E)]))
        x = dev(S.gen_x(rng, M, H))
        ids, p = (dev(a) for a in S.gen_routing(rng, M, E, k))

        def call(stream=None):
            return Z.zinc_moe_q4k_experts(wg, wu, wd, E, H, I, x, ids, p, 3, 12, stream=stream)
        ws_bytes = Z.moe_workspace_size(M, k, E, H, I)
    else:
        wg, wu, wd = (dev(S.gen_q4k_blob(rng, I, H)), dev(S.gen_q4k_blob(rng, I, H)), dev(S.gen_q4k_blob(rng, H, I)))
        x = dev(S.gen_x(rng, M, H))
        fn = Z.zinc_mlp_q4k_prefill if entry == "prefill" else Z.zinc_mlp_q4k_decode

        def call(stream=None):
            return fn(wg, wu, wd, H, I, x, 3, 12, stream=stream)
        ws_bytes = (Z.prefill_workspace_size if entry == "prefill" else Z.decode_workspace_size)(M, H, I)

    want = call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    keep = _slow_work(s)
    got = call(stream=s)
    # the call's workspace was freed on return; the default stream now
    # allocates blocks of that size and overwrites them while s still runs
    junk = [torch.full((max(ws_bytes, 16),), 0xFF, dtype=torch.uint8, device="cuda:0") for _ in range(4)]
    junk_y = [torch.full(tuple(want.shape), float("nan"), dtype=torch.float16, device="cuda:0") for _ in range(4)]
    torch.cuda.synchronize()
    del keep, junk, junk_y
    assert torch.equal(got, want), f"{entry}: the side-stream call differs from the default-stream call"
