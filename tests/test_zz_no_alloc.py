"""The decode entry point that allocates nothing (zinc_mlp_q4k_decode_noalloc),
called through the C ABI: the same bits as zinc_mlp_q4k_decode on two calls in
a row, the second with fewer tokens and a shorter intermediate, so it reuses
the library's device-resident scratch array left as the first call wrote it;
and its size limit, rejected on the host."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import q4_swiglu_mlp_amd as Z
import q4k_synth as S
from tests.gpu_common import assert_parity, dev, shifts_for

A = 0x10000   # a 16-byte aligned fake device address (never dereferenced)

_fn = Z.lib.zinc_mlp_q4k_decode_noalloc            # the C entry point (argument types set by the binding)
_max = Z.lib.zinc_mlp_q4k_decode_noalloc_max_bytes


def _noalloc(wg, wu, wd, H, I, x, y, a, b, stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return _fn(wg.data_ptr(), wu.data_ptr(), wd.data_ptr(), H, I, x.data_ptr(), y.data_ptr(), int(x.shape[0]), a, b,
               s.cuda_stream)


def test_noalloc_limit_rejected_on_the_host():
    cap = int(_max())
    assert cap == 512 << 10
    # 8 tokens x 65536 intermediate = 1 MiB of intermediate: over the limit,
    # refused before any HIP call (fake pointers, no GPU needed)
    assert _fn(A, A, A, 256, 65536, A, A, 8, 0, 0, None) == -4
    assert _fn(A, A, A, 256, 768, A, A, 9, 0, 0, None) == -5       # M above 8
    assert _fn(A, A, A, 256, 768, A, A, 0, 0, 0, None) == 0        # M = 0: nothing to do
    assert _fn(None, A, A, 256, 768, A, A, 1, 0, 0, None) == -1
    assert _fn(A, A, A, 300, 768, A, A, 1, 0, 0, None) == -2
    assert _fn(A + 4, A, A, 256, 768, A, A, 1, 0, 0, None) == -3


@pytest.mark.gpu
def test_noalloc_matches_decode_on_two_calls_in_a_row():
    # first call: 4096/11008, M = 8 (176 KB of intermediate, the eight-token
    # kernels); second: a smaller layer and M = 1, reading the array the first
    # call left behind
    cases = []
    w = S.WORKLOADS["decode_m4"]
    wg, wu, wd = S.layer_weights(w.seed, 5, w.hidden, w.inter)
    rng = np.random.default_rng(17)
    cases.append((wg, wu, wd, w.hidden, w.inter, S.gen_x(rng, 8, w.hidden)))
    H, I = 1024, 2816
    cases.append((S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, H, I), H, I,
                  S.gen_x(rng, 1, H)))
    for wg, wu, wd, H, I, x in cases:
        print(f"[noalloc] H={H} I={I} M={x.shape[0]}", flush=True)
        y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
        a, b = shifts_for(y_ref, h_ref)
        gw = [dev(wg), dev(wu), dev(wd)]
        gx = dev(x)
        y_na = torch.full((x.shape[0], H), float("nan"), dtype=torch.float16, device="cuda:0")
        st = _noalloc(*gw, H, I, gx, y_na, a, b)
        assert st == 0, Z.strerror(st)
        y_ws = Z.zinc_mlp_q4k_decode(*gw, H, I, gx, a, b)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), "no-allocation decode differs from the workspace decode"
        assert_parity(y_na.float().cpu().numpy().astype(np.float64) * 2.0 ** b, y_ref, f"noalloc H={H} M={x.shape[0]}")
