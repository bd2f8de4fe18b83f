"""GPU parity: every entry point through the C ABI against the CPU oracle on the
same seeded inputs.  Decoder: bit-exact.  MLP outputs: max|err| <= 2e-2 RMS(ref)
and sum|err|/sum|ref| <= 5e-3 (the acceptance bound of the study)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import q4_swiglu_mlp_amd as Z
import q4k_synth as S
from tests import q4k_blocks as B
from tests.gpu_common import assert_parity, decode, dev, prefill, shifts_for, unscale

pytestmark = pytest.mark.gpu


def _rand_mlp(seed, H, I, M, sd=1.0):
    rng = np.random.default_rng(seed)
    wg = S.gen_q4k_blob(rng, I, H)
    wu = S.gen_q4k_blob(rng, I, H)
    wd = S.gen_q4k_blob(rng, H, I)
    x = S.gen_x(rng, M, H, sd)
    return wg, wu, wd, x


# ---------------------------------------------------------------------------
# decoder: bit-exact fp32
# ---------------------------------------------------------------------------
def _dequant_bits(blob, rows, cols):
    out = Z.zinc_q4k_dequant_f32(dev(blob), rows, cols)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def test_dequant_bit_exact_tiny_workload():
    w = S.WORKLOADS["tiny"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    for blob, r, c in ((wg, w.inter, w.hidden), (wu, w.inter, w.hidden), (wd, w.hidden, w.inter)):
        assert np.array_equal(_dequant_bits(blob, r, c), O.q4k_dequant_f32(blob, r, c).view(np.uint32))


def test_dequant_bit_exact_hand_built_blocks():
    blocks = [B.block(), B.unit_block()]
    for k in range(12):
        Sb = [0] * 12
        Sb[k] = 0xFF
        blocks.append(B.block(B.F16_ONE, 0, Sb, [0x11] * 128))
        blocks.append(B.block(0, B.F16_ONE, Sb, [0x11] * 128))
    for byte in range(128):
        for nib in (0x01, 0x10):
            Q = [0] * 128
            Q[byte] = nib
            blocks.append(B.block(B.F16_ONE, 0, B.S_UNIT_SCALES, Q))
    blocks.append(B.block(B.F16_NEG_ONE, B.F16_HALF, [0xFF] * 12, [0xFF] * 128))
    blob = np.stack(blocks).reshape(len(blocks), 1, 144)
    assert np.array_equal(_dequant_bits(blob, len(blocks), 256),
                          O.q4k_dequant_f32(blob, len(blocks), 256).view(np.uint32))


def test_dequant_bit_exact_full_down_matrix():
    w = S.WORKLOADS["prefill_m256"]
    _, _, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    got = _dequant_bits(wd, w.hidden, w.inter)
    ref = O.q4k_dequant_f32(wd, w.hidden, w.inter).view(np.uint32)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# fused prefill
# ---------------------------------------------------------------------------
def test_prefill_tiny_workload():
    w = S.WORKLOADS["tiny"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.workload_x(w)
    y_ref, _ = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    assert_parity(prefill(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift), y_ref, "prefill tiny")


@pytest.mark.parametrize("M", [1, 3, 31, 63, 64, 65, 127, 200])
def test_prefill_ragged_token_counts(M):
    H, I = 512, 768
    wg, wu, wd, x = _rand_mlp(100 + M, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, f"prefill M={M}")


@pytest.mark.parametrize("H,I", [(256, 1280), (768, 256), (1024, 2304)])
def test_prefill_other_shapes(H, I):
    M = 70
    wg, wu, wd, x = _rand_mlp(H + I, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, f"prefill H={H} I={I}")


@pytest.mark.parametrize("H,I,M", [(512, 1536, 512), (512, 1536, 600), (768, 1280, 1000), (256, 2304, 530),
                                   (512, 256, 640), (256, 2816, 2048)])
def test_prefill_unit_e(H, I, M):
    # from 512 tokens the plan takes the 128-token unit (two 128-row passes per
    # chunk of at most 256 rows): several tiles and chunks, ragged token tails,
    # chunks of two panels (one pass) and of two or three panels (the second
    # pass half idle, 2816 / 64 = 44 panels in 16 chunks)
    wg, wu, wd, x = _rand_mlp(300 + M + I, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, f"prefill unit E H={H} I={I} M={M}")


@pytest.mark.parametrize("M", [257, 320, 500])
def test_prefill_unit_c(M):
    # past four 64-token tiles the plan takes the 32x32x16 unit with 384-row
    # chunks (unit C): several tiles, chunks and a ragged tail
    H, I = 512, 1280
    wg, wu, wd, x = _rand_mlp(77 + M, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, f"prefill unit C M={M}")


def test_prefill_m256_workload_full():
    w = S.WORKLOADS["prefill_m256"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.workload_x(w)
    y = prefill(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift)
    y_ref, _ = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    assert_parity(y, y_ref, "prefill 4096/11008 M=256")


@pytest.mark.parametrize("H,I,M", [(16384, 256, 3), (256, 65536, 2)])
def test_max_sizes(H, I, M):
    # the library's largest hidden and intermediate widths (the row decode
    # kernels' longest contraction is hidden = 16384; inter = 65536 sends M = 1
    # decode to the MFMA kernels' passes)
    wg, wu, wd, x = _rand_mlp(70 + M, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, f"prefill H={H} I={I} M={M}")
    assert_parity(decode(wg, wu, wd, H, I, x, a, b), y_ref, f"decode H={H} I={I} M={M}")
    assert_parity(decode(wg, wu, wd, H, I, x[:1], a, b), y_ref[:1], f"decode H={H} I={I} M=1")


@pytest.mark.parametrize("M", [150, 256, 257, 320, 383, 520])
def test_prefill_default_plan_switch(M):
    # the default unit changes past four 64-token tiles (16x16x32 unit up to
    # 256 tokens, 32x32x16 unit with 384-row chunks after), and the chunk count
    # with the number of tiles: both sides of each change
    H, I = 1024, 2304
    wg, wu, wd, x = _rand_mlp(40 + M, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, f"prefill default plan M={M}")


def test_prefill_workspace_sized_for_larger_m():
    # one workspace sized for 520 tokens serves calls with fewer tokens, on
    # both sides of the unit switch, with the same result as a workspace of
    # each call's own size (the plan, hence the arithmetic, is the same)
    H, I = 1024, 2304
    M_max = 520
    wg, wu, wd, x = _rand_mlp(77, H, I, M_max)
    a, b = shifts_for(*O.mlp(x, wg, wu, wd, H, I))
    gw, uw, dw = dev(wg), dev(wu), dev(wd)
    ws = torch.empty(Z.prefill_workspace_size(M_max, H, I), dtype=torch.uint8, device="cuda")
    for M in (520, 257, 256, 130, 1):
        xm = dev(x[:M])
        y_shared = Z.zinc_mlp_q4k_prefill(gw, uw, dw, H, I, xm, a, b, workspace=ws)
        y_own = Z.zinc_mlp_q4k_prefill(gw, uw, dw, H, I, xm, a, b)
        torch.cuda.synchronize()
        assert torch.equal(y_shared, y_own), f"shared workspace M={M}"


@pytest.mark.parametrize("M", [1, 65, 256])
def test_prefill_staged_baseline_matches(M):
    # the comparison baseline (intermediate in device memory) computes the
    # same y: against the oracle, and close to the fused call (it rounds G
    # and U to fp16 on the way, the fused call does not)
    w = S.WORKLOADS["prefill_m256"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.workload_x(w, M=M)
    ys = unscale(Z.zinc_mlp_q4k_prefill_staged(dev(wg), dev(wu), dev(wd), w.hidden, w.inter, dev(x), w.inter_shift,
                                               w.out_shift), w.out_shift)
    yf = prefill(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift)
    y_ref, _ = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    assert_parity(ys, y_ref, f"staged baseline M={M}")
    assert_parity(ys, yf, f"staged baseline vs fused M={M}")


@pytest.mark.parametrize("layer", [0, 31])
def test_prefill_m2048_workload_sampled_tokens(layer):
    w = S.WORKLOADS["prefill_m2048"]
    wg, wu, wd = S.layer_weights(w.seed, layer, w.hidden, w.inter)
    x = S.workload_x(w)
    y = prefill(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift)
    rng = np.random.default_rng(layer)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 2047], rng.choice(w.M, 59, replace=False)]))
    y_ref, _ = O.mlp(x[rows], wg, wu, wd, w.hidden, w.inter)   # tokens are independent rows
    assert_parity(y[rows], y_ref, f"prefill M=2048 layer {layer}, {len(rows)} sampled tokens")


def test_prefill_large_m_sampled_tokens():
    # 8200 tokens (a ragged last 128-token tile) put the split-K partials at
    # 43 x 8200 x 4096 x 2 B = 2.9 GB, past 2^31 bytes: every partial and
    # workspace offset must be 64-bit
    w = S.WORKLOADS["prefill_m2048"]
    M = 8200
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.gen_x(np.random.default_rng([w.seed, M]), M, w.hidden, w.x_sd)
    assert Z.prefill_workspace_size(M, w.hidden, w.inter) > 2**31
    y = prefill(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095, 4096, 8191, 8192, M - 1], rng.choice(M, 23, replace=False)]))
    y_ref, _ = O.mlp(x[rows], wg, wu, wd, w.hidden, w.inter)   # tokens are independent rows
    assert_parity(y[rows], y_ref, f"prefill M={M}, {len(rows)} sampled tokens")


def test_prefill_intermediate_near_fp16_limit():
    # the shift is one less than the 4x-headroom choice, so the fp16 strip holds
    # values up to 2^14: sums of 32 such values would overflow fp16, the kernel's
    # sub-block means must not
    H, I, M = 512, 768, 96
    wg, wu, wd, x = _rand_mlp(12, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    a = max(a - 1, 0)
    assert np.abs(h_ref).max() * 2.0 ** -a < 65504
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, "prefill strip near fp16 limit")


# structured probes (a layout slip inside the fused kernel shows up here even
# when the mean-dominated random case still passes)
def test_prefill_zero_input_is_exact_zero():
    H, I, M = 512, 768, 40
    wg, wu, wd, _ = _rand_mlp(7, H, I, M)
    y = prefill(wg, wu, wd, H, I, np.zeros((M, H), np.float16), 0, 0)
    assert np.all(y == 0.0)


def test_prefill_one_hot_inputs():
    H, I, M = 512, 768, 64
    wg, wu, wd, _ = _rand_mlp(8, H, I, M)
    x = np.zeros((M, H), np.float16)
    x[np.arange(M), (np.arange(M) * 37) % H] = 1.0      # token t selects hidden column 37t mod H
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, "prefill one-hot x")


def test_prefill_unit_up_weights():
    H, I, M = 512, 768, 64
    wg, _, wd, x = _rand_mlp(9, H, I, M)
    wu = B.unit_matrix(I, H)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, "prefill W_up = 1")


def test_prefill_single_subblock_down_rows():
    # every W_down row has exactly one non-zero sub-block (zero mins), so each
    # output reads one 32-wide slice of the strip: a staging slip moves it.
    H, I, M = 512, 768, 64
    wg, wu, wd, x = _rand_mlp(10, H, I, M)
    rng = np.random.default_rng(11)
    wd = wd.copy()
    nbI = I // 256
    wd[:, :, 2:4] = 0                       # dmin = 0
    wd[:, :, 4:16] = 0                      # all scales and mins 0
    for r in range(H):
        b = rng.integers(nbI)
        j = rng.integers(8)
        sc = rng.integers(1, 64)
        if j < 4:
            wd[r, b, 4 + j] = sc
        else:
            wd[r, b, 4 + j + 4] = sc & 15
            wd[r, b, 4 + j - 4] = (sc >> 4) << 6
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, "prefill single-sub-block W_down")


# ---------------------------------------------------------------------------
# decode pair
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_decode_tiny_workload(M):
    w = S.WORKLOADS["tiny"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.workload_x(w)[:M]
    y_ref, _ = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    assert_parity(decode(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift), y_ref, f"decode tiny M={M}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_decode_long_down_contraction(M):
    # inter = 16640 > 16384: longer than the M = 1 row kernels cover, so both M
    # take the MFMA passes; the prefill kernel runs the same shape
    H, I = 256, 16640
    wg, wu, wd, x = _rand_mlp(777 + M, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(decode(wg, wu, wd, H, I, x, a, b), y_ref, f"decode H={H} I={I} M={M}")
    assert_parity(prefill(wg, wu, wd, H, I, x, a, b), y_ref, f"prefill H={H} I={I} M={M}")


@pytest.mark.parametrize("name,layer", [("decode_m1", 0), ("decode_m4", 0), ("decode_m4", 17)])
def test_decode_workloads(name, layer):
    w = S.WORKLOADS[name]
    wg, wu, wd = S.layer_weights(w.seed, layer, w.hidden, w.inter)
    x = S.workload_x(w)
    y_ref, _ = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    assert_parity(decode(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift), y_ref, f"{name} layer {layer}")


@pytest.mark.parametrize("M", [6, 8])
def test_decode_eight_token_group_full_size(M):
    # five to eight tokens share one launch per pass (two blocks per wave and
    # pass), here at the 4096/11008 shape: the down pass takes two passes
    w = S.WORKLOADS["decode_m4"]
    wg, wu, wd = S.layer_weights(w.seed, 5, w.hidden, w.inter)
    x = S.gen_x(np.random.default_rng(880 + M), M, w.hidden)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(decode(wg, wu, wd, w.hidden, w.inter, x, a, b), y_ref, f"decode 4096/11008 M={M}")


@pytest.mark.parametrize("M", [1, 4])
def test_decode_repeated_calls_reuse_workspace(M):
    # back-to-back calls on one workspace (filled with garbage first) give the
    # same result bit for bit: every row is summed in a fixed order
    w = S.WORKLOADS["decode_m4"]
    wts = S.layer_weights(w.seed, 3, w.hidden, w.inter)
    wg, wu, wd = (dev(a) for a in wts)
    x = S.workload_x(w)[:M]
    y_ref, _ = O.mlp(x, *wts, w.hidden, w.inter)
    ws = torch.full((Z.decode_workspace_size(M, w.hidden, w.inter),), 0x5A, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        y = Z.zinc_mlp_q4k_decode(wg, wu, wd, w.hidden, w.inter, dev(x), w.inter_shift, w.out_shift, workspace=ws)
        outs.append(unscale(y, w.out_shift))
    for y in outs:
        assert_parity(y, y_ref, f"decode M={M} repeated")
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


# the MFMA decode kernels at hidden widths of one to four 4096-wide spans (the
# library's maximum, eight passes per wave at eight tokens), and one that is
# not a multiple of 4096 (the K split's last pass ragged)
@pytest.mark.parametrize("H", [4096, 4352, 8192, 12288, 16384])
@pytest.mark.parametrize("M", [2, 3, 4, 5, 8])
def test_decode_mfma_hidden_widths(M, H):
    I = 768
    wg, wu, wd, x = _rand_mlp(4100 + M + H, H, I, M)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(decode(wg, wu, wd, H, I, x, a, b), y_ref, f"decode H={H} I={I} M={M}")


def test_decode_and_prefill_agree_at_m8():
    w = S.WORKLOADS["tiny"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.workload_x(w)
    y_ref, _ = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    yd = decode(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift)
    yp = prefill(wg, wu, wd, w.hidden, w.inter, x, w.inter_shift, w.out_shift)
    assert_parity(yd, y_ref, "decode M=8")
    assert_parity(yp, y_ref, "prefill M=8")
    assert_parity(yd, yp, "decode vs prefill")


# ---------------------------------------------------------------------------
# batched-expert MoE
# ---------------------------------------------------------------------------
def _moe_inputs(E, H, I, M, k, seed):
    rng = np.random.default_rng(seed)
    wg = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wd = np.stack([S.gen_q4k_blob(rng, H, I) for _ in range(E)])
    x = S.gen_x(rng, M, H)
    ids, p = S.gen_routing(rng, M, E, k)
    return wg, wu, wd, x, ids, p


def _moe_gpu(wg, wu, wd, E, H, I, x, ids, p, a, b, dev_error=None):
    y = Z.zinc_moe_q4k_experts(dev(wg), dev(wu), dev(wd), E, H, I, dev(x), dev(ids), dev(p), a, b,
                               dev_error=dev_error)
    return unscale(y, b)


def test_moe_tiny():
    E, H, I, M, k = 4, 256, 256, 40, 2
    wg, wu, wd, x, ids, p = _moe_inputs(E, H, I, M, k, 21)
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I)
    assert bad == 0
    assert_parity(_moe_gpu(wg, wu, wd, E, H, I, x, ids, p, 0, 8), y_ref, "moe E=4 top-2")


@pytest.mark.parametrize("E,k,M", [(1024, 16, 40), (3, 3, 50)])
def test_moe_expert_count_limits(E, k, M):
    # the most experts the boundary takes (1024: most of them get no slot and
    # the rest one or two, so nearly every tile holds a row or two), and every
    # token routed to all of its experts (top_k == E)
    H, I = 256, 256
    wg, wu, wd, x, ids, p = _moe_inputs(E, H, I, M, k, 23)
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I)
    assert bad == 0
    print(f"[moe limits] E={E} k={k} M={M}: {len(np.unique(ids))} experts used", flush=True)
    assert_parity(_moe_gpu(wg, wu, wd, E, H, I, x, ids, p, 0, 8), y_ref, f"moe E={E} top-{k} M={M}")


@pytest.mark.parametrize("M", [32768, 32769])
def test_moe_routing_paths_around_the_switch(M):
    # up to 65536 slots the routing runs in one workgroup, past it as three
    # grid-wide kernels: both sides of the switch against the oracle, with an
    # invalid id that is flagged and contributes nothing
    E, H, I, k = 16, 256, 256, 2
    wg, wu, wd, x, ids, p = _moe_inputs(E, H, I, M, k, 25)
    ids = ids.copy()
    ids[5, 1] = E + 3
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I)
    assert bad == 1
    b = max(0, int(np.ceil(np.log2(np.abs(y_ref).max() / 2 ** 13))))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    y = _moe_gpu(wg, wu, wd, E, H, I, x, ids, p, 0, b, dev_error=flag)
    assert int(flag.item()) == 1
    assert_parity(y, y_ref, f"moe routing, {M * k} slots")


def test_moe_top1_weight1_matches_dense():
    E, H, I, M = 4, 512, 512, 70
    wg, wu, wd, x, _, _ = _moe_inputs(E, H, I, M, 1, 22)
    ids = np.full((M, 1), 3, np.int32)
    p = np.ones((M, 1), np.float32)
    y_ref, h_ref = O.mlp(x, wg[3], wu[3], wd[3], H, I)
    a, b = shifts_for(y_ref, h_ref)
    ym = _moe_gpu(wg, wu, wd, E, H, I, x, ids, p, a, b)
    yd = prefill(wg[3], wu[3], wd[3], H, I, x, a, b)
    assert_parity(ym, y_ref, "moe top-1 vs oracle dense")
    assert_parity(ym, yd, "moe top-1 vs GPU dense")


def test_moe_repeat_calls_bit_identical():
    # tiles hold up to 80 rows; experts of 81-83 rows here are a full tile plus
    # a remainder of <= 16 rows, so they take 128-row chunks in both their
    # tiles, and the scatter places their rows in one tile or the other by
    # atomics; a row's arithmetic must not depend on its tile: repeated calls
    # give the same bits (the other experts are one tile of 192-row chunks)
    E, H, I, M, k = 16, 256, 512, 300, 4
    wg, wu, wd, x, ids, p = _moe_inputs(E, H, I, M, k, 26)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert any(c > 80 and c % 80 <= 16 for c in counts) and any(c % 80 > 16 for c in counts)
    y_ref, _ = O.moe(x, wg, wu, wd, ids, p, H, I)
    b = max(0, int(np.ceil(np.log2(np.abs(y_ref).max() / 2 ** 13))))
    ys = [_moe_gpu(wg, wu, wd, E, H, I, x, ids, p, 0, b) for _ in range(3)]
    assert_parity(ys[0], y_ref, "moe mixed chunkings")
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def test_moe_permuted_slots_same_output():
    E, H, I, M, k = 8, 256, 512, 50, 3
    wg, wu, wd, x, ids, p = _moe_inputs(E, H, I, M, k, 23)
    y_ref, _ = O.moe(x, wg, wu, wd, ids, p, H, I)
    y1 = _moe_gpu(wg, wu, wd, E, H, I, x, ids, p, 0, 10)
    y2 = _moe_gpu(wg, wu, wd, E, H, I, x, ids[:, ::-1].copy(), p[:, ::-1].copy(), 0, 10)
    assert_parity(y1, y_ref, "moe slots")
    assert_parity(y2, y_ref, "moe permuted slots")


def test_moe_invalid_ids_flag_and_contribute_nothing():
    E, H, I, M, k = 4, 256, 256, 30, 2
    wg, wu, wd, x, ids, p = _moe_inputs(E, H, I, M, k, 24)
    ids = ids.copy()
    ids[2, 0] = -5
    ids[9, 1] = 4
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    y = _moe_gpu(wg, wu, wd, E, H, I, x, ids, p, 0, 8, dev_error=flag)
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I)
    assert bad == 2
    assert int(flag.item()) == 1
    assert_parity(y, y_ref, "moe with invalid ids")


@pytest.mark.parametrize("M", [1, 3])
def test_moe_decode_sized_batches(M):
    # the E=64 top-8 2048 -> 768 experts with one or three tokens (MoE decode):
    # every tile then holds one to three rows
    w = S.WORKLOADS["moe_e64"]
    wg, wu, wd = S.expert_weights(w.seed, w.n_experts, w.hidden, w.inter)
    x = S.workload_x(w, M)
    ids, p = S.workload_routing(w, M)
    y = _moe_gpu(wg, wu, wd, w.n_experts, w.hidden, w.inter, x, ids, p, w.inter_shift, w.out_shift)
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, w.hidden, w.inter)
    assert bad == 0
    assert_parity(y, y_ref, f"moe E=64 top-8 M={M}")


def test_moe_workload_full():
    w = S.WORKLOADS["moe_e64"]
    wg, wu, wd = S.expert_weights(w.seed, w.n_experts, w.hidden, w.inter)
    x = S.workload_x(w)
    ids, p = S.workload_routing(w)
    y = _moe_gpu(wg, wu, wd, w.n_experts, w.hidden, w.inter, x, ids, p, w.inter_shift, w.out_shift)
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, w.hidden, w.inter)
    assert bad == 0
    assert_parity(y, y_ref, "moe E=64 top-8 M=512")
