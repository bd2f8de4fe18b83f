"""Structured parity probes on every path that runs at full size, and the
zero-centred weight recipe.

The uniform recipe's weights have a mean of about +1.1, so its outputs are
dominated by the mean and a slip in a kernel's sub-block or tile layout can
stay inside the tolerance.  These inputs cannot hide one:
  * x = 0 must give exactly y = 0;
  * one-hot x (token t selects one hidden column) reads single columns of
    W_gate and W_up;
  * W_up = 1 (every weight exactly 1.0) makes h = silu(W_gate x) * sum(x);
  * a W_down whose every row has exactly one non-zero sub-block (zero mins)
    makes each output read one 32-wide slice of the intermediate;
  * zero-centred Q4_K blocks (m_j = sc_j, dmin = 7.5 d) make y come from
    cancellation, which tests the fp16 operands of the -dmin*m term and the
    fp16 split-K partials where the uniform recipe does not.
Each probe runs on every unit the default plans use: the 64-token 16x16x32
prefill unit (up to 256 tokens), the 32x32x16 unit with 384-row chunks (257 to
511 tokens), the 128-token unit (from 512 tokens), the M = 1 row kernels, the 2 <= M <= 8 MFMA decode kernels and
the MoE's 80-token unit (an expert with more than 80 routed rows)."""
from __future__ import annotations

import zlib

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
    return S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, H, I), S.gen_x(rng, M, H, sd)


def _single_subblock_rows(wd, seed):
    """W_down with exactly one non-zero sub-block per row (dmin = 0, every
    other scale and min 0)."""
    rng = np.random.default_rng(seed)
    wd = wd.copy()
    rows, nb = wd.shape[0], wd.shape[1]
    wd[:, :, 2:4] = 0
    wd[:, :, 4:16] = 0
    for r in range(rows):
        b, j, sc = rng.integers(nb), rng.integers(8), rng.integers(1, 64)
        if j < 4:
            wd[r, b, 4 + j] = sc
        else:
            wd[r, b, 4 + j + 4] = sc & 15
            wd[r, b, 4 + j - 4] = (sc >> 4) << 6
    return wd


PROBES = ("zero_x", "one_hot_x", "unit_up", "single_subblock_down", "centred")


def _probe_inputs(probe, H, I, M, seed):
    wg, wu, wd, x = _rand_mlp(seed, H, I, M)
    if probe == "zero_x":
        x = np.zeros((M, H), np.float16)
    elif probe == "one_hot_x":
        x = np.zeros((M, H), np.float16)
        x[np.arange(M), (np.arange(M) * 37 + 5) % H] = 1.0
    elif probe == "unit_up":
        wu = B.unit_matrix(I, H)
    elif probe == "single_subblock_down":
        wd = _single_subblock_rows(wd, seed + 1)
    elif probe == "centred":
        rng = np.random.default_rng(seed + 2)
        wg, wu, wd = (S.gen_q4k_blob_centred(rng, I, H), S.gen_q4k_blob_centred(rng, I, H),
                      S.gen_q4k_blob_centred(rng, H, I))
    return wg, wu, wd, x


# (entry point, H, I, M): the unit each one reaches under the default plan
PATHS = {
    "prefill_unit_d": ("prefill", 512, 1536, 200),    # 64-token 16x16x32 unit, 4 tiles, ragged tail
    "prefill_unit_c": ("prefill", 512, 1536, 330),    # 32x32x16 unit, 384-row chunks
    "prefill_unit_e": ("prefill", 512, 1536, 600),    # 128-token unit, two 128-row passes per chunk
    "decode_rows_m1": ("decode", 1024, 2816, 1),      # row-streaming kernels
    "decode_rows_m1_w": ("decode", 4352, 1280, 1),    # two chunk slots per lane in the gate/up pass
    "decode_mfma_m4": ("decode", 1024, 2816, 4),      # 16x16x32 MFMA decode
    "decode_mfma_m3_w": ("decode", 4352, 1280, 3),    # a hidden width that is not a multiple of 4096
    "decode_mfma_m7": ("decode", 1024, 2816, 7),      # the eight-token kernels, one token column unused
    "decode_mfma_m8": ("decode", 4352, 1280, 8),      # all eight columns, two blocks per wave and pass
}


@pytest.mark.parametrize("probe", PROBES)
@pytest.mark.parametrize("path", list(PATHS))
def test_structured_probe(path, probe):
    fn, H, I, M = PATHS[path]
    wg, wu, wd, x = _probe_inputs(probe, H, I, M, seed=zlib.crc32(f"{path}/{probe}".encode()) % 10000)
    call = prefill if fn == "prefill" else decode
    if probe == "zero_x":
        y = call(wg, wu, wd, H, I, x, 0, 0)
        assert np.all(y == 0.0), f"{path}: x = 0 gave a non-zero output"
        return
    y_ref, h_ref = O.mlp(x, wg, wu, wd, H, I)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(call(wg, wu, wd, H, I, x, a, b), y_ref, f"{path} probe {probe}")


# ---------------------------------------------------------------------------
# the MoE unit: one expert with more than 80 routed rows
# ---------------------------------------------------------------------------
def _moe_call(wg, wu, wd, E, H, I, x, ids, p, a, b, flag=None):
    y = Z.zinc_moe_q4k_experts(dev(wg), dev(wu), dev(wd), E, H, I, dev(x), dev(ids), dev(p), a, b, dev_error=flag)
    return unscale(y, b)


@pytest.mark.parametrize("M", [200, 170])
@pytest.mark.parametrize("probe", PROBES)
def test_moe_probe_hot_expert(probe, M):
    # slot 0 of every token goes to expert 3 (M rows: tiles of 80 with a
    # remainder of 40 rows, 192-row chunks; or of 10 rows, which sends that
    # expert to 128-row chunks); slot 1 is random among the others.  The
    # probe is applied to expert 3's weights.
    E, H, I, k = 8, 512, 768, 2
    rng = np.random.default_rng(1000 + M)
    wg = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wd = np.stack([S.gen_q4k_blob(rng, H, I) for _ in range(E)])
    g3, u3, d3, x = _probe_inputs(probe, H, I, M, seed=77 + M)
    wg[3], wu[3], wd[3] = g3, u3, d3
    ids = np.empty((M, k), np.int32)
    ids[:, 0] = 3
    ids[:, 1] = rng.choice([0, 1, 2, 4, 5, 6, 7], size=M)
    p = np.stack([np.full(M, 0.75), np.full(M, 0.25)], axis=1).astype(np.float32)
    if probe == "zero_x":
        y = _moe_call(wg, wu, wd, E, H, I, x, ids, p, 0, 0)
        assert np.all(y == 0.0)
        return
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I)
    assert bad == 0
    b = max(0, int(np.ceil(np.log2(np.abs(y_ref).max() / 2 ** 13))))
    # the intermediate shift from every expert's largest |h| over these tokens
    hmax = max(float(np.abs(O.mlp(x, wg[e], wu[e], wd[e], H, I)[1]).max()) for e in range(E))
    a = max(0, int(np.ceil(np.log2(hmax / 2 ** 13)))) if hmax > 0 else 0
    assert_parity(_moe_call(wg, wu, wd, E, H, I, x, ids, p, a, b), y_ref, f"moe hot expert M={M} probe {probe}")


def test_moe_duplicate_ids_within_a_token_each_count():
    # the same expert twice in one token: both slots contribute, each with
    # its own mixing weight
    E, H, I, M, k = 6, 256, 512, 90, 4
    rng = np.random.default_rng(31)
    wg = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wd = np.stack([S.gen_q4k_blob(rng, H, I) for _ in range(E)])
    x = S.gen_x(rng, M, H)
    ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    ids[:, 1] = ids[:, 0]                   # every token repeats its first expert
    ids[::3, 3] = ids[::3, 0]               # a third of them three times
    p = rng.uniform(0.1, 1.0, size=(M, k)).astype(np.float32)
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I)
    assert bad == 0
    # against the oracle, and against the same call with the repeated slots merged
    merged_p = p.copy()
    merged_p[:, 0] += p[:, 1]
    merged_p[:, 1] = 0.0
    y_m, _ = O.moe(x, wg, wu, wd, ids, merged_p, H, I)
    assert O.within_tolerance(y_m, y_ref)
    b = max(0, int(np.ceil(np.log2(np.abs(y_ref).max() / 2 ** 13))))
    assert_parity(_moe_call(wg, wu, wd, E, H, I, x, ids, p, 0, b), y_ref, "moe duplicate ids")


def test_moe_skewed_routing_full_size():
    # the E = 64, top-8, M = 512 shape with most slots on a few experts:
    # slot 0 -> expert 0 for every token (512 rows: 6 full tiles and a
    # remainder of 32), slot 1 -> expert 1 for 490 tokens (a remainder of 10:
    # 128-row chunks), slot 2 -> expert 2 for 100 tokens, the rest uniform
    # over experts 3..63 without repeats
    w = S.WORKLOADS["moe_e64"]
    E, H, I, M, k = w.n_experts, w.hidden, w.inter, w.M, w.top_k
    wg, wu, wd = S.expert_weights(w.seed, E, H, I)
    x = S.workload_x(w)
    rng = np.random.default_rng(4242)
    ids = np.empty((M, k), np.int32)
    for t in range(M):
        rest = rng.choice(np.arange(3, E), size=k, replace=False)
        ids[t] = rest
        ids[t, 0] = 0
        if t < 490:
            ids[t, 1] = 1
        if t < 100:
            ids[t, 2] = 2
    p = S.gen_routing(rng, M, E, k)[1]
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts[0] == 512 and counts[1] == 490 and counts[2] == 100
    y_ref, bad = O.moe(x, wg, wu, wd, ids, p, H, I)
    assert bad == 0
    y = _moe_call(wg, wu, wd, E, H, I, x, ids, p, w.inter_shift, w.out_shift)
    assert_parity(y, y_ref, "moe E=64 skewed routing")


# ---------------------------------------------------------------------------
# zero-centred weights at the full 4096/11008 shape
# ---------------------------------------------------------------------------
def _centred_layer(layer=0):
    w = S.WORKLOADS["prefill_m256"]
    return S.centred_layer_weights(w.seed, layer, w.hidden, w.inter)


def test_centred_prefill_m256_full():
    w = S.WORKLOADS["prefill_m256"]
    wg, wu, wd = _centred_layer()
    x = S.workload_x(w)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(prefill(wg, wu, wd, w.hidden, w.inter, x, a, b), y_ref, "centred prefill 4096/11008 M=256")


def test_centred_prefill_m2048_sampled_tokens():
    w = S.WORKLOADS["prefill_m2048"]
    wg, wu, wd = _centred_layer(1)
    x = S.workload_x(w)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 2047], np.random.default_rng(3).choice(w.M, 59, replace=False)]))
    y_ref, h_ref = O.mlp(x[rows], wg, wu, wd, w.hidden, w.inter)
    a, b = shifts_for(y_ref, h_ref)
    a, b = a + 1, b + 1   # headroom for the tokens not sampled
    y = prefill(wg, wu, wd, w.hidden, w.inter, x, a, b)
    assert_parity(y[rows], y_ref, f"centred prefill M=2048, {len(rows)} sampled tokens")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_centred_decode_full_shape(M):
    w = S.WORKLOADS["decode_m4"]
    wg, wu, wd = _centred_layer(2)
    x = S.workload_x(w)[:M] if M <= 4 else S.gen_x(np.random.default_rng(990), M, w.hidden)
    y_ref, h_ref = O.mlp(x, wg, wu, wd, w.hidden, w.inter)
    a, b = shifts_for(y_ref, h_ref)
    assert_parity(decode(wg, wu, wd, w.hidden, w.inter, x, a, b), y_ref, f"centred decode 4096/11008 M={M}")


def test_centred_moe_full_size():
    w = S.WORKLOADS["moe_e64"]
    rng = np.random.default_rng([w.seed, 700])
    E, H, I = w.n_experts, w.hidden, w.inter
    wg = np.stack([S.gen_q4k_blob_centred(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob_centred(rng, I, H) for _ in range(E)])
    wd = np.stack([S.gen_q4k_blob_centred(rng, H, I) for _ in range(E)])
    x = S.workload_x(w)
    ids, p = S.workload_routing(w)
    y_ref, _ = O.moe(x, wg, wu, wd, ids, p, H, I)
    b = max(0, int(np.ceil(np.log2(np.abs(y_ref).max() / 2 ** 13))))
    assert_parity(_moe_call(wg, wu, wd, E, H, I, x, ids, p, 0, b), y_ref, "centred moe E=64 top-8 M=512")


# ---------------------------------------------------------------------------
# every layer of the 32-layer decode workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layer", range(32))
def test_decode_workloads_every_layer(layer):
    w = S.WORKLOADS["decode_m4"]
    assert S.WORKLOADS["decode_m1"].seed == w.seed
    wg, wu, wd = S.layer_weights(w.seed, layer, w.hidden, w.inter)
    x4 = S.workload_x(w)
    x1 = S.workload_x(S.WORKLOADS["decode_m1"])
    assert np.array_equal(x1, x4[:1])
    y_ref, _ = O.mlp(x4, wg, wu, wd, w.hidden, w.inter)   # tokens are independent rows
    gw = (dev(wg), dev(wu), dev(wd))
    for M in (1, 4):
        y = Z.zinc_mlp_q4k_decode(*gw, w.hidden, w.inter, dev(x4[:M]), w.inter_shift, w.out_shift)
        assert_parity(unscale(y, w.out_shift), y_ref[:M], f"decode layer {layer} M={M}")
