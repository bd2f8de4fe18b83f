"""Pins for the CPU oracle: each test checks it against something other than
itself -- literal hand-built blocks, a bit-level field reader, exact rational
arithmetic, library routines, brute-force loops, closed-form probes and exact
invariants.  CPU only."""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle as O
import q4k_synth as S
from tests import q4k_blocks as B



def _w(blk):
    """Decoded float64 weights of one block."""
    return O.q4k_dequant(blk.reshape(1, 1, 144), 1, 256)[0]


def _per_subblock(values):
    """256 weights from 8 per-sub-block constants."""
    return np.repeat(np.asarray(values, dtype=np.float64), 32)


# ---------------------------------------------------------------------------
# Q4_K decode: literal hand-built blocks
# ---------------------------------------------------------------------------
def test_zero_block_is_all_positive_zero():
    w = _w(B.block())
    assert np.all(w == 0.0)
    assert not np.any(np.signbit(w.astype(np.float32)))


def test_unit_scales_with_quants_i_mod_16():
    # Q[32c + l] carries l % 16 in both nibbles, so weight i holds i % 16.
    Q = [(l % 16) | ((l % 16) << 4) for c in range(4) for l in range(32)]
    w = _w(B.block(B.F16_ONE, 0, B.S_UNIT_SCALES, Q))
    assert np.array_equal(w, np.arange(256) % 16)


# With d = 1, dmin = 0 and every quant 1, setting scale byte S[k] = 0xFF alone
# gives these per-sub-block weights (worked out by hand from the field table:
# S[0..3] carry sc_0..3 in bits 0-5 and the top two bits of sc_4..7 in bits 6-7;
# S[4..7] carry only mins; S[8..11] carry the low nibble of sc_4..7).
SCALE_WALK = {
    0: [63, 0, 0, 0, 48, 0, 0, 0],
    1: [0, 63, 0, 0, 0, 48, 0, 0],
    2: [0, 0, 63, 0, 0, 0, 48, 0],
    3: [0, 0, 0, 63, 0, 0, 0, 48],
    4: [0] * 8, 5: [0] * 8, 6: [0] * 8, 7: [0] * 8,
    8: [0, 0, 0, 0, 15, 0, 0, 0],
    9: [0, 0, 0, 0, 0, 15, 0, 0],
    10: [0, 0, 0, 0, 0, 0, 15, 0],
    11: [0, 0, 0, 0, 0, 0, 0, 15],
}

# With d = 0, dmin = 1: S[4..7] carry m_0..3 in bits 0-5 and the top two bits
# of m_4..7 in bits 6-7; S[8..11] carry the low nibble of m_4..7 in bits 4-7.
MIN_WALK = {
    0: [0] * 8, 1: [0] * 8, 2: [0] * 8, 3: [0] * 8,
    4: [-63, 0, 0, 0, -48, 0, 0, 0],
    5: [0, -63, 0, 0, 0, -48, 0, 0],
    6: [0, 0, -63, 0, 0, 0, -48, 0],
    7: [0, 0, 0, -63, 0, 0, 0, -48],
    8: [0, 0, 0, 0, -15, 0, 0, 0],
    9: [0, 0, 0, 0, 0, -15, 0, 0],
    10: [0, 0, 0, 0, 0, 0, -15, 0],
    11: [0, 0, 0, 0, 0, 0, 0, -15],
}


@pytest.mark.parametrize("k", range(12))
def test_scale_byte_walk(k):
    Sb = [0] * 12
    Sb[k] = 0xFF
    w = _w(B.block(B.F16_ONE, 0, Sb, [0x11] * 128))
    assert np.array_equal(w, _per_subblock(SCALE_WALK[k]))


@pytest.mark.parametrize("k", range(12))
def test_min_byte_walk(k):
    Sb = [0] * 12
    Sb[k] = 0xFF
    w = _w(B.block(0, B.F16_ONE, Sb, [0x11] * 128))
    assert np.array_equal(w, _per_subblock(MIN_WALK[k]))


def test_min_j_gives_minus_j():
    # m_j = j: S[4..7] = 0,1,2,3 and the high nibbles of S[8..11] = 4..7.
    Sb = [0, 0, 0, 0, 0, 1, 2, 3, 0x40, 0x50, 0x60, 0x70]
    w = _w(B.block(0, B.F16_ONE, Sb, [0x55] * 128))
    assert np.array_equal(w, _per_subblock([0, -1, -2, -3, -4, -5, -6, -7]))


# Positions of the low and high nibbles of the 128 quant bytes, in byte order:
# bytes 0-31 -> weights 0-31 (low) and 32-63 (high); bytes 32-63 -> 64-95 and
# 96-127; bytes 64-95 -> 128-159 and 160-191; bytes 96-127 -> 192-223, 224-255.
LOW_POS = list(range(0, 32)) + list(range(64, 96)) + list(range(128, 160)) + list(range(192, 224))
HIGH_POS = list(range(32, 64)) + list(range(96, 128)) + list(range(160, 192)) + list(range(224, 256))


def test_single_nibble_walk_is_a_permutation():
    seen = []
    for byte in range(128):
        for nib, table in ((0x01, LOW_POS), (0x10, HIGH_POS)):
            Q = [0] * 128
            Q[byte] = nib
            w = _w(B.block(B.F16_ONE, 0, B.S_UNIT_SCALES, Q))
            nz = np.flatnonzero(w)
            assert nz.tolist() == [table[byte]] and w[nz[0]] == 1.0
            seen.append(int(nz[0]))
    assert sorted(seen) == list(range(256))


def test_fp16_header_fields_literal():
    # d = 0.5, dmin = 2: w = 0.5*1*q - 2*0 on unit scales
    w = _w(B.block(B.F16_HALF, B.F16_TWO, B.S_UNIT_SCALES, [0x33] * 128))
    assert np.all(w == 1.5)
    # negative d is decoded literally
    w = _w(B.block(B.F16_NEG_ONE, 0, B.S_UNIT_SCALES, [0x22] * 128))
    assert np.all(w == -2.0)
    # d and dmin are not swapped: d = 2, dmin = 0.5 with unit mins (m_j = 1)
    Sb = [1, 1, 1, 1, 1, 1, 1, 1, 0x11, 0x11, 0x11, 0x11]
    w = _w(B.block(B.F16_TWO, B.F16_HALF, Sb, [0x44] * 128))
    assert np.all(w == 2.0 * 4 - 0.5)


# ---------------------------------------------------------------------------
# Q4_K decode: brute-force bit reader and exact arithmetic on random blocks
# ---------------------------------------------------------------------------
def _bit(blk, pos):
    return (int(blk[pos // 8]) >> (pos % 8)) & 1


def _field(blk, positions):
    return sum(_bit(blk, p) << t for t, p in enumerate(positions))


def _field_positions():
    """Absolute LSB-first bit positions of every field inside a block."""
    pos = {}
    for j in range(4):
        pos[("sc", j)] = [8 * (4 + j) + t for t in range(6)]
        pos[("m", j)] = [8 * (8 + j) + t for t in range(6)]
    for j in range(4, 8):
        pos[("sc", j)] = [8 * (4 + j + 4) + t for t in range(4)] + [8 * (4 + j - 4) + 6, 8 * (4 + j - 4) + 7]
        pos[("m", j)] = [8 * (4 + j + 4) + 4 + t for t in range(4)] + [8 * (4 + j) + 6, 8 * (4 + j) + 7]
    for c in range(4):
        for l in range(32):
            byte = 16 + 32 * c + l
            pos[("q", 64 * c + l)] = [8 * byte + t for t in range(4)]
            pos[("q", 64 * c + 32 + l)] = [8 * byte + 4 + t for t in range(4)]
    return pos


def test_bit_reader_partitions_the_block():
    # sixteen 6-bit fields + 256 nibbles cover bits 32..1151 exactly once
    all_bits = [p for v in _field_positions().values() for p in v]
    assert sorted(all_bits) == list(range(32, 144 * 8))


def test_fields_match_bit_level_reader():
    rng = np.random.default_rng(12345)
    blob = S.gen_q4k_blob(rng, 40, 256 * 5)
    d, dmin, sc, m, q = O.q4k_fields(blob)
    pos = _field_positions()
    for r in range(40):
        for b in range(5):
            blk = blob[r, b]
            for j in range(8):
                assert sc[r, b, j] == _field(blk, pos[("sc", j)])
                assert m[r, b, j] == _field(blk, pos[("m", j)])
            for i in range(256):
                assert q[r, b, i] == _field(blk, pos[("q", i)])
            assert d[r, b] == float(np.frombuffer(bytes(blk[0:2]), dtype="<f2")[0])
            assert dmin[r, b] == float(np.frombuffer(bytes(blk[2:4]), dtype="<f2")[0])


def test_dequant_is_exact_rational_value():
    rng = np.random.default_rng(7)
    blob = S.gen_q4k_blob(rng, 3, 512)
    W = O.q4k_dequant(blob, 3, 512)
    pos = _field_positions()
    for r in range(3):
        for b in range(2):
            blk = blob[r, b]
            dF = Fraction(float(np.frombuffer(bytes(blk[0:2]), dtype="<f2")[0]))
            mF = Fraction(float(np.frombuffer(bytes(blk[2:4]), dtype="<f2")[0]))
            for i in range(256):
                j = i // 32
                exact = dF * _field(blk, pos[("sc", j)]) * _field(blk, pos[("q", i)]) \
                    - mF * _field(blk, pos[("m", j)])
                assert Fraction(W[r, 256 * b + i]) == exact


def test_fp32_dequant_is_round_to_nearest_even_of_exact():
    rng = np.random.default_rng(8)
    blob = S.gen_q4k_blob(rng, 16, 512)
    W64 = O.q4k_dequant(blob, 16, 512)
    W32 = O.q4k_dequant_f32(blob, 16, 512)
    # RNE: |w32 - w| <= half an ulp of w32, and ties go to the even mantissa
    ulp = np.spacing(np.abs(W32).astype(np.float32)).astype(np.float64)
    diff = np.abs(W32.astype(np.float64) - W64)
    assert np.all(diff <= ulp / 2)


# ---------------------------------------------------------------------------
# silu
# ---------------------------------------------------------------------------
def test_silu_identities_and_library():
    z = np.linspace(-30, 30, 6001)
    s = O.silu(z)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - O.silu(-z), z, rtol=0, atol=1e-12)       # silu(z) - silu(-z) = z
    assert np.allclose(s, z * expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-20)
    big_neg = O.silu(np.array([-800.0]))[0]
    assert big_neg == 0.0 and not math.isnan(big_neg)


# ---------------------------------------------------------------------------
# MLP
# ---------------------------------------------------------------------------
def _tiny_mlp_inputs(seed=3, H=256, I=256, M=2):
    rng = np.random.default_rng(seed)
    wg = S.gen_q4k_blob(rng, I, H)
    wu = S.gen_q4k_blob(rng, I, H)
    wd = S.gen_q4k_blob(rng, H, I)
    x = S.gen_x(rng, M, H)
    return x, wg, wu, wd


def test_mlp_matches_brute_force_loops():
    H, I, M = 256, 256, 2
    x, wg, wu, wd = _tiny_mlp_inputs(H=H, I=I, M=M)
    Wg, Wu, Wd = (O.q4k_dequant(wg, I, H), O.q4k_dequant(wu, I, H), O.q4k_dequant(wd, H, I))
    y, h = O.mlp(x, wg, wu, wd, H, I)
    xs = x.astype(np.float64).tolist()
    for t in range(M):
        hh = []
        for j in range(I):
            g = sum(Wg[j][k] * xs[t][k] for k in range(H))
            u = sum(Wu[j][k] * xs[t][k] for k in range(H))
            hh.append(g / (1.0 + math.exp(-g)) * u if g > -700 else -0.0)
        for n in range(H):
            yy = sum(Wd[n][j] * hh[j] for j in range(I))
            assert y[t, n] == pytest.approx(yy, rel=1e-11, abs=1e-9 * abs(yy) + 1e-300)
        assert np.allclose(h[t], hh, rtol=1e-11)


def _bitlevel_dequant(blob):
    """A second Q4_K decoder, written from the bit positions of every field
    (``_field_positions``) instead of the oracle's byte arithmetic."""
    rows, nb, _ = blob.shape
    bits = np.unpackbits(blob.reshape(rows, nb, 144), axis=2, bitorder="little").astype(np.int64)
    pos = _field_positions()

    def field(key):
        return sum(bits[:, :, p] << t for t, p in enumerate(pos[key]))

    d = blob[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)
    dmin = blob[:, :, 2:4].copy().view("<f2")[:, :, 0].astype(np.float64)
    W = np.empty((rows, nb, 256))
    for i in range(256):
        j = i // 32
        W[:, :, i] = d * field(("sc", j)) * field(("q", i)) - dmin * field(("m", j))
    return W.reshape(rows, nb * 256)


def test_mlp_matches_unfused_four_step_reference():
    # the staged dataflow of "The MLP is two trips up to a wider width": gate GEMM,
    # up GEMM, SwiGLU elementwise, down GEMM, every intermediate materialised, on
    # weights decoded by the bit-level reader and with the library sigmoid
    H, I, M = 512, 768, 16
    x, wg, wu, wd = _tiny_mlp_inputs(seed=21, H=H, I=I, M=M)
    X = x.astype(np.float64)
    G = X @ _bitlevel_dequant(wg).T
    U = X @ _bitlevel_dequant(wu).T
    Hm = G * expit(G) * U
    Y = Hm @ _bitlevel_dequant(wd).T
    y, h = O.mlp(x, wg, wu, wd, H, I)
    assert np.sum(np.abs(h - Hm)) / np.sum(np.abs(Hm)) <= 1e-12
    assert np.sum(np.abs(y - Y)) / np.sum(np.abs(Y)) <= 1e-12


def test_one_hot_x_selects_weight_columns():
    H, I = 512, 256
    x, wg, wu, wd = _tiny_mlp_inputs(H=H, I=I, M=1)
    k = 300
    x = np.zeros((1, H), dtype=np.float16)
    x[0, k] = 1.0
    _, h = O.mlp(x, wg, wu, wd, H, I)
    g_col = O.q4k_dequant(wg, I, H)[:, k]         # column k of W_gate (not row k)
    u_col = O.q4k_dequant(wu, I, H)[:, k]
    assert np.array_equal(h[0], g_col / (1.0 + np.exp(-g_col)) * u_col)


def test_gate_branch_is_the_one_through_silu():
    H, I = 256, 256
    x, wg, wu, wd = _tiny_mlp_inputs(H=H, I=I, M=1)
    x = np.zeros((1, H), dtype=np.float16)
    x[0, 17] = 1.0
    ones = B.unit_matrix(I, H)
    # W_up = 1 everywhere: u = 1, so h = silu(g) with g = column 17 of W_gate
    _, h = O.mlp(x, wg, ones, wd, H, I)
    g = O.q4k_dequant(wg, I, H)[:, 17]
    assert np.allclose(h[0], g * expit(g), rtol=1e-14)
    # W_gate = 1 everywhere: g = 1, so h = silu(1) * u
    _, h = O.mlp(x, ones, wu, wd, H, I)
    u = O.q4k_dequant(wu, I, H)[:, 17]
    assert np.allclose(h[0], expit(1.0) * u, rtol=1e-14)


def test_zero_input_gives_exact_zero():
    x, wg, wu, wd = _tiny_mlp_inputs()
    y, h = O.mlp(np.zeros_like(x), wg, wu, wd, 256, 256)
    assert np.all(y == 0.0) and np.all(h == 0.0)


def test_doubling_down_scales_doubles_output_exactly():
    x, wg, wu, wd = _tiny_mlp_inputs()
    y1, _ = O.mlp(x, wg, wu, wd, 256, 256)
    wd2 = B.scaled_blob(wd, B.double_fp16_bits)
    y2, _ = O.mlp(x, wg, wu, wd2, 256, 256)
    assert np.array_equal(y2, 2.0 * y1)


def test_hidden_block_permutation_invariance():
    H, I = 1024, 256
    x, wg, wu, wd = _tiny_mlp_inputs(H=H, I=I, M=3)
    y1, _ = O.mlp(x, wg, wu, wd, H, I)
    perm = np.array([2, 0, 3, 1])          # permute the four 256-column blocks of the hidden axis
    xp = x.reshape(3, 4, 256)[:, perm].reshape(3, H)
    y2, _ = O.mlp(xp, wg[:, perm], wu[:, perm], wd, H, I)
    # the down projection's outputs are hidden columns too; they are not permuted
    assert np.allclose(y1, y2, rtol=1e-11, atol=1e-9 * np.abs(y1).max())


# ---------------------------------------------------------------------------
# MoE
# ---------------------------------------------------------------------------
def _tiny_moe(E=4, H=256, I=256, M=5, k=2, seed=11):
    rng = np.random.default_rng(seed)
    wg = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wd = np.stack([S.gen_q4k_blob(rng, H, I) for _ in range(E)])
    x = S.gen_x(rng, M, H)
    ids, p = S.gen_routing(rng, M, E, k)
    return x, wg, wu, wd, ids, p


def test_moe_top1_weight1_is_dense():
    x, wg, wu, wd, ids, p = _tiny_moe()
    ids1 = np.full((x.shape[0], 1), 2, dtype=np.int32)
    y, bad = O.moe(x, wg, wu, wd, ids1, np.ones((x.shape[0], 1), np.float32), 256, 256)
    yd, _ = O.mlp(x, wg[2], wu[2], wd[2], 256, 256)
    assert bad == 0 and np.array_equal(y, yd)


def test_moe_slot_permutation_invariance():
    x, wg, wu, wd, ids, p = _tiny_moe()
    y1, _ = O.moe(x, wg, wu, wd, ids, p, 256, 256)
    y2, _ = O.moe(x, wg, wu, wd, ids[:, ::-1].copy(), p[:, ::-1].copy(), 256, 256)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-12 * np.abs(y1).max())


def test_moe_identical_experts_reduce_to_dense():
    x, wg, wu, wd, ids, p = _tiny_moe()
    E = wg.shape[0]
    same = lambda a: np.stack([a[0]] * E)
    y, _ = O.moe(x, same(wg), same(wu), same(wd), ids, p, 256, 256)
    yd, _ = O.mlp(x, wg[0], wu[0], wd[0], 256, 256)
    scale = p.astype(np.float64).sum(axis=1, keepdims=True)     # = 1 up to fp32 rounding
    assert np.allclose(y, scale * yd, rtol=1e-12, atol=1e-12 * np.abs(yd).max())


def test_moe_out_of_range_ids_contribute_nothing():
    x, wg, wu, wd, ids, p = _tiny_moe()
    bad_ids = ids.copy()
    bad_ids[1, 0] = -1
    bad_ids[3, 1] = 99
    y, bad = O.moe(x, wg, wu, wd, bad_ids, p, 256, 256)
    keep = p.copy()
    keep[1, 0] = 0
    keep[3, 1] = 0
    y2, _ = O.moe(x, wg, wu, wd, np.where(bad_ids < 0, 0, np.where(bad_ids > 3, 0, bad_ids)), keep, 256, 256)
    assert bad == 2 and np.allclose(y, y2, rtol=1e-13, atol=1e-12 * np.abs(y).max())


# ---------------------------------------------------------------------------
# Q5_K and Q5_1 blocks (the experts' other down-projection formats)
# ---------------------------------------------------------------------------
def _q5k_block(d_bits=0x3C00, dmin_bits=0, S=None, QH=None, Q=None):
    b = np.zeros(176, dtype=np.uint8)
    b[0:2] = [d_bits & 0xFF, d_bits >> 8]
    b[2:4] = [dmin_bits & 0xFF, dmin_bits >> 8]
    b[4:16] = B.S_UNIT_SCALES if S is None else S
    if QH is not None:
        b[16:48] = QH
    if Q is not None:
        b[48:176] = Q
    return b


def _q5_1_block(d_bits=0x3C00, m_bits=0, qh=0, Q=None):
    b = np.zeros(24, dtype=np.uint8)
    b[0:2] = [d_bits & 0xFF, d_bits >> 8]
    b[2:4] = [m_bits & 0xFF, m_bits >> 8]
    b[4:8] = [(qh >> (8 * k)) & 0xFF for k in range(4)]
    if Q is not None:
        b[8:24] = Q
    return b


def test_q5k_unit_scales_closed_forms():
    # quants 0x21 everywhere: low nibble 1, high nibble 2; no fifth bits
    w = O.q5k_dequant(_q5k_block(Q=[0x21] * 128), 1, 256)[0]
    assert np.array_equal(w, np.where((np.arange(256) % 64) < 32, 1.0, 2.0))
    # every fifth bit set: +16 on every weight
    w = O.q5k_dequant(_q5k_block(QH=[0xFF] * 32, Q=[0x21] * 128), 1, 256)[0]
    assert np.array_equal(w, np.where((np.arange(256) % 64) < 32, 17.0, 18.0))


@pytest.mark.parametrize("bit", range(8))
def test_q5k_fifth_bit_walk(bit):
    """Bit b of QH[l] is the fifth bit of weight 64*(b//2) + 32*(b%2) + l only
    (the inverse of the field formula, walked bit by bit)."""
    for l in (0, 7, 31):
        QH = np.zeros(32, dtype=np.uint8)
        QH[l] = 1 << bit
        w = O.q5k_dequant(_q5k_block(QH=QH), 1, 256)[0]
        expect = np.zeros(256)
        expect[64 * (bit // 2) + 32 * (bit % 2) + l] = 16.0
        assert np.array_equal(w, expect)


def test_q5k_scales_and_mins_follow_q4k_packing():
    rng = np.random.default_rng(91)
    blob = S.gen_q5k_blob(rng, 3, 512)
    # the same header and quant nibbles in a Q4_K block decode to the Q5_K
    # weights minus 16*d*sc on the weights whose fifth bit is set
    q4 = np.concatenate([blob[..., :16], blob[..., 48:]], axis=-1)
    w4 = O.q4k_dequant(q4, 3, 512).reshape(3, 2, 256)
    w5 = O.q5k_dequant(blob, 3, 512).reshape(3, 2, 256)
    d, dmin, sc, m, q = O.q5k_fields(blob)
    sub = np.arange(256) // 32
    assert np.array_equal(w5 - w4, d[..., None] * sc[..., sub] * 16.0 * (q >> 4))


def test_q5_1_closed_forms():
    # d = 1, m = 0: low nibbles 1 (weights 0..15), high nibbles 2 (16..31)
    w = O.q5_1_dequant(_q5_1_block(Q=[0x21] * 16), 1, 32)[0]
    assert np.array_equal(w, np.r_[np.ones(16), 2 * np.ones(16)])
    # m = -1 adds -1; d = 0.5 halves
    w = O.q5_1_dequant(_q5_1_block(d_bits=0x3800, m_bits=0xBC00, Q=[0x21] * 16), 1, 32)[0]
    assert np.array_equal(w, np.r_[-0.5 * np.ones(16), np.zeros(16)])
    # each bit of QH is one weight's fifth bit
    for j in (0, 5, 15, 16, 31):
        w = O.q5_1_dequant(_q5_1_block(qh=1 << j), 1, 32)[0]
        expect = np.zeros(32)
        expect[j] = 16.0
        assert np.array_equal(w, expect)


def test_q5_1_matrix_layout_and_brute_force():
    rng = np.random.default_rng(92)
    blob = S.gen_q5_1_blob(rng, 2, 64)
    w = O.q5_1_dequant(blob, 2, 64)
    for r in range(2):
        for col in range(64):
            b = blob[r, col // 32]
            i = col % 32
            d = float(np.frombuffer(b[0:2].tobytes(), np.float16)[0])
            m = float(np.frombuffer(b[2:4].tobytes(), np.float16)[0])
            qh = int.from_bytes(b[4:8].tobytes(), "little")
            nib = (b[8 + i % 16] >> (4 if i >= 16 else 0)) & 15
            assert w[r, col] == d * (nib + 16 * ((qh >> i) & 1)) + m


@pytest.mark.parametrize("fmt", ["q5_k", "q5_1"])
def test_q5_float64_weights_are_exact(fmt):
    """The float64 weights equal the exact rational values of the fields, so
    rounding them once to fp32 gives the unique fp32 weight."""
    rng = np.random.default_rng(93)
    blob = S.gen_down_blob(rng, fmt, 4, 512)
    w = O.DOWN_DECODERS[fmt](blob, 4, 512)
    F = lambda v: Fraction(float(v))
    if fmt == "q5_k":
        d, dmin, sc, m, q = O.q5k_fields(blob)
        for r, b, i in [(0, 0, 0), (1, 1, 77), (3, 0, 255), (2, 1, 130)]:
            j = i // 32
            exact = F(d[r, b]) * int(sc[r, b, j]) * int(q[r, b, i]) - F(dmin[r, b]) * int(m[r, b, j])
            assert Fraction(float(w[r, 256 * b + i])) == exact
    else:
        d, mm, q = O.q5_1_fields(blob)
        for r, b, i in [(0, 0, 0), (1, 7, 19), (3, 15, 31), (2, 3, 16)]:
            exact = F(d[r, b]) * int(q[r, b, i]) + F(mm[r, b])
            assert Fraction(float(w[r, 32 * b + i])) == exact


def test_moe_down_formats_reduce_to_dense():
    E, H, I, M = 3, 256, 256, 5
    rng = np.random.default_rng(94)
    wg = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    wu = np.stack([S.gen_q4k_blob(rng, I, H) for _ in range(E)])
    x = rng.standard_normal((M, H))
    for fmt in ("q5_k", "q5_1"):
        wd = np.stack([S.gen_down_blob(rng, fmt, H, I) for _ in range(E)])
        ids = np.full((M, 1), 2, np.int32)
        y, _ = O.moe(x, wg, wu, wd, ids, np.ones((M, 1), np.float32), H, I, fmt)
        Wd = O.DOWN_DECODERS[fmt](wd[2], H, I)
        g = x @ O.q4k_dequant(wg[2], I, H).T
        u = x @ O.q4k_dequant(wu[2], I, H).T
        assert np.allclose(y, (O.silu(g) * u) @ Wd.T, rtol=1e-12, atol=1e-9)


# ---------------------------------------------------------------------------
# Pre-MLP RMS norm and the residual block
# ---------------------------------------------------------------------------
def test_rms_norm_matches_torch():
    import torch
    rng = np.random.default_rng(81)
    x = rng.standard_normal((7, 512)) * 3
    g = rng.uniform(0.5, 1.5, 512)
    for eps in (0.0, 1e-6, 1e-2):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(g), eps).numpy()
        assert np.allclose(O.rms_norm(x, g, eps), ref, rtol=1e-12, atol=0)


def test_rms_norm_closed_forms():
    # a row of +-c has mean square c^2: entries become +-c / sqrt(c^2 + eps)
    c, eps = 3.0, 0.5
    x = np.array([[c, -c, c, c]])
    assert np.allclose(O.rms_norm(x, np.ones(4), eps), x / math.sqrt(c * c + eps), rtol=1e-15)
    # with eps = 0 the result is scale invariant and has unit mean square
    rng = np.random.default_rng(82)
    x = rng.standard_normal((5, 64))
    xn = O.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.mean(xn * xn, axis=1), 1.0, rtol=1e-13)
    assert np.allclose(O.rms_norm(x * 7.5, np.ones(64), 0.0), xn, rtol=1e-13)
    # gamma multiplies column-wise
    g = np.arange(1, 65, dtype=np.float64)
    assert np.allclose(O.rms_norm(x, g, 0.0), xn * g, rtol=1e-13)


def test_mlp_block_reductions():
    H, I, M = 256, 512, 6
    rng = np.random.default_rng(83)
    wg, wu, wd = S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, I, H), S.gen_q4k_blob(rng, H, I)
    x = rng.standard_normal((M, H))
    g = rng.uniform(0.5, 1.5, H)
    # zero scale: the residual alone, exactly
    y0, _ = O.mlp_block(x, g, 1e-5, 0.0, wg, wu, wd, H, I)
    assert np.array_equal(y0, x)
    # zero down weights: the MLP contributes exactly zero
    wd0 = np.zeros((H, I // 256, 144), dtype=np.uint8)   # d = dmin = 0: every weight is zero
    yz, _ = O.mlp_block(x, g, 1e-5, 2.0, wg, wu, wd0, H, I)
    assert np.array_equal(yz, x)
    # the MLP part is linear in the scale and is the MLP of the normalised rows
    y1, xn = O.mlp_block(x, g, 1e-5, 1.0, wg, wu, wd, H, I)
    y3, _ = O.mlp_block(x, g, 1e-5, 3.0, wg, wu, wd, H, I)
    assert np.allclose(y3 - x, 3.0 * (y1 - x), rtol=1e-12, atol=1e-9)
    # the norm's output does not depend on the residual's scale (eps = 0)
    y2, xn2 = O.mlp_block(2.0 * x, g, 0.0, 1.0, wg, wu, wd, H, I)
    assert np.allclose(xn2, O.rms_norm(x, g, 0.0), rtol=1e-13)


# ---------------------------------------------------------------------------
# Router: top-k selection and the softmax of the chosen logits
# ---------------------------------------------------------------------------
def test_router_matches_brute_force_subset_search():
    """For distinct logits the chosen set is the k-subset with the largest sum
    (found by enumerating every subset), listed in decreasing logit order."""
    import itertools
    rng = np.random.default_rng(71)
    for _ in range(60):
        E = int(rng.integers(1, 8))
        k = int(rng.integers(1, E + 1))
        row = rng.permutation(E).astype(np.float32) + rng.standard_normal(E).astype(np.float32) * 0.1
        ids, p = O.route_topk(row[None, :], k)
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(float(row[j]) for j in c))
        assert sorted(ids[0].tolist()) == sorted(best)
        vals = [float(row[j]) for j in ids[0]]
        assert all(a > b for a, b in zip(vals, vals[1:]))
        assert abs(p[0].sum() - 1.0) < 1e-12


def test_router_ties_go_to_the_lower_index():
    ids, p = O.route_topk(np.zeros((2, 10), dtype=np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2
    assert np.all(p == 0.25)
    row = np.array([[1.0, 3.0, 2.0, 3.0, 1.0, 3.0]], dtype=np.float32)
    ids, _ = O.route_topk(row, 5)
    assert ids[0].tolist() == [1, 3, 5, 2, 0]


def test_router_top1_is_first_argmax_with_weight_one():
    rng = np.random.default_rng(72)
    L = rng.integers(-3, 4, size=(50, 12)).astype(np.float32)   # many ties
    ids, p = O.route_topk(L, 1)
    assert np.array_equal(ids[:, 0], np.argmax(L, axis=1))
    assert np.all(p == 1.0)


def test_router_weights_match_library_softmax():
    from scipy.special import softmax
    rng = np.random.default_rng(73)
    L = (rng.standard_normal((40, 64)) * 3).astype(np.float32)
    ids, p = O.route_topk(L, 8)
    for t in range(40):
        chosen = L[t, ids[t]].astype(np.float64)
        assert np.allclose(p[t], softmax(chosen), rtol=1e-13, atol=0)
        # the full softmax over all experts, renormalised over the chosen ones
        full = softmax(L[t].astype(np.float64))[ids[t]]
        assert np.allclose(p[t], full / full.sum(), rtol=1e-12, atol=0)


def test_router_shift_invariance_and_ratio():
    rng = np.random.default_rng(74)
    # logits on a 2^-10 grid below 8 in magnitude, so adding 16 is exact in fp32
    L = (np.round(np.clip(rng.standard_normal((20, 32)), -7, 7) * 1024) / 1024).astype(np.float32)
    ids, p = O.route_topk(L, 6)
    ids2, p2 = O.route_topk(L + np.float32(16.0), 6)
    assert np.array_equal((L + np.float32(16.0)).astype(np.float64) - 16.0, L.astype(np.float64))
    assert np.array_equal(ids, ids2)
    assert np.allclose(p, p2, rtol=1e-12, atol=0)
    # p_a / p_b = exp(l_a - l_b)
    t = 3
    a, b = ids[t, 0], ids[t, 1]
    assert math.isclose(p[t, 0] / p[t, 1], math.exp(float(L[t, a]) - float(L[t, b])), rel_tol=1e-12)


def test_router_nan_ranks_below_every_number():
    row = np.array([[np.nan, -np.inf, 2.0, np.nan, -5.0]], dtype=np.float32)
    ids, p = O.route_topk(row, 3)
    assert ids[0].tolist() == [2, 4, 1]
    assert p[0, 2] == 0.0 and p[0, 0] > p[0, 1] > 0
    ids, p = O.route_topk(row, 5)
    assert ids[0].tolist() == [2, 4, 1, 0, 3]
    assert np.all(np.isnan(p[0]))
    ids, p = O.route_topk(np.full((1, 6), np.nan, dtype=np.float32), 2)
    assert ids[0].tolist() == [0, 1] and np.all(np.isnan(p[0]))


# ---------------------------------------------------------------------------
# Workload shift exponents keep the fp16 intermediate and output in range
# ---------------------------------------------------------------------------
def test_tiny_workload_shifts_have_headroom():
    w = S.WORKLOADS["tiny"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    y, h = O.mlp(S.workload_x(w), wg, wu, wd, w.hidden, w.inter)
    assert np.abs(h).max() * 2.0 ** -w.inter_shift <= 2 ** 13
    assert np.abs(y).max() * 2.0 ** -w.out_shift <= 2 ** 13


def test_oracle_matches_committed_regression_fixture(root_dir):
    import os
    path = os.path.join(root_dir, "tests", "golden", "tiny_oracle.txt")
    sections, cur = {}, None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = line[1:-1]
            sections[cur] = []
        else:
            sections[cur].append(float.fromhex(line))
    w = S.WORKLOADS["tiny"]
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    y, _ = O.mlp(S.workload_x(w), wg, wu, wd, w.hidden, w.inter)
    assert np.array_equal(O.q4k_dequant_f32(wg[0:1, 0:1], 1, 256)[0], np.array(sections["w32"], np.float32))
    assert np.allclose(y[0], sections["y0"], rtol=1e-12, atol=0)
    assert np.allclose(y[7], sections["y7"], rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# acceptance metrics: closed forms on hand-built arrays
# ---------------------------------------------------------------------------
def test_parity_metrics_closed_forms():
    # y_ref = (3, -4, 0, 1): sum|r| = 8, mean r^2 = 26/4, RMS = sqrt(6.5)
    # err = (0.5, 0, 0.25, 0): max 0.5, sum 0.75
    ref = np.array([3.0, -4.0, 0.0, 1.0])
    got = np.array([3.5, -4.0, 0.25, 1.0])
    m = O.parity_metrics(got, ref)
    assert m["rms_ref"] == pytest.approx(np.sqrt(6.5), rel=1e-15)
    assert m["max_err_over_rms"] == pytest.approx(0.5 / np.sqrt(6.5), rel=1e-15)
    assert m["mean_rel_err"] == pytest.approx(0.75 / 8.0, rel=1e-15)
    assert m["finite"]
    # the plausible slips give other numbers here: a per-element mean of
    # |e|/|r| (infinite: r has a zero), RMS of the error over RMS(ref)
    # (0.2795/2.55), max error over max |ref| (0.125)
    assert m["max_err_over_rms"] != pytest.approx(0.125)
    assert m["max_err_over_rms"] != pytest.approx(np.sqrt(0.3125 / 4) / np.sqrt(6.5))


def test_parity_metrics_pool_every_output_of_the_call():
    # two rows of very different size: the sums run over all four outputs,
    # not row by row (a row-wise mean relative error would be (0.05 + 0) / 2)
    ref = np.array([[1.0, 1.0], [10.0, 10.0]])
    got = np.array([[1.1, 1.0], [10.0, 10.0]])
    m = O.parity_metrics(got, ref)
    assert m["mean_rel_err"] == pytest.approx(0.1 / 22.0, rel=1e-12)
    assert m["max_err_over_rms"] == pytest.approx(0.1 / np.sqrt(50.5), rel=1e-12)
    assert m["rms_ref"] == pytest.approx(np.sqrt(50.5), rel=1e-15)


def test_within_tolerance_bounds_are_inclusive_and_both_bind():
    assert O.MAX_ERR_OVER_RMS == 2e-2 and O.MEAN_REL_ERR == 5e-3
    ref = np.ones(1000)                       # RMS 1, sum|r| 1000
    # mean relative error 2^-8 = 0.0039 (inside), 2^-7 = 0.0078 (outside);
    # max|err|/RMS stays below 2e-2 in both
    assert O.within_tolerance(ref + 2.0 ** -8, ref)
    assert not O.within_tolerance(ref + 2.0 ** -7, ref)
    # one large error: 2^-6 = 0.0156 (inside), 2^-5 = 0.031 (outside); the
    # mean relative error stays tiny in both
    for e, ok in ((2.0 ** -6, True), (2.0 ** -5, False)):
        got = ref.copy()
        got[17] += e
        assert O.within_tolerance(got, ref) is ok
    # at the mean bound (as exact as binary allows): decided by <=, not <
    ref2 = np.full(4, 2.0)
    got2 = ref2 + np.array([0.04, 0.0, 0.0, 0.0])   # sum|e| / sum|r| = 0.04 / 8 = 5e-3
    assert O.parity_metrics(got2, ref2)["mean_rel_err"] == pytest.approx(5e-3, rel=1e-12)
    assert O.within_tolerance(got2, ref2) == (O.parity_metrics(got2, ref2)["mean_rel_err"] <= 5e-3)


def test_within_tolerance_rejects_non_finite_outputs():
    ref = np.ones(8)
    for bad in (np.nan, np.inf, -np.inf):
        got = ref.copy()
        got[2] = bad
        assert not O.within_tolerance(got, ref)
        assert not O.parity_metrics(got, ref)["finite"]
    assert O.within_tolerance(ref.copy(), ref)


# ---------------------------------------------------------------------------
# the zero-centred weight recipe (input generator) read by the oracle
# ---------------------------------------------------------------------------
def test_centred_recipe_fields_and_mean():
    rng = np.random.default_rng(9)
    blob = S.gen_q4k_blob_centred(rng, 64, 512)
    d, dmin, sc, m, q = O.q4k_fields(blob)
    assert np.array_equal(sc, m)                                   # m_j = sc_j for every sub-block
    assert np.array_equal(dmin, np.float16(d * 7.5).astype(np.float64))
    assert sc.min() == 0 and sc.max() == 63 and q.min() == 0 and q.max() == 15
    w = O.q4k_dequant(blob, 64, 512)
    # each weight is sc*(d*q - dmin) with dmin within an fp16 rounding of 7.5*d
    d_b = np.repeat(d[..., None], 256, axis=-1).reshape(64, 512)
    assert np.all(np.abs(w) <= 63 * 8.0 * d_b * (1 + 2e-3))
    # centred: the mean is small against the spread (the uniform recipe's
    # mean is about 1.1 at a spread of about 1.5)
    assert abs(w.mean()) < 0.02 * w.std()
    wu = O.q4k_dequant(S.gen_q4k_blob(rng, 64, 512), 64, 512)
    assert wu.mean() > 0.5 * wu.std()
