"""CPU oracle for the Q4_K SwiGLU MLP -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never calls
it, shares no code with it and must not fall back to it.

Plain, slow, obviously-correct float64 numpy:

* ``q4k_fields`` / ``q4k_dequant``: the Q4_K super-block definition written out
  field by field (256 weights, fp16 ``d`` and ``dmin``, eight 6-bit scales and
  eight 6-bit mins, ``w = d*sc*q - dmin*m``).  The pages name the Q4_K block
  ("Fused SwiGLU MLP: ZINC RDNA4 Down-Projection Bandwidth", the opening Q&A and
  "Why this fusion is harder than the last one"; "VGPR pressure caps the fused
  RDNA4 prefill GEMM at nine waves", "What the fused GEMM actually spends
  registers on") but print no byte layout; the layout used is the public GGUF
  Q4_K block, the reading the engine implies by loading GGUF files.
* ``mlp``: the SwiGLU feed-forward block of "The MLP is two trips up to a wider
  width" -- the hidden state is projected up twice (gate and up), combined by
  SwiGLU, and projected back down:  y = W_down (silu(W_gate x) * (W_up x)),
  silu(z) = z / (1 + exp(-z)).
* ``moe``: the batched-expert form of "Four bottlenecks, one CUDA backend",
  "Bottleneck 2": each token's output is the mixing-weighted sum of its chosen
  experts' MLP outputs; expert ids are inputs.
* ``q5k_fields`` / ``q5k_dequant`` and ``q5_1_fields`` / ``q5_1_dequant``: the
  two other block formats the pages name for the experts' down projections,
  written out from the public GGUF definitions like Q4_K; ``mlp`` and ``moe``
  take the down projection's format.
* ``rms_norm`` / ``mlp_block``: the block with its neighbours -- the pre-MLP
  RMS norm and the residual add (with a per-layer scale on the MLP output).
* ``route_topk``: the router step before it -- per token the top-k experts by
  router logit and the softmax of the chosen logits.

Every function is pinned in ``tests/test_oracle.py`` against things other than
itself: hand-built blocks with closed-form weights, a bit-level brute-force
field reader, silu identities and a library sigmoid, brute-force loops on tiny
shapes, one-hot / zero / unit-weight probes, exact scaling and permutation
invariants, and MoE reductions to the dense MLP; the router against a
brute-force search over expert subsets, tie and NaN rules written out, a
library softmax, and the renormalised full softmax; the RMS norm against
torch's rms_norm, closed forms and its scale invariance, the block against its
zero-weight and zero-scale reductions.
"""
from __future__ import annotations

import numpy as np

QK_K = 256
BLOCK_BYTES = 144


# ----------------------------------------------------------------------------
# Q4_K super-block decode
# ----------------------------------------------------------------------------
def q4k_fields(blob: np.ndarray):
    """Unpack every super-block of ``blob`` (uint8, last axis 144).

    Returns ``d, dmin`` (float64, shape ``blob.shape[:-1]``), ``sc, m`` (int64,
    ``[..., 8]``: the scale and min of sub-block j covering weights
    32j..32j+31) and ``q`` (int64, ``[..., 256]``: the 4-bit quant of weight i).

    Field layout (GGUF Q4_K, little-endian):
      bytes 0-1 ``d`` (IEEE fp16), bytes 2-3 ``dmin`` (IEEE fp16);
      S = bytes 4..15:
        j < 4 : sc_j = S[j] & 63,            m_j = S[j+4] & 63
        j >= 4: sc_j = (S[j+4] & 15) | ((S[j-4] >> 6) << 4)
                m_j  = (S[j+4] >> 4) | ((S[j]   >> 6) << 4)
      Q = bytes 16..143: weight i lives in byte Q[32*(i//64) + i%32], in the
      low nibble when i%64 < 32 and in the high nibble otherwise.
    """
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.shape[-1] != BLOCK_BYTES:
        raise ValueError("last axis must be 144 bytes")
    d = blob[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = blob[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)

    S = blob[..., 4:16].astype(np.int64)
    sc = np.empty(blob.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty(blob.shape[:-1] + (8,), dtype=np.int64)
    for j in range(4):
        sc[..., j] = S[..., j] & 63
        m[..., j] = S[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (S[..., j + 4] & 15) | ((S[..., j - 4] >> 6) << 4)
        m[..., j] = (S[..., j + 4] >> 4) | ((S[..., j] >> 6) << 4)

    Q = blob[..., 16:144]
    i = np.arange(QK_K)
    byte = Q[..., 32 * (i // 64) + i % 32].astype(np.int64)   # byte holding weight i
    high = (i % 64) >= 32                                     # second half of a 64-chunk
    q = np.where(high, byte >> 4, byte & 15)
    return d, dmin, sc, m, q


def q4k_dequant(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Exact float64 weights ``[rows x cols]`` of a Q4_K matrix:
    W[r, 256*b + i] = d*sc_{i//32}*q_i - dmin*m_{i//32}  (block b of row r).

    With fp16 ``d``/``dmin`` and 6-bit scales every product needs at most 21
    significant bits, so each weight is the exact real value (the subtraction
    of two such numbers is exact in float64 too)."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(rows, cols // QK_K, BLOCK_BYTES)
    d, dmin, sc, m, q = q4k_fields(blob)
    sub = np.arange(QK_K) // 32                          # sub-block of weight i
    scale = d[..., None] * sc[..., sub]                  # [rows, nb, 256]
    minv = dmin[..., None] * m[..., sub]
    w = scale * q - minv
    return w.reshape(rows, cols)


def q4k_dequant_f32(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The fp32 weights: each exact value rounded once to nearest-even fp32."""
    return q4k_dequant(blob, rows, cols).astype(np.float32)


# ----------------------------------------------------------------------------
# Q5_K and Q5_1 decode (the experts' down projections of "Four bottlenecks,
# one CUDA backend", "Bottleneck 2": Q5_K for one MoE family, Q5_1 for the
# other).  The pages name the formats only; the layouts are the public GGUF
# blocks, as for Q4_K.
# ----------------------------------------------------------------------------
Q5K_BLOCK_BYTES = 176
Q5_1_WEIGHTS = 32
Q5_1_BLOCK_BYTES = 24


def q5k_fields(blob: np.ndarray):
    """Unpack every Q5_K super-block of ``blob`` (uint8, last axis 176).

    Returns ``d, dmin, sc, m`` as ``q4k_fields`` and ``q`` (int64, ``[..., 256]``,
    0..31).  Layout (GGUF Q5_K, little-endian): bytes 0-15 as in Q4_K (d, dmin
    and the twelve bytes of 6-bit scales and mins, same packing); QH = bytes
    16..47; Q = bytes 48..175.  Weight i = 64*c + 32*u + l (chunk c, half u,
    l < 32): its low four bits are the low (u = 0) or high (u = 1) nibble of
    Q[32*c + l], its fifth bit is bit 2*c + u of QH[l]."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.shape[-1] != Q5K_BLOCK_BYTES:
        raise ValueError("last axis must be 176 bytes")
    d, dmin, sc, m, _ = q4k_fields(np.concatenate([blob[..., :16], blob[..., 48:176]], axis=-1))
    QH = blob[..., 16:48].astype(np.int64)
    Q = blob[..., 48:176].astype(np.int64)
    i = np.arange(QK_K)
    c, u, l = i // 64, (i % 64) // 32, i % 32
    byte = Q[..., 32 * c + l]
    low4 = np.where(u == 1, byte >> 4, byte & 15)
    fifth = (QH[..., l] >> (2 * c + u)) & 1
    return d, dmin, sc, m, low4 | (fifth << 4)


def q5k_dequant(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Exact float64 weights of a Q5_K matrix: d*sc_{i//32}*q_i - dmin*m_{i//32}
    (every product fits 22 significant bits, so the value is exact)."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(rows, cols // QK_K, Q5K_BLOCK_BYTES)
    d, dmin, sc, m, q = q5k_fields(blob)
    sub = np.arange(QK_K) // 32
    w = d[..., None] * sc[..., sub] * q - dmin[..., None] * m[..., sub]
    return w.reshape(rows, cols)


def q5_1_fields(blob: np.ndarray):
    """Unpack every Q5_1 block of ``blob`` (uint8, last axis 24): ``d, m``
    (float64) and ``q`` (int64, ``[..., 32]``, 0..31).  Layout (GGUF Q5_1,
    little-endian): bytes 0-1 ``d``, bytes 2-3 ``m`` (IEEE fp16), bytes 4-7 QH (a
    32-bit word), bytes 8..23 Q.  Weight i < 16 takes the low nibble of Q[i],
    weight 16 + i the high nibble of Q[i]; bit i of QH is the fifth bit of
    weight i."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.shape[-1] != Q5_1_BLOCK_BYTES:
        raise ValueError("last axis must be 24 bytes")
    d = blob[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    mm = blob[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    qh = (blob[..., 4].astype(np.int64) | (blob[..., 5].astype(np.int64) << 8) |
          (blob[..., 6].astype(np.int64) << 16) | (blob[..., 7].astype(np.int64) << 24))
    Q = blob[..., 8:24].astype(np.int64)
    i = np.arange(Q5_1_WEIGHTS)
    byte = Q[..., i % 16]
    low4 = np.where(i >= 16, byte >> 4, byte & 15)
    fifth = (qh[..., None] >> i) & 1
    return d, mm, low4 | (fifth << 4)


def q5_1_dequant(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Exact float64 weights of a Q5_1 matrix: W[r, 32*b + i] = d*q_i + m."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(rows, cols // Q5_1_WEIGHTS, Q5_1_BLOCK_BYTES)
    d, mm, q = q5_1_fields(blob)
    return (d[..., None] * q + mm[..., None]).reshape(rows, cols)


DOWN_DECODERS = {"q4_k": q4k_dequant, "q5_k": q5k_dequant, "q5_1": q5_1_dequant}


# ----------------------------------------------------------------------------
# SwiGLU MLP
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)).  For very negative z, exp overflows to +inf
    and the quotient is -0, the correct limit; the overflow warning is muted."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def mlp_from_weights(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray):
    """Dense SwiGLU block on float64 weights.  ``x`` is ``[M x hidden]``;
    ``Wg``, ``Wu`` are ``[inter x hidden]``, ``Wd`` is ``[hidden x inter]``.
    Returns ``(y [M x hidden], h [M x inter])``."""
    x64 = np.asarray(x, dtype=np.float64)
    g = x64 @ Wg.T                  # gate projection
    u = x64 @ Wu.T                  # up projection
    h = silu(g) * u                 # SwiGLU
    y = h @ Wd.T                    # down projection
    return y, h


def mlp(x, wg_blob, wu_blob, wd_blob, hidden: int, inter: int, down_format: str = "q4_k"):
    """Dense SwiGLU block: ``(y, h)`` in float64 from the raw blobs (Q4_K gate
    and up; the down projection in ``down_format``)."""
    Wg = q4k_dequant(wg_blob, inter, hidden)
    Wu = q4k_dequant(wu_blob, inter, hidden)
    Wd = DOWN_DECODERS[down_format](wd_blob, hidden, inter)
    return mlp_from_weights(x, Wg, Wu, Wd)


def rms_norm(x, gamma, eps: float):
    """RMS norm of each row: x * gamma / sqrt(mean(x^2) + eps), in float64."""
    x64 = np.asarray(x, dtype=np.float64)
    g64 = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(x64 * x64, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        return x64 / np.sqrt(ms + eps) * g64


def mlp_block(x, gamma, eps: float, mlp_scale: float, wg_blob, wu_blob, wd_blob, hidden: int, inter: int):
    """The MLP with its neighbours of "Four bottlenecks, one CUDA backend",
    "Bottleneck 3" (norm and residual steps folded into the MLP's launches,
    the per-layer output scale with them): the pre-MLP RMS norm feeds the MLP
    and the residual stream x is added back,
        y = x + mlp_scale * MLP(rms_norm(x) * gamma).
    Returns ``(y [M x hidden], xn [M x hidden])`` in float64."""
    xn = rms_norm(x, gamma, eps)
    ym, _ = mlp(xn, wg_blob, wu_blob, wd_blob, hidden, inter)
    return np.asarray(x, dtype=np.float64) + float(mlp_scale) * ym, xn


def moe(x, wg_blobs, wu_blobs, wd_blobs, ids, p, hidden: int, inter: int, down_format: str = "q4_k"):
    """Batched-expert MLP: y[t] = sum_s p[t,s] * MLP_{ids[t,s]}(x[t]).

    ``wg_blobs``/``wu_blobs``: ``[E, inter, hidden/256, 144]``; ``wd_blobs``:
    ``[E, hidden, ...]`` blocks of ``down_format`` (Q4_K by default, or Q5_K /
    Q5_1); ``ids`` int ``[M, k]``; ``p`` float32
    ``[M, k]`` (widened to float64).  A slot whose id is outside [0, E)
    contributes nothing.  Returns ``(y [M x hidden] float64, n_bad_slots)``."""
    x64 = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    p64 = np.asarray(p, dtype=np.float32).astype(np.float64)
    E = wg_blobs.shape[0]
    M = x64.shape[0]
    y = np.zeros((M, hidden), dtype=np.float64)
    bad = int(np.count_nonzero((ids < 0) | (ids >= E)))
    for e in range(E):
        rows, slots = np.nonzero(ids == e)
        if rows.size == 0:
            continue
        ye, _ = mlp(x64[rows], wg_blobs[e], wu_blobs[e], wd_blobs[e], hidden, inter, down_format)
        np.add.at(y, rows, p64[rows, slots][:, None] * ye)
    return y, bad


# ----------------------------------------------------------------------------
# MoE router: top-k experts and mixing weights
# ----------------------------------------------------------------------------
def route_topk(logits, top_k: int):
    """The router step of "Four bottlenecks, one CUDA backend", "Bottleneck 2"
    (every MoE layer computes router logits and picks the top-k experts).

    Per token: the ``top_k`` experts with the largest logits, largest first;
    equal logits in increasing expert index; a NaN logit ranks below every
    number.  Mixing weights: the softmax of the chosen logits (the reading
    taken: the full softmax renormalised over the chosen experts, the same
    value), computed in float64 as exp(l_s - l_0) / sum_j exp(l_j - l_0) with
    l_0 the first (largest) chosen logit.

    ``logits`` float32 ``[M, E]``.  Returns ``(ids int32 [M, k], p float64 [M, k])``."""
    L = np.asarray(logits, dtype=np.float32)
    M, E = L.shape
    ids = np.empty((M, top_k), dtype=np.int32)
    p = np.empty((M, top_k), dtype=np.float64)
    for t in range(M):
        row = [float(v) for v in L[t]]

        def rank(j):
            v = row[j]
            is_number = not np.isnan(v)
            return (is_number, v if is_number else 0.0, -j)

        chosen = sorted(range(E), key=rank, reverse=True)[:top_k]
        v = np.array([row[j] for j in chosen], dtype=np.float64)
        with np.errstate(invalid="ignore"):
            e = np.exp(v - v[0])
            p[t] = e / e.sum()
        ids[t] = chosen
    return ids, p


# ----------------------------------------------------------------------------
# Acceptance metrics
# ----------------------------------------------------------------------------
def parity_metrics(y_test: np.ndarray, y_ref: np.ndarray) -> dict:
    """max|err| / RMS(ref) and sum|err| / sum|ref| (the mean relative error
    read over all outputs of a call)."""
    yt = np.asarray(y_test, dtype=np.float64)
    yr = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(yt - yr)
    rms = float(np.sqrt(np.mean(yr * yr)))
    return {
        "max_err_over_rms": float(err.max() / rms) if rms > 0 else float(err.max()),
        "mean_rel_err": float(err.sum() / np.abs(yr).sum()) if np.abs(yr).sum() > 0 else float(err.sum()),
        "rms_ref": rms,
        "finite": bool(np.isfinite(yt).all()),
    }


MAX_ERR_OVER_RMS = 2e-2
MEAN_REL_ERR = 5e-3


def within_tolerance(y_test, y_ref) -> bool:
    m = parity_metrics(y_test, y_ref)
    return m["finite"] and m["max_err_over_rms"] <= MAX_ERR_OVER_RMS and m["mean_rel_err"] <= MEAN_REL_ERR
