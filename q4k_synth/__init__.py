"""Seeded synthetic inputs for the Q4_K SwiGLU MLP: the only module that both the
HIP path's tests/benchmark and the CPU oracle read.

It draws raw Q4_K super-block bytes, fp16 activations and MoE routing tables,
and holds none of the method's arithmetic: nothing here decodes a block, takes
a product or applies SwiGLU.

Q4_K super-block (144 bytes, 256 weights along the contraction dimension):
bytes 0-1 fp16 ``d``, bytes 2-3 fp16 ``dmin``, bytes 4-15 twelve bytes that
carry eight 6-bit scales and eight 6-bit mins, bytes 16-143 the 256 4-bit
quants.  A matrix ``[rows x cols]`` is stored row-major as
``rows x (cols/256)`` blocks, blocks running along ``cols``.

Value recipe (the workloads' weight generator):
  * ``d`` and ``dmin``: independent uniform reals in [1e-3, 1e-2], rounded to
    fp16 (round-to-nearest-even, numpy's float64->float16 cast);
  * bytes 4..143: independent uniform bytes.  The 12 scale bytes map one-to-one
    onto the sixteen 6-bit fields and each quant byte holds two nibbles, so
    uniform bytes are exactly uniform 6-bit scales/mins in 0..63 and uniform
    quants in 0..15, whatever the bit layout is;
  * ``x``: normal(0, sd) in float64, rounded to fp16.

Seeding: every workload has a base seed.  ``x`` comes from
``default_rng([seed, 0])``; the weights of layer ``l`` come from
``default_rng([seed, l + 1])`` (gate, up, down in that order; for MoE all
experts' gate, then all up, then all down); MoE routing comes from
``default_rng([seed, 1000])``.  A single layer can therefore be generated
without drawing the others.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

QK_K = 256            # weights per super-block
BLOCK_BYTES = 144     # bytes per super-block


def gen_q4k_blob(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Random Q4_K matrix ``[rows x cols]`` as a uint8 array ``[rows, cols/256, 144]``."""
    if cols % QK_K:
        raise ValueError("cols must be a multiple of 256")
    nb = cols // QK_K
    blob = np.empty((rows, nb, BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(1e-3, 1e-2, size=(rows, nb)).astype(np.float16)
    dmin = rng.uniform(1e-3, 1e-2, size=(rows, nb)).astype(np.float16)
    blob[:, :, 0:2] = d.view(np.uint8).reshape(rows, nb, 2)
    blob[:, :, 2:4] = dmin.view(np.uint8).reshape(rows, nb, 2)
    blob[:, :, 4:] = rng.integers(0, 256, size=(rows, nb, BLOCK_BYTES - 4), dtype=np.uint8)
    return blob


def gen_q4k_blob_centred(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Random Q4_K matrix whose sub-blocks are centred on zero, as the blocks of
    a real GGUF tensor are: every sub-block's min field equals its scale field
    (m_j = sc_j) and dmin = fp16(7.5 * d), so each weight is close to
    d * sc_j * (q - 7.5), spread evenly around 0 (the uniform recipe of
    gen_q4k_blob has a mean of about +1.1).  Scales and quants stay uniform
    random.

    The equal fields come from the byte layout of the block's 12 scale bytes
    S: sc_j and m_j of the first four sub-blocks are the low six bits of S[j]
    and S[j + 4], and those of the last four are split between the nibbles of
    S[j + 4] and the top two bits of S[j - 4] and S[j].  So S[4:8] = S[0:4]
    with both nibbles of each of S[8:12] equal gives m_j = sc_j for all eight.
    """
    if cols % QK_K:
        raise ValueError("cols must be a multiple of 256")
    nb = cols // QK_K
    blob = np.empty((rows, nb, BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(1e-3, 1e-2, size=(rows, nb)).astype(np.float16)
    dmin = (d.astype(np.float64) * 7.5).astype(np.float16)
    blob[:, :, 0:2] = d.view(np.uint8).reshape(rows, nb, 2)
    blob[:, :, 2:4] = dmin.view(np.uint8).reshape(rows, nb, 2)
    low = rng.integers(0, 256, size=(rows, nb, 4), dtype=np.uint8)
    nib = rng.integers(0, 16, size=(rows, nb, 4), dtype=np.uint8)
    blob[:, :, 4:8] = low
    blob[:, :, 8:12] = low
    blob[:, :, 12:16] = nib | (nib << 4)
    blob[:, :, 16:] = rng.integers(0, 256, size=(rows, nb, BLOCK_BYTES - 16), dtype=np.uint8)
    return blob


def centred_layer_weights(seed: int, layer: int, hidden: int, inter: int):
    """The zero-centred recipe's gate, up and down blobs for one layer."""
    rng = np.random.default_rng([seed, 500 + layer])
    wg = gen_q4k_blob_centred(rng, inter, hidden)
    wu = gen_q4k_blob_centred(rng, inter, hidden)
    wd = gen_q4k_blob_centred(rng, hidden, inter)
    return wg, wu, wd


def gen_x(rng: np.random.Generator, M: int, hidden: int, sd: float = 1.0) -> np.ndarray:
    """fp16 activations ``[M x hidden]``, normal(0, sd) rounded to fp16."""
    return (rng.standard_normal((M, hidden)) * sd).astype(np.float16)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  ``inter_shift``/``out_shift`` are the power-of-two
    exponents the intermediate and the output are divided by before they are
    stored in fp16 (see the entry points' header); they were chosen from the
    oracle's value ranges on this recipe with at least 4x headroom below 2^15."""
    name: str
    hidden: int
    inter: int
    M: int
    seed: int
    x_sd: float = 1.0
    layers: int = 1
    inter_shift: int = 0
    out_shift: int = 0
    n_experts: int = 0
    top_k: int = 0
    extra: dict = field(default_factory=dict)


# The five workloads of the study, named by what they are.
WORKLOADS = {
    # tiny fused MLP, hidden 256 / intermediate 768, 8 tokens, seed 0
    "tiny": Workload("tiny", 256, 768, 8, seed=0, inter_shift=0, out_shift=8),
    # one 9B-shaped MLP layer on a 256-token prefill tile, seed 1
    "prefill_m256": Workload("prefill_m256", 4096, 11008, 256, seed=1,
                             inter_shift=5, out_shift=16),
    # large compute-bound prefill, 2048 tokens, 32 independent layers, seed 2
    "prefill_m2048": Workload("prefill_m2048", 4096, 11008, 2048, seed=2, x_sd=0.5,
                              layers=32, inter_shift=4, out_shift=15),
    # HBM-bound decode, 1 and 4 tokens, 32 independent layers, seed 3
    "decode_m1": Workload("decode_m1", 4096, 11008, 1, seed=3, layers=32,
                          inter_shift=5, out_shift=14),
    "decode_m4": Workload("decode_m4", 4096, 11008, 4, seed=3, layers=32,
                          inter_shift=5, out_shift=14),
    # batched-expert MoE: 64 experts of 2048 -> 768, 512 tokens, top-8, seed 4
    "moe_e64": Workload("moe_e64", 2048, 768, 512, seed=4, inter_shift=4, out_shift=13,
                        n_experts=64, top_k=8),
}


def layer_weights(seed: int, layer: int, hidden: int, inter: int):
    """Gate ``[inter x hidden]``, up ``[inter x hidden]``, down ``[hidden x inter]`` blobs."""
    rng = np.random.default_rng([seed, layer + 1])
    wg = gen_q4k_blob(rng, inter, hidden)
    wu = gen_q4k_blob(rng, inter, hidden)
    wd = gen_q4k_blob(rng, hidden, inter)
    return wg, wu, wd


def workload_x(w: Workload, M: int | None = None) -> np.ndarray:
    rng = np.random.default_rng([w.seed, 0])
    return gen_x(rng, w.M if M is None else M, w.hidden, w.x_sd)


def expert_weights(seed: int, n_experts: int, hidden: int, inter: int, layer: int = 0):
    """Stacked expert blobs: gate/up ``[E, inter, hidden/256, 144]``, down ``[E, hidden, inter/256, 144]``."""
    rng = np.random.default_rng([seed, layer + 1])
    wg = np.stack([gen_q4k_blob(rng, inter, hidden) for _ in range(n_experts)])
    wu = np.stack([gen_q4k_blob(rng, inter, hidden) for _ in range(n_experts)])
    wd = np.stack([gen_q4k_blob(rng, hidden, inter) for _ in range(n_experts)])
    return wg, wu, wd


def gen_routing(rng: np.random.Generator, M: int, n_experts: int, top_k: int):
    """Per token ``top_k`` distinct expert ids (uniform, without replacement) and
    mixing weights = softmax of ``top_k`` standard-normal logits (computed in
    float64, stored as float32).  Returns ``(ids int32 [M, k], p float32 [M, k])``."""
    ids = np.empty((M, top_k), dtype=np.int32)
    for t in range(M):
        ids[t] = rng.choice(n_experts, size=top_k, replace=False)
    logits = rng.standard_normal((M, top_k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, p


def workload_routing(w: Workload, M: int | None = None):
    rng = np.random.default_rng([w.seed, 1000])
    return gen_routing(rng, w.M if M is None else M, w.n_experts, w.top_k)


def gen_router_logits(rng: np.random.Generator, M: int, n_experts: int, scale: float = 1.0):
    """Router logits ``float32 [M, n_experts]``: ``scale`` times standard normals."""
    return (rng.standard_normal((M, n_experts)) * scale).astype(np.float32)


def workload_router_logits(w: Workload, M: int | None = None):
    rng = np.random.default_rng([w.seed, 2000])
    return gen_router_logits(rng, w.M if M is None else M, w.n_experts)


def gen_q5k_blob(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """A Q5_K matrix ``[rows, cols/256, 176]``: uniform random bytes for the
    scales, the fifth bits and the quants; d and dmin as for Q4_K."""
    nb = cols // 256
    blob = rng.integers(0, 256, size=(rows, nb, 176), dtype=np.uint8)
    for off in (0, 2):
        v = rng.uniform(1e-3, 1e-2, size=(rows, nb)).astype(np.float16)
        blob[..., off:off + 2] = v.view(np.uint8).reshape(rows, nb, 2)
    return blob


def gen_q5_1_blob(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """A Q5_1 matrix ``[rows, cols/32, 24]``: uniform random fifth bits and
    quants, d ~ U[1e-3, 1e-2] and m = -16 d u with u ~ U[0.5, 1.5] (so the
    weights d q + m straddle zero), both rounded to fp16."""
    nb = cols // 32
    blob = rng.integers(0, 256, size=(rows, nb, 24), dtype=np.uint8)
    d = rng.uniform(1e-3, 1e-2, size=(rows, nb))
    m = -16.0 * d * rng.uniform(0.5, 1.5, size=(rows, nb))
    blob[..., 0:2] = d.astype(np.float16).view(np.uint8).reshape(rows, nb, 2)
    blob[..., 2:4] = m.astype(np.float16).view(np.uint8).reshape(rows, nb, 2)
    return blob


def gen_down_blob(rng: np.random.Generator, fmt: str, rows: int, cols: int) -> np.ndarray:
    return {"q4_k": gen_q4k_blob, "q5_k": gen_q5k_blob, "q5_1": gen_q5_1_blob}[fmt](rng, rows, cols)
