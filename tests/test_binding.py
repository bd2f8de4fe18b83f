"""The Python binding's argument checks (CPU only, no compute call).

The C ABI sees pointers only, so the binding is the one layer that can compare
a tensor's dtype, shape and byte size with what a call reads or writes.  Every
wrong tensor must raise ValueError before any pointer reaches the library; a
tensor that is right in every respect but lives on the CPU is rejected last,
for being off the GPU."""
from __future__ import annotations

import pytest
import torch

import q4_swiglu_mlp_amd as Z

H, I = 256, 512


def q4k(rows, cols, extra=0):
    return torch.zeros(rows * (cols // 256) * 144 + extra, dtype=torch.uint8)


def dense_args(M=4):
    return dict(w_gate=q4k(I, H), w_up=q4k(I, H), w_down=q4k(H, I), hidden=H, inter=I,
                x=torch.zeros((M, H), dtype=torch.float16))


def call_prefill(**over):
    a = dense_args()
    a.update(over)
    return Z.zinc_mlp_q4k_prefill(a["w_gate"], a["w_up"], a["w_down"], a["hidden"], a["inter"], a["x"],
                                  y=a.get("y"), workspace=a.get("workspace"))


def test_right_tensors_on_the_cpu_are_rejected_for_the_device_only():
    with pytest.raises(ValueError, match="GPU"):
        call_prefill()


@pytest.mark.parametrize("bad,msg", [
    (dict(x=torch.zeros((4, H), dtype=torch.float32)), "float16"),
    (dict(x=torch.zeros((4, H), dtype=torch.bfloat16)), "float16"),
    (dict(x=torch.zeros((4, H + 256), dtype=torch.float16)), "shape"),
    (dict(x=torch.zeros((H,), dtype=torch.float16)), "2-D"),
    (dict(x=torch.zeros((H, 4), dtype=torch.float16).t()), "contiguous"),
    (dict(w_gate=q4k(I, H, extra=-144)), "w_gate holds"),
    (dict(w_up=q4k(I, H, extra=16)), "w_up holds"),
    (dict(w_down=q4k(I, H)[: q4k(H, I).numel() - 1]), "w_down holds"),
    (dict(y=torch.zeros((4, H), dtype=torch.float32)), "y must be"),
    (dict(y=torch.zeros((5, H), dtype=torch.float16)), "y must have shape"),
    (dict(workspace=torch.zeros(16, dtype=torch.uint8)), "workspace holds"),
    (dict(hidden=300), "multiples of 256"),
])
def test_dense_wrong_tensors_raise_before_any_call(bad, msg):
    with pytest.raises(ValueError, match=msg):
        call_prefill(**bad)


def test_decode_block_and_staged_check_like_prefill():
    a = dense_args()
    with pytest.raises(ValueError, match="float16"):
        Z.zinc_mlp_q4k_decode(a["w_gate"], a["w_up"], a["w_down"], H, I, a["x"].float())
    with pytest.raises(ValueError, match="w_down holds"):
        Z.zinc_mlp_q4k_prefill_staged(a["w_gate"], a["w_up"], q4k(H, I, extra=144), H, I, a["x"])
    with pytest.raises(ValueError, match="norm_weight must be"):
        Z.zinc_mlp_q4k_prefill_block(a["w_gate"], a["w_up"], a["w_down"], H, I, a["x"],
                                     torch.zeros(H, dtype=torch.float32), 1e-5)
    with pytest.raises(ValueError, match="norm_weight must have shape"):
        Z.zinc_mlp_q4k_decode_block(a["w_gate"], a["w_up"], a["w_down"], H, I, a["x"],
                                    torch.zeros(H - 8, dtype=torch.float16), 1e-5)


def moe_args(E=4, M=6, k=2):
    return dict(w_gate=q4k(E * I, H), w_up=q4k(E * I, H), w_down=q4k(E * H, I), n_experts=E, hidden=H, inter=I,
                x=torch.zeros((M, H), dtype=torch.float16), expert_ids=torch.zeros((M, k), dtype=torch.int32),
                expert_weights=torch.zeros((M, k), dtype=torch.float32))


def call_moe(fmt=None, **over):
    a = moe_args()
    a.update(over)
    if fmt is None:
        return Z.zinc_moe_q4k_experts(a["w_gate"], a["w_up"], a["w_down"], a["n_experts"], a["hidden"], a["inter"],
                                      a["x"], a["expert_ids"], a["expert_weights"], dev_error=a.get("dev_error"))
    return Z.zinc_moe_experts_fmt(a["w_gate"], a["w_up"], a["w_down"], fmt, a["n_experts"], a["hidden"], a["inter"],
                                  a["x"], a["expert_ids"], a["expert_weights"])


def test_moe_right_tensors_on_the_cpu_are_rejected_for_the_device_only():
    with pytest.raises(ValueError, match="GPU"):
        call_moe()


@pytest.mark.parametrize("bad,msg", [
    # torch.topk returns int64 ids: read as int32 pairs they would route half
    # the slots to expert 0 without an error
    (dict(expert_ids=torch.zeros((6, 2), dtype=torch.int64)), "int32"),
    (dict(expert_ids=torch.zeros((6, 3), dtype=torch.int32)), "expert_weights must have shape"),
    (dict(expert_ids=torch.zeros((5, 2), dtype=torch.int32)), "expert_ids must have shape"),
    (dict(expert_weights=torch.zeros((6, 2), dtype=torch.float16)), "float32"),
    (dict(w_gate=q4k(3 * I, H)), "w_gate holds"),
    (dict(w_down=q4k(4 * H, I, extra=144)), "w_down holds"),
    (dict(dev_error=torch.zeros(1, dtype=torch.int64)), "dev_error"),
    (dict(n_experts=0), "n_experts"),
])
def test_moe_wrong_tensors_raise_before_any_call(bad, msg):
    with pytest.raises(ValueError, match=msg):
        call_moe(**bad)


def test_moe_down_formats_are_sized_by_their_own_blocks():
    E = 4
    q5k = torch.zeros(E * H * (I // 256) * 176, dtype=torch.uint8)
    q51 = torch.zeros(E * H * (I // 32) * 24, dtype=torch.uint8)
    for fmt, wd in (("q5_k", q5k), ("q5_1", q51)):
        with pytest.raises(ValueError, match="GPU"):
            call_moe(fmt, w_down=wd)
    with pytest.raises(ValueError, match="w_down holds"):
        call_moe("q5_k", w_down=q51)
    with pytest.raises(ValueError, match="unknown down format"):
        call_moe("q8_0", w_down=q51)


def test_dequant_and_router_checks():
    with pytest.raises(ValueError, match="blocks holds"):
        Z.zinc_q4k_dequant_f32(q4k(3, 512, extra=1), 3, 512)
    with pytest.raises(ValueError, match="out must be"):
        Z.zinc_q4k_dequant_f32(q4k(3, 512), 3, 512, out=torch.zeros((3, 512), dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        Z.zinc_q5_dequant_f32("q5_1", torch.zeros(2 * 2 * 24, dtype=torch.uint8), 2, 64)
    with pytest.raises(ValueError, match="logits"):
        Z.zinc_moe_route_topk(torch.zeros((4, 8), dtype=torch.float64), 2)
    with pytest.raises(ValueError, match="expert_ids must be"):
        Z.zinc_moe_route_topk(torch.zeros((4, 8), dtype=torch.float32), 2,
                              expert_ids=torch.zeros((4, 2), dtype=torch.int64))
