"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments before any HIP call (no GPU needed)."""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")

kq = pytest.importorskip("gguf_quant_matmul_amd.kq", reason="libkq.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree_and_library_exports_all():
    declared = _declared()
    assert declared == sorted(kq.EXPORTS)
    for name in declared:
        assert hasattr(kq._lib, name), name


def test_no_torch_types_in_header():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("pytorch", "") or "at::" not in text
    assert "at::Tensor" not in text and "c10" not in text


def test_codec_registry():
    # mlx-kquant README "Codec reference" table
    assert kq.kq_codec_info("q4_k") == (256, 144)
    assert kq.kq_codec_info("q6_k") == (256, 210)
    assert kq.kq_codec_info("q8_0") == (32, 34)
    assert kq.kq_codec_info("q4_0") == (32, 18)
    assert kq.kq_codec_info("q5_k") == (256, 176)
    assert kq.kq_codec_from_name("Q4_K") == kq.KQ_Q4_K
    assert kq.kq_codec_from_name("q5_k") == kq.KQ_Q5_K == 13
    assert kq.kq_row_bytes("q5_k", 4096) == 2816
    for name, cid, geo in (("q4_1", 3, (32, 20)), ("q5_0", 6, (32, 22)), ("q5_1", 7, (32, 24)), ("q2_k", 10, (256, 84)),
                             ("q3_k", 11, (256, 110))):
        assert kq.kq_codec_from_name(name) == cid and kq.kq_codec_info(name) == geo
    assert kq.kq_row_bytes("q6_k", 4096) == 3360
    assert kq.kq_row_bytes("q8_0", 4096) == 4352
    with pytest.raises(kq.KQError) as e:
        kq.kq_codec_from_name("iq2_xxs")
    assert e.value.status == kq.KQ_ERR_CODEC
    with pytest.raises(kq.KQError) as e:
        kq.kq_row_bytes("q4_k", 4000)
    assert e.value.status == kq.KQ_ERR_SHAPE and "not a multiple of 256" in str(e.value)
    assert kq.kq_version()


def test_tile_map_capacity_matches_bound():
    from oracle import matmul

    for rows, e in [(0, 1), (1, 1), (4096, 64), (100, 500), (65, 1), (12345, 7)]:
        assert kq.kq_expert_tile_map_capacity(rows, e) == matmul.tile_map_capacity(rows, e)


# Argument errors: fake (never dereferenced) pointers; each call must fail on the host.
A16 = 0x10000  # a 16-byte aligned fake address
L = kq._lib


def _st(ret):
    return ret, kq.kq_last_error()


@pytest.mark.parametrize(
    "call, status, msg",
    [
        (lambda: L.kq_qmv(12, A16, 64, 4000, A16, 1, A16, 0, None), kq.KQ_ERR_SHAPE, "K=4000"),
        (lambda: L.kq_qmv(12, A16, 64, 4096, A16, 17, A16, 0, None), kq.KQ_ERR_SHAPE, "M=17"),
        (lambda: L.kq_qmv(99, A16, 64, 4096, A16, 1, A16, 0, None), kq.KQ_ERR_CODEC, "codec"),
        (lambda: L.kq_qmv(12, A16 + 4, 64, 4096, A16, 1, A16, 0, None), kq.KQ_ERR_ALIGN, "w="),
        (lambda: L.kq_qmv(12, A16, 64, 4096, A16 + 2, 1, A16, 0, None), kq.KQ_ERR_ALIGN, "x="),
        (lambda: L.kq_qmv(12, None, 64, 4096, A16, 1, A16, 0, None), kq.KQ_ERR_ARG, "null"),
        (lambda: L.kq_qmv(12, A16, 64, 4096, A16, 1, A16, 7, None), kq.KQ_ERR_ARG, "dtype"),
        (lambda: L.kq_qmm(14, A16, 64, 0, A16, 1, A16, 0, None), kq.KQ_ERR_SHAPE, "K=0"),
        (lambda: L.kq_qmm(8, A16, -1, 64, A16, 1, A16, 0, None), kq.KQ_ERR_ARG, "N=-1"),
        (lambda: L.kq_qmm(8, A16, 64, 64, A16, 1, A16 + 1, 0, None), kq.KQ_ERR_ALIGN, "y="),
        (lambda: L.kq_dequantize(2, A16, 4, 48, A16, 0, None), kq.KQ_ERR_SHAPE, "K=48"),
        (lambda: L.kq_dequantize(2, A16, 4, 64, A16 + 8, 0, None), kq.KQ_ERR_ALIGN, "out="),
        (lambda: L.kq_expert_tile_map(A16, 4096, 64, A16, A16, 100, None, None), kq.KQ_ERR_CAPACITY, "cap=100"),
        (lambda: L.kq_expert_tile_map(A16, 10, 0, A16, A16, 100, None, None), kq.KQ_ERR_ARG, "n_experts"),
        (lambda: L.kq_expert_tile_map(A16 + 2, 10, 4, A16, A16, 100, None, None), kq.KQ_ERR_ALIGN, "aligned"),
        (lambda: L.kq_gather_qmm_seg(12, A16, 0, 64, 256, A16, 10, A16, A16, 8, A16, 1, None), kq.KQ_ERR_ARG,
         "n_experts"),
        (lambda: L.kq_gather_qmm_seg(12, A16, 4, 64, 256, A16, 10, None, A16, 8, A16, 1, None), kq.KQ_ERR_ARG,
         "map"),
        (lambda: L.kq_gather_qmv(8, A16, 4, 64, 96, A16, A16, 8, A16, 0, None), kq.KQ_ERR_SHAPE, "K=96"),
        (lambda: L.kq_gather_qmv(12, A16, 0, 64, 256, A16, A16, 8, A16, 0, None), kq.KQ_ERR_ARG, "n_experts"),
        (lambda: L.kq_gather_qmv(12, A16, 4, 64, 256, A16, None, 8, A16, 0, None), kq.KQ_ERR_ARG, "ids"),
        (lambda: L.kq_gather_qmv(12, A16, 4, 64, 256, A16, A16 + 2, 8, A16, 0, None), kq.KQ_ERR_ALIGN, "ids="),
        (lambda: L.kq_moe_glu_gather(8, A16, A16, 4, 64, 96, A16, 2, A16, 2, 0, 0.0, A16, 0, None),
         kq.KQ_ERR_SHAPE, "K=96"),
        (lambda: L.kq_moe_glu_gather(12, A16, A16, 0, 64, 256, A16, 2, A16, 2, 0, 0.0, A16, 0, None),
         kq.KQ_ERR_ARG, "n_experts"),
        (lambda: L.kq_moe_glu_gather(12, A16, A16, 4, 64, 256, A16, 2, A16, 2, 3, 0.0, A16, 0, None),
         kq.KQ_ERR_ARG, "act=3"),
        (lambda: L.kq_moe_glu_gather(12, A16, A16, 4, 64, 256, A16, 2, A16, 2, 2, 0.0, A16, 0, None),
         kq.KQ_ERR_ARG, "limit"),
        (lambda: L.kq_moe_glu_gather(12, A16, A16, 4, 64, 256, A16, 2, A16, 2, 2, float("inf"), A16, 0, None),
         kq.KQ_ERR_ARG, "limit"),
        (lambda: L.kq_moe_glu_gather(12, A16, None, 4, 64, 256, A16, 2, A16, 2, 0, 0.0, A16, 0, None),
         kq.KQ_ERR_ARG, "up_w"),
        (lambda: L.kq_moe_glu_gather(12, A16, A16 + 2, 4, 64, 256, A16, 2, A16, 2, 0, 0.0, A16, 0, None),
         kq.KQ_ERR_ALIGN, "up_w="),
        (lambda: L.kq_moe_glu_gather(12, A16, A16, 4, 64, 256, A16, 2, None, 2, 0, 0.0, A16, 0, None),
         kq.KQ_ERR_ARG, "ids"),
        (lambda: L.kq_moe_glu_gather(12, A16, A16, 4, 64, 256, A16, -1, A16, 2, 0, 0.0, A16, 0, None),
         kq.KQ_ERR_ARG, "tokens"),
        (lambda: L.kq_moe_glu_gather(12, A16, A16, 4, 64, 256, A16, 2, A16, -2, 0, 0.0, A16, 0, None),
         kq.KQ_ERR_ARG, "top_k"),
        (lambda: L.kq_gather_mix(A16, 8, 6, A16, A16, 2, 4, A16, 1, None), kq.KQ_ERR_SHAPE, "N=6"),
        (lambda: L.kq_gather_mix(A16, 8, 8, A16, A16, 2, 4, A16, 3, None), kq.KQ_ERR_ARG, "dtype"),
        (lambda: L.kq_gather_mix(A16, 8, 8, None, A16, 2, 4, A16, 1, None), kq.KQ_ERR_ARG, "inv_order"),
        (lambda: L.kq_gather_mix(A16, 8, 8, A16, A16, 2, 4, None, 1, None), kq.KQ_ERR_ARG, "out"),
        (lambda: L.kq_gather_mix(A16 + 4, 8, 8, A16, A16, 2, 4, A16, 1, None), kq.KQ_ERR_ALIGN, "y="),
        (lambda: L.kq_gather_mix(A16, 8, 8, A16 + 2, A16, 2, 4, A16, 1, None), kq.KQ_ERR_ALIGN, "inv_order"),
        (lambda: L.kq_stream_read(A16, 24, A16, 4, None), kq.KQ_ERR_ARG, "bytes=24"),
        (lambda: L.kq_stream_read(A16, 64, A16, 0, None), kq.KQ_ERR_ARG, "groups=0"),
        (lambda: L.kq_stream_read(None, 64, A16, 4, None), kq.KQ_ERR_ARG, "null"),
        (lambda: L.kq_stream_read(A16 + 4, 64, A16, 4, None), kq.KQ_ERR_ALIGN, "16-byte"),
        (lambda: L.kq_gather_mix(A16, 8, 8, A16, A16, -1, 4, A16, 1, None), kq.KQ_ERR_ARG, "tokens"),
        (lambda: L.kq_quantized_matmul_residual(12, A16, 64, 256, A16, 4, A16 * 4, A16 * 8, 3, A16, 0, None),
         kq.KQ_ERR_SHAPE, "gate_rows=3"),
        (lambda: L.kq_quantized_matmul_residual(12, A16, 64, 256, A16, 4, None, None, 0, A16, 0, None),
         kq.KQ_ERR_ARG, "null residual"),
        (lambda: L.kq_quantized_matmul_residual(12, A16, 64, 256, A16, 4, A16 * 4 + 2, None, 0, A16, 0, None),
         kq.KQ_ERR_ALIGN, "residual"),
        (lambda: L.kq_quantized_matmul_residual(12, A16, 64, 256, A16, 4, A16 + 256, None, 0, A16, 0, None),
         kq.KQ_ERR_ARG, "residual overlaps"),
        (lambda: L.kq_quantized_matmul_residual(12, A16, 64, 256, A16, 4, A16, A16 + 256, 2, A16, 1, None),
         kq.KQ_ERR_ARG, "gate overlaps"),
        (lambda: L.kq_quantized_matmul_qmv_bias(8, A16, 64, 256, A16, 2, A16 * 4, A16, 0, None),
         kq.KQ_ERR_SHAPE, "M=2"),
        (lambda: L.kq_quantized_matmul_qmv_bias(8, A16, 64, 256, A16, 1, None, A16, 0, None),
         kq.KQ_ERR_ARG, "null bias"),
        (lambda: L.kq_quantized_matmul_qmv_bias(8, A16, 64, 256, A16, 1, A16 + 64, A16, 1, None),
         kq.KQ_ERR_ARG, "bias overlaps"),
        (lambda: L.kq_quantized_matmul_glu(12, A16, A16, 64, 256, A16, 4, 2, A16, 0, None),
         kq.KQ_ERR_ARG, "act=2"),
        (lambda: L.kq_quantized_matmul_glu(12, A16, None, 64, 256, A16, 4, 0, A16, 0, None),
         kq.KQ_ERR_ARG, "w_up"),
        (lambda: L.kq_quantized_matmul_glu(12, A16, A16 + 8, 64, 256, A16, 4, 0, A16, 0, None),
         kq.KQ_ERR_ALIGN, "w_up="),
        (lambda: L.kq_quantized_matmul_glu(12, A16, A16, 64, 250, A16, 4, 0, A16, 0, None),
         kq.KQ_ERR_SHAPE, "K=250"),
        (lambda: L.kq_quantize(12, A16, 4, 512, A16 + 4, None), kq.KQ_ERR_ALIGN, "aligned"),
        (lambda: L.kq_quantize(9, A16, 4, 512, A16, None), kq.KQ_ERR_CODEC, "codec"),
    ],
)
def test_argument_errors_return_before_launch(call, status, msg):
    ret, err = _st(call())
    assert ret == status, (ret, err)
    assert msg in err, err
    assert err.startswith("[kq_")


def test_empty_inputs_are_no_ops():
    # Zero-sized problems return KQ_OK without touching the device.
    assert L.kq_qmv(12, None, 0, 256, None, 1, None, 0, None) == 0
    assert L.kq_qmm(12, None, 64, 256, None, 0, None, 1, None) == 0
    assert L.kq_dequantize(14, None, 0, 256, None, 1, None) == 0
    assert L.kq_gather_qmm_seg(12, None, 4, 64, 256, None, 0, None, None, 8, None, 1, None) == 0
    assert L.kq_gather_qmv(12, None, 4, 64, 256, None, None, 0, None, 0, None) == 0
    assert L.kq_moe_glu_gather(12, None, None, 4, 64, 256, None, 0, None, 8, 0, 0.0, None, 0, None) == 0
    assert L.kq_gather_mix(None, 0, 8, None, None, 0, 4, None, 1, None) == 0
    assert L.kq_gather_mix(None, 0, 0, None, None, 5, 4, None, 1, None) == 0
    assert L.kq_moe_glu_gather(12, None, None, 4, 64, 256, None, 3, None, 0, 1, 0.0, None, 0, None) == 0
    assert L.kq_quantize(8, None, 0, 64, None, None) == 0
    assert L.kq_quantized_matmul_residual(12, None, 64, 256, None, 0, None, None, 0, None, 0, None) == 0
    assert L.kq_quantized_matmul_qmv_bias(8, None, 0, 256, None, 1, None, None, 1, None) == 0
    assert L.kq_quantized_matmul_glu(14, None, None, 0, 256, None, 3, 1, None, 0, None) == 0
