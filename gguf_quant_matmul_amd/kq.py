"""Thin ctypes binding of libkq (include/kq.h): same names, argument marshalling only.

Every function here forwards device pointers, sizes and the current HIP stream
to the C ABI; all work runs in libkq's HIP kernels.  PyTorch supplies device
memory and streams.  There is no fallback: if libkq.so is missing the import
fails, and a failing call raises ``KQError`` with the library's message.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m gguf_quant_matmul_amd.build`")

# torch's HIP runtime must be the only one in the process.  libkq.so asks for
# libamdhip64.so.7 and takes whichever copy of that soname is already loaded;
# torch's own libraries name their bundled copy by another file name, so
# opening libkq.so first would bring in a second HIP runtime that, once torch
# holds the GPU, finds no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

c_int, c_i64, c_vp, c_cp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_char_p
_P = ctypes.POINTER

_SIGS = {
    "kq_codec_from_name": (c_int, [c_cp, _P(c_int)]),
    "kq_codec_info": (c_int, [c_int, _P(c_int), _P(c_int)]),
    "kq_row_bytes": (c_int, [c_int, c_i64, _P(c_i64)]),
    "kq_last_error": (c_cp, []),
    "kq_version": (c_cp, []),
    "kq_dequantize": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_int, c_vp]),
    "kq_qmv": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_int, c_vp]),
    "kq_qmm": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_int, c_vp]),
    "kq_quantized_matmul": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_int, c_vp]),
    "kq_quantized_matmul_residual": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_int,
                                             c_vp]),
    "kq_quantized_matmul_qmv_bias": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_int, c_vp]),
    "kq_quantized_matmul_glu": (c_int, [c_int, c_vp, c_vp, c_i64, c_i64, c_vp, c_i64, c_int, c_vp, c_int, c_vp]),
    "kq_expert_tile_map_capacity": (c_i64, [c_i64, c_i64]),
    "kq_expert_tile_map": (c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp]),
    "kq_gather_qmm_seg": (c_int, [c_int, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_int, c_vp]),
    "kq_gather_qmv": (c_int, [c_int, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_int, c_vp]),
    "kq_moe_glu_gather": (c_int, [c_int, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_int,
                                  ctypes.c_float, c_vp, c_int, c_vp]),
    "kq_gather_mix": (c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_i64, c_i64, c_vp, c_int, c_vp]),
    "kq_quantize": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_vp]),
    "kq_stream_read": (c_int, [c_vp, c_i64, c_vp, c_i64, c_vp]),
    "kq_qmv_bf16": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_int, c_vp]),
    "kq_qmm_bf16": (c_int, [c_int, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_int, c_vp]),
    "kq_gather_qmm_seg_bf16": (c_int, [c_int, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_int,
                                       c_vp]),
}

#: every symbol the header declares
EXPORTS = tuple(_SIGS)

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

# ids and enums of include/kq.h
KQ_Q4_0, KQ_Q4_1, KQ_Q5_0, KQ_Q5_1, KQ_Q8_0 = 2, 3, 6, 7, 8
KQ_Q2_K, KQ_Q3_K, KQ_Q4_K, KQ_Q5_K, KQ_Q6_K = 10, 11, 12, 13, 14
KQ_F32, KQ_F16, KQ_BF16 = 0, 1, 2
KQ_GLU_SILU, KQ_GLU_GELU_TANH, KQ_GLU_SILU_LIMIT = 0, 1, 2
_GLU_ACTS = {"silu": KQ_GLU_SILU, "gelu": KQ_GLU_GELU_TANH, "gelu_tanh": KQ_GLU_GELU_TANH,
             "silu_limit": KQ_GLU_SILU_LIMIT}
KQ_OK, KQ_ERR_ARG, KQ_ERR_CODEC, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_CAPACITY, KQ_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "KQ_OK", -1: "KQ_ERR_ARG", -2: "KQ_ERR_CODEC", -3: "KQ_ERR_SHAPE", -4: "KQ_ERR_ALIGN",
                -5: "KQ_ERR_CAPACITY", -6: "KQ_ERR_HIP"}


class KQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(status: int) -> None:
    if status != KQ_OK:
        raise KQError(status, _lib.kq_last_error().decode())


def _codec(c) -> int:
    if isinstance(c, str):
        return kq_codec_from_name(c)
    return int(c)


def _ptr(t) -> int | None:
    """Device pointer of a tensor (None for None)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _dtype_id(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return KQ_F32
    if t.dtype == torch.float16:
        return KQ_F16
    if t.dtype == torch.bfloat16:
        return KQ_BF16
    raise TypeError(f"output dtype must be float32, float16 or bfloat16, got {t.dtype}")


def _bf16(x) -> bool:
    """True for bfloat16 activations (the *_bf16 entry points), False for float16."""
    import torch

    if x.dtype == torch.bfloat16:
        return True
    if x.dtype == torch.float16:
        return False
    raise TypeError(f"activations must be float16 or bfloat16, got {x.dtype}")


# ---------------------------------------------------------------------------
# registry
# ---------------------------------------------------------------------------

def kq_codec_from_name(name: str) -> int:
    out = c_int()
    _check(_lib.kq_codec_from_name(name.encode(), ctypes.byref(out)))
    return out.value


def kq_codec_info(codec) -> tuple[int, int]:
    bv, bb = c_int(), c_int()
    _check(_lib.kq_codec_info(_codec(codec), ctypes.byref(bv), ctypes.byref(bb)))
    return bv.value, bb.value


def kq_row_bytes(codec, k: int) -> int:
    out = c_i64()
    _check(_lib.kq_row_bytes(_codec(codec), k, ctypes.byref(out)))
    return out.value


def kq_last_error() -> str:
    return _lib.kq_last_error().decode()


def kq_version() -> str:
    return _lib.kq_version().decode()


def kq_expert_tile_map_capacity(rows: int, n_experts: int) -> int:
    return int(_lib.kq_expert_tile_map_capacity(rows, n_experts))


# ---------------------------------------------------------------------------
# ops: tensors in, outputs written in place (the caller allocates)
# ---------------------------------------------------------------------------

def kq_dequantize(codec, w, k: int, out, stream=None) -> None:
    """w: uint8 [rows, row_bytes] -> out: float32/float16 [rows, k]."""
    rows = w.shape[0] if w.dim() > 1 else 1
    _check(_lib.kq_dequantize(_codec(codec), _ptr(w), rows, k, _ptr(out), _dtype_id(out), _stream(stream)))


def kq_qmv(codec, w, n: int, k: int, x, y, stream=None) -> None:
    """y[m, n] = x[m, :] . dequant(w)[n, :]; x float16 or bfloat16 [m, k] with 1 <= m <= 16."""
    fn = _lib.kq_qmv_bf16 if _bf16(x) else _lib.kq_qmv
    _check(fn(_codec(codec), _ptr(w), n, k, _ptr(x), x.shape[0], _ptr(y), _dtype_id(y), _stream(stream)))


def kq_qmm(codec, w, n: int, k: int, x, y, stream=None) -> None:
    fn = _lib.kq_qmm_bf16 if _bf16(x) else _lib.kq_qmm
    _check(fn(_codec(codec), _ptr(w), n, k, _ptr(x), x.shape[0], _ptr(y), _dtype_id(y), _stream(stream)))


def kq_quantized_matmul(codec, w, n: int, k: int, x, y, stream=None) -> None:
    if _bf16(x):  # bfloat16: the GEMV to 16 rows, the GEMM above
        fn = _lib.kq_qmv_bf16 if x.shape[0] <= 16 else _lib.kq_qmm_bf16
        _check(fn(_codec(codec), _ptr(w), n, k, _ptr(x), x.shape[0], _ptr(y), _dtype_id(y), _stream(stream)))
        return
    _check(_lib.kq_quantized_matmul(_codec(codec), _ptr(w), n, k, _ptr(x), x.shape[0], _ptr(y), _dtype_id(y),
                                    _stream(stream)))


def kq_quantized_matmul_residual(codec, w, n: int, k: int, x, residual, y, gate=None, stream=None) -> None:
    """y = residual + gate * (x @ dequant(w)^T).  residual, y [M, n]; gate None, [n] or [G, n] (G rows, one per
    M / G consecutive rows), all three in y's dtype.  residual may be y itself."""
    gate_rows = 0 if gate is None else gate.numel() // max(n, 1)
    _check(_lib.kq_quantized_matmul_residual(_codec(codec), _ptr(w), n, k, _ptr(x), x.shape[0], _ptr(residual),
                                             _ptr(gate), gate_rows, _ptr(y), _dtype_id(y), _stream(stream)))


def kq_quantized_matmul_qmv_bias(codec, w, n: int, k: int, x, bias, y, stream=None) -> None:
    """y = x @ dequant(w)^T + bias for one row of x; bias [n] in y's dtype."""
    _check(_lib.kq_quantized_matmul_qmv_bias(_codec(codec), _ptr(w), n, k, _ptr(x), x.shape[0], _ptr(bias), _ptr(y),
                                             _dtype_id(y), _stream(stream)))


def kq_quantized_matmul_glu(codec, w_gate, w_up, n: int, k: int, x, y, act="silu", stream=None) -> None:
    """y = act(x @ dequant(w_gate)^T) * (x @ dequant(w_up)^T); act 'silu' or 'gelu_tanh' (or a KQ_GLU_* id)."""
    a = _GLU_ACTS[act] if isinstance(act, str) else int(act)
    _check(_lib.kq_quantized_matmul_glu(_codec(codec), _ptr(w_gate), _ptr(w_up), n, k, _ptr(x), x.shape[0], a,
                                        _ptr(y), _dtype_id(y), _stream(stream)))


def kq_expert_tile_map(sorted_ids, n_experts: int, map_, counts, status=None, stream=None) -> None:
    """sorted_ids uint32 (int32 storage) [rows]; map_ [cap, 3]; counts [1]; status [1] or None."""
    _check(_lib.kq_expert_tile_map(_ptr(sorted_ids), sorted_ids.numel(), n_experts, _ptr(map_), _ptr(counts),
                                   map_.shape[0], _ptr(status), _stream(stream)))


def kq_gather_qmm_seg(codec, w, n_experts: int, n: int, k: int, x, map_, counts, y, stream=None) -> None:
    """w uint8 [E, n, row_bytes]; x float16 or bfloat16 [rows, k] expert-sorted; y [rows, n]."""
    fn = _lib.kq_gather_qmm_seg_bf16 if _bf16(x) else _lib.kq_gather_qmm_seg
    _check(fn(_codec(codec), _ptr(w), n_experts, n, k, _ptr(x), x.shape[0], _ptr(map_), _ptr(counts), map_.shape[0],
              _ptr(y), _dtype_id(y), _stream(stream)))


def kq_gather_qmv(codec, w, n_experts: int, n: int, k: int, x, ids, y, stream=None) -> None:
    """w uint8 [E, n, row_bytes]; x float16 [rows, k]; ids int32/uint32 [rows]; y [rows, n]."""
    _check(_lib.kq_gather_qmv(_codec(codec), _ptr(w), n_experts, n, k, _ptr(x), _ptr(ids), x.shape[0], _ptr(y),
                              _dtype_id(y), _stream(stream)))


def kq_moe_glu_gather(codec, gate_w, up_w, n_experts: int, n: int, k: int, x, ids, y, act="silu",
                      limit: float = 0.0, stream=None) -> None:
    """gate_w, up_w uint8 [E, n, row_bytes]; x float16 [T, k]; ids int32/uint32 [T, R]; y [T * R, n] (or
    [T, R, n]).  act: 'silu', 'gelu' (tanh form) or 'silu_limit', or a KQ_GLU_* id."""
    a = _GLU_ACTS[act] if isinstance(act, str) else int(act)
    top_k = ids.shape[1] if ids.dim() > 1 else 1
    _check(_lib.kq_moe_glu_gather(_codec(codec), _ptr(gate_w), _ptr(up_w), n_experts, n, k, _ptr(x), x.shape[0],
                                  _ptr(ids), top_k, a, float(limit), _ptr(y), _dtype_id(y), _stream(stream)))


def kq_gather_mix(y, inv_order, scores, out, stream=None) -> None:
    """y [rows, n] (float16/float32, routing-sorted rows); inv_order int32/uint32 [T * k]; scores float32 [T, k];
    out [T, n] of y's dtype."""
    if out.dtype != y.dtype:
        raise TypeError("out must have y's dtype")
    tokens, top_k = scores.shape
    _check(_lib.kq_gather_mix(_ptr(y), y.shape[0], y.shape[1], _ptr(inv_order), _ptr(scores), tokens, top_k,
                              _ptr(out), _dtype_id(out), _stream(stream)))


def kq_quantize(codec, w, out, stream=None) -> None:
    """w float32 [rows, k] -> out uint8 [rows, row_bytes]."""
    rows, k = (w.shape[0], w.shape[1]) if w.dim() > 1 else (1, w.shape[0])
    _check(_lib.kq_quantize(_codec(codec), _ptr(w), rows, k, _ptr(out), _stream(stream)))


def kq_stream_read(src, out, nbytes: int | None = None, stream=None) -> None:
    """Plain read of src's bytes (a multiple of 16) by out.numel() // 4 workgroups; out int32/uint32 [4 * groups]
    (one word per wave)."""
    nb = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(_lib.kq_stream_read(_ptr(src), nb, _ptr(out), out.numel() // 4, _stream(stream)))


# ---------------------------------------------------------------------------
# allocating conveniences (torch allocates; the library computes)
# ---------------------------------------------------------------------------

def dequantize(codec, w, k: int, dtype=None):
    import torch

    out = torch.empty((w.shape[0], k), dtype=dtype or torch.float16, device=w.device)
    kq_dequantize(codec, w, k, out)
    return out


def quantized_matmul(codec, w, n: int, k: int, x, out_dtype=None):
    import torch

    y = torch.empty((x.shape[0], n), dtype=out_dtype or x.dtype, device=x.device)
    kq_quantized_matmul(codec, w, n, k, x, y)
    return y


def quantize(codec, w):
    import torch

    out = torch.empty((w.shape[0], kq_row_bytes(codec, w.shape[1])), dtype=torch.uint8, device=w.device)
    kq_quantize(codec, w, out)
    return out


def expert_tile_map(sorted_ids, n_experts: int):
    import torch

    cap = kq_expert_tile_map_capacity(sorted_ids.numel(), n_experts)
    map_ = torch.empty((max(cap, 1), 3), dtype=torch.int32, device=sorted_ids.device)
    counts = torch.empty((1,), dtype=torch.int32, device=sorted_ids.device)
    kq_expert_tile_map(sorted_ids, n_experts, map_[:cap] if cap else map_, counts)
    return map_, counts
