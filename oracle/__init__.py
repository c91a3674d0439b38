"""The oracle: a plain, slow, CPU-only statement of what the kq hot path computes.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it. The product
path (the HIP library and its Python binding) never imports it, never links it
and never falls back to it.

It shares no code with the HIP path: no kernels, headers, helpers, tables or
constant generators. It is written from the pages' statement of the problem
(sources below) plus the readings listed in each function's docstring.

Sources (cited by page title and section in every docstring):
  * mlx-kquant README (package METADATA page): "Codec reference" table
    (values per block, bits, bytes per block) and "Using K-quant ops directly".
  * mlx-kquant ``bindings.cpp`` page: the ``dequantize``, ``quantized_matmul``,
    ``gather_qmm``, ``expert_tile_map``, ``gather_qmm_seg`` and ``quantize``
    docstrings.
  * nuvec-core ``quantized.rs`` page: the module comment's affine closed form
    and the ``gather_qmm`` semantics.
  * hanzo-ml ``quantized/mod.rs`` page: ``moe_grouped_per_expert`` (group
    routed rows by expert, one product per expert, scatter back).

Pins (what each function is checked against in ``tests/``, independent of the
oracle's own code) are listed in each module's header. Parity status:
  * codecs.decode_* / dequantize: pinned (hand-decoded superblocks in
    tests/golden, binary16 library decode, MLX affine closed form, byte totals
    from the codec table).
  * encode.*: pinned (brute-force nearest grid point on tiny tensors, q8_0
    error bound d/2, decode-then-encode fixed point).
  * matmul.*: pinned (exact rational arithmetic on tiny shapes, one-hot rows).
  * tilemap / gather: pinned (brute-force invariants, hand example, reduction
    to a plain per-expert loop and to qmm with one expert).
  * Interop with GGUF files written by other tools: parity unpinned (no GGUF
    file or gguf package is available to check the byte layout against).
"""

from . import codecs, encode, matmul  # noqa: F401
