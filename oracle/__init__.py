"""CPU oracle for weight-only quantized decode linear layers.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library: no kernels, headers, helpers, tables or constants.

What it computes, and where each step comes from:

* ``quant.quantize_int8_b32`` -- int8 symmetric absmax quantization per block
  of 32 consecutive weights along K with one fp16 scale per block.  The pages
  name this format ("int8 per-block-32 body + untied absmax int8 head") on the
  Qwen3-VL 4B/8B Core AI cards (Files table) and the zoo's Qwen3-VL page
  (Measured paragraph); the zoo's Qwen3.8-27B page (Numerics paragraph) names
  the "absmax symmetric per-block-32 head rule" and says clipping must not be
  used for the head.  Divisor 127 and fp16 scales are the workload definition.
* ``quant.quantize_int4_g64`` -- 4-bit per-group-64 quantization, named by the
  CoreML-LLM handoff page (Architecture: "INT4 per-grouped-channel, group_size
  64"); the affine form (fp16 scale + fp16 min, 8 codes per uint32) is the
  workload definition.
* ``layout`` -- this library's tiled byte layout, rewritten here from its
  prose specification with numpy reshapes (no index arithmetic is shared with
  the HIP packer).
* ``glue`` -- the element-wise steps either side of the projections: the
  RMSNorm that feeds q|k|v and gate|up, and the SwiGLU that feeds down (zoo
  Qwen3-VL page, Architecture paragraph, names a Qwen3 decoder with a SwiGLU
  MLP; the formulas and the fp16 rounding points are readings).
* ``linear`` -- the result: dequantize, then multiply, in fp64.  Decode is
  bandwidth-bound because every weight is read once per token (Core AI cards,
  Measured paragraph); the arithmetic is the plain matrix-vector product.

Readings of points the pages leave open are listed in each function's
docstring.  Functions whose agreement with the pages rests only on such a
reading are marked "parity unpinned" (the tiled layout, the INT4 format, the
glue formulas and their fp16 rounding points).
"""
from . import quant, layout, glue, linear  # noqa: F401
