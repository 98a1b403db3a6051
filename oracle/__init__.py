"""CPU oracle for fine-grained block-scaled FP8 quantization and GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code, header, table or constant with
the HIP library in ``fine_grained_block_fp8q_amd/``; every constant (the E4M3
value set, 448, the group sizes) is re-derived here from the format and method
definitions.

Sources (web pages, cited by page and passage; the pages carry no section
numbers, so the passage is named by topic):

* [goodkr-2169793] the-good.kr free board post 2169793 -- the mixed-precision
  framework and fine-grained quantization passages (E4M3 on all tensors; online
  max-abs per 1x128 activation tile / 128x128 weight block; scale the max-abs to
  the largest FP8 value; per-group scaling along K, dequantized on the general
  ALUs), and the limited accumulation bit-width passage.
* [whybe-57820] why-be.co.kr as_center post 57820 -- the promotion passage
  (partial results copied out of the matrix unit every N_C interval, multiplied
  by the scaling factors, added into FP32 registers) and the hardware
  suggestion of higher-precision FP8 accumulation inside the matrix units.
* [pkd-78017] pkd.ac.th webboard post 78017 -- the increased-precision
  accumulation passage (128 elements, i.e. four WGMMAs, is the smallest
  promotion interval that helps).
* [whybe-72410] why-be.co.kr as_center post 72410 -- the fixed-point accumulation
  passage (products aligned to the largest exponent by sign-fill right shift,
  only the top 14 bits kept) and the power-of-two scaling passage.

Modules:
  e4m3        OCP E4M3 (E4M3FN) decode table and round-to-nearest-even encoder
  quant       1x128 activation / 128x128 weight quantizers (FP32 and pow2
              scales), their transposed forms for the backward GEMMs, and
              per-tensor scaling (accuracy study)
  gemm        block-scaled GEMM with per-128-K promotion, exact in float64; the
              variant with row-group scales on both operands (weight gradient);
              the BF16 reference product
  mfma_model  model of the gfx950 FP8 matrix core's dot product (a diagnostic)
              and the truncation term T of the fast GEMM's a-priori bound, also
              evaluated by a plain C loop (truncation_bound.c) for full-size
              matrices
  native      builds and loads that C loop (libtbound.so)
  narrow_acc  emulator of a narrow fixed-point accumulator (accuracy study)
"""

from . import e4m3, quant, gemm, narrow_acc  # noqa: F401
