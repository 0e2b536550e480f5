"""CPU oracle for block-scaled quantized matmul.  TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written reference that every GPU result is
checked against.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import it; the library's product path never does,
and this package imports nothing from the library (the two share no code).
The only thing both sides use is the seeded input generator in ``synth``.

What it computes, and the page passage each part follows:

* ``formats``   fp8 e4m3fn / e5m2, e8m0 and bf16 codecs (the formats named in
                jax.nn.scaled_matmul's Notes and the NKI backward API's
                float8_dtype / output_dtype).  Encoding = nearest value of the
                format, ties to the even code, found by search over the table
                of the format's values.
* ``quantize``  the quantizers: 1 x 128 and 128 x 128 fp8 (atrex-bench
                block_scaled_mm, "Input Generation"), int8 per-channel
                (TensorTonic "Int8 Matmul with Per-Channel Scales", the scale
                and code formulas) and MX 32-element e8m0 blocks
                (jax.nn.scaled_matmul Notes, mxfp8; NKI backward, float8_dtype).
* ``matmul``    scaled_matmul (jax.nn.scaled_matmul, "Mathematically"), the
                2-D tiled block_scaled_mm (atrex-bench, "Reference
                Implementation"), the int8 per-channel matmul and its epilogue
                (TensorTonic, output formula and Requirements).
* ``backward``  dX = dY W and dW = dY^T X with on-the-fly MXFP8 quantization
                (NKI matmul_mxfp8_backward, opening paragraph and Parameters).

Precision: quantizers run in float32 exactly as the pages state them (numpy
float32 arithmetic is IEEE-754 round-to-nearest-even, division included);
matmuls accumulate in float64 (int64-exact for the int8 path).

Pins (tests/test_oracle_*.py, run with ``-m "not gpu"``): every function
here is pinned to something other than itself - printed worked examples,
closed forms, torch's CPU casts, exact rational brute force, and invariants
that a dropped term, wrong sign, wrong index or transposed operand breaks.
Parity status per function is listed in the module docstrings; the MX scale
rule is a reading (the pages do not state it) and its pins are invariants.
"""
