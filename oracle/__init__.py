"""CPU oracle for the TetraJet-v2 NVFP4 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything under ``oracle/``; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, table or constant generator with the
HIP path.

The oracle is plain numpy: every fp32 step is a numpy float32 operation (IEEE
round-to-nearest per operation, no contraction, subnormals kept), fp64 where
stated.  It follows the method as the pages describe it:

* double-block NVFP4 quantization (E2M1 elements, an 8-bit scale per 16
  elements, an FP32 scale per 128-element outer block), round-to-nearest in
  the forward pass and stochastic rounding in the backward pass, weights in
  1x16 groups with a re-grouped transpose
  -- TetraJet-v2 technical summary, section 2.A;
* a random Hadamard transform on the operands of the dX and dW products and
  static FP8 retention of the top-p% channels -- section 2.C (OutControl);
* OsciReset: oscillation risk as the ratio of the distance travelled by the
  quantized weight to that of the master weight, with a reset to the centre
  of the current bin -- section 2.B.

Where the pages leave a step open, the reading taken is stated in the
function's docstring.  Pins (tests/test_oracle_*.py) tie every function to
something other than itself: library routines (numpy rounding, torch's
float8_e4m3fn conversion, scipy's Hadamard matrix, rocrand's Philox), closed
forms, invariants and brute force on tiny inputs.

Modules
-------
formats   E2M1 and E4M3FN encode/decode, element RTN and SR rules
philox    Philox4x32-10 (scalar and vectorised), per-element 16-bit draws
rht       16-wide random Hadamard transform
quant     double-block NVFP4 and per-128 FP8 quantizers, dequantization
gemm      fp64 reference GEMMs on dequantized operands
linear    forward / backward composition of the linear layer (+ OutControl)
osci      OsciReset state update
calib     OutControl calibration (channel scores, top-p selection)
"""
