"""Tolerance bars of the fp16-intermediate GPU tests, each set from the
error that tests/rounding_model.py (a float64 model of exactly the roundings
the fp16 path makes) shows on the same inputs.  tests/test_rounding_model.py
recomputes every emulated error below on the CPU and checks that each bar
is about twice it (between 1.5 and 3 times).  The smaller fp16 tests need no
constant: they compute twice the model's error on their own inputs
(rounding_model.core_bar).

Metric: max |out - ref| / RMS(ref) against the float64 oracle.
"""

# mha_forward, bf16 inputs, fp16 intermediates, at B=4, T=4096,
# d_model=1024, h=16, d_h=64, causal: the model's error on batch item 0.
HEADLINE_MODEL_ERR_ITEM0 = 1.490e-2

# attn_core on the headline's fp16 heads with fp16 Z (the benchmark's launch
# configuration): the model's largest error over the four batch items, and
# the bar.
HEADLINE_CORE_MODEL_ERR = 1.364e-2
F16_CORE_HEADLINE_BAR = 2.8e-2
# The same heads through the exact-shift form (the kernels that take a
# boolean mask or an additive bias): the model's largest error over the four
# items (item 0).  The headline core bar covers it too.
HEADLINE_CORE_EXACT_MODEL_ERR = 1.330e-2


# Backward of the attention core (normwise ||err|| / ||ref||, max-normalised
# max|err| / max|ref|), per element type of the heads.  The backward's
# rounding model (rounding_model.attn_core_grad_model) gives, over the
# backward test cases (tests/bwd_cases.py), at most 2.51e-3 / 3.76e-3 (bf16)
# and 3.38e-4 / 6.18e-4 (fp16); tests/test_kernel_emulations.py recomputes
# them and checks that each bar is 1.5 to 3.5 times the model's error.
BWD_TOL = {"bf16": (5e-3, 1e-2), "f16": (1e-3, 2e-3),
           # fp32 heads (vector-ALU kernels, nothing rounded below fp32): the
           # fp32 bar of the forward
           "f32": (1e-4, 1e-4)}
