"""Acceptance tolerances for the HIP path against the FP64 oracle.

Max-abs error on O: 4e-3 for fp16 inputs, 1.6e-2 for bf16 inputs; on the
natural-log LSE: 1e-3.  Row softmax (fp32): max-abs 1e-6, the pass threshold
of the softmax kernel study (lpnh.cn/news/2830604, section 3.2), and every
row sums to 1 within 1e-5.
"""
ATTN_O = {"f16": 4e-3, "bf16": 1.6e-2}
ATTN_LSE = 1e-3
SOFTMAX_Y = 1e-6
SOFTMAX_ROWSUM = 1e-5

# Attention backward: no tolerance is given for it, so this is an empirical
# margin, not a derived bound.  What the arithmetic fixes: P and dS are
# rounded to the input dtype (unit roundoff u = 2^-11 for fp16, 2^-8 for
# bf16) before the FP32-accumulated products, which perturbs each term of the
# dV, dK and dQ contractions by at most about 2u relative.  What is assumed:
# that the sum of a gradient entry's absolute terms stays within 2x of the
# largest gradient entry (cancellation can break this), which gives
# max |G - G_ref| <= 4u * max(1, max |G_ref|); measurement, not proof,
# supports it.
BWD_REL = {"f16": 4 * 2.0 ** -11, "bf16": 4 * 2.0 ** -8}
