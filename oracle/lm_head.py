"""Target logits from the LM head, written plainly, for the fused verification.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing in the product
path imports it.  It shares no code with the HIP library.

Sources (page title and section):

* [TB] tbxsx.cn, "推测解码采样验证优化策略 —— 深度调研报告", section
  "6. 扩展性与安全性": fuse the verification-stage forward pass of the target
  model with the sampling step.  Section "3. 数学形式化": the target
  distribution is softmax(logits / T) of the target model's logits.

Reading: the pages do not write the last layer out.  The logits of a
position are the product of that position's final hidden state with the
LM-head weight matrix, logits[m][v] = sum_d hidden[m][d] * weight[v][d],
and the verification consumes them as bfloat16 values (the precision of the
logits it is given elsewhere), i.e. the exact product rounded to the nearest
bfloat16, ties to even.

Functions:

* ``round_bf16(x)``: float64 -> nearest bfloat16 value (as float64), ties to
  even, from the definition: an 8-bit significand.
* ``bf16_bits(y)``: bfloat16 values -> their 16-bit patterns.
* ``lm_head_logits(hidden_bits, weight_bits)``: the float64 product of the
  widened inputs (one library matmul); exact when every product and partial
  sum fits float64's significand, as for small-integer inputs.
* ``lm_head_target_bits(hidden_bits, weight_bits)``: the bfloat16 logits the
  verification reads, as bit patterns.

Pinned by ``tests/test_oracle_lm_head.py`` against brute-force sums, worked
rounding cases and an exhaustive nearest-value search.
"""

import numpy as np


def widen_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64 values, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(x):
    """Nearest bfloat16 value of each float64 in ``x``, ties to even.

    x = f * 2**e with 0.5 <= |f| < 1 (frexp); a bfloat16 keeps 8 significant
    bits, so the rounded value is round_half_even(f * 2**8) * 2**(e - 8).
    Finite inputs of bfloat16's normal range only.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    r = np.round(f * 256.0)                 # numpy rounds halves to even
    return np.ldexp(r, e - 8)


def bf16_bits(y):
    """Bit patterns of values that are bfloat16 (e.g. ``round_bf16`` output)."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    if not np.array_equal(y32.astype(np.float64), np.asarray(y, dtype=np.float64)):
        raise ValueError("not bfloat16 values")
    b = y32.view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("not bfloat16 values")
    return (b >> np.uint32(16)).astype(np.uint16)


def lm_head_logits(hidden_bits, weight_bits):
    """logits[..., v] = sum_d hidden[..., d] * weight[v, d] in float64.

    hidden_bits [..., D], weight_bits [V, D]: bfloat16 bit patterns.
    """
    h = widen_bf16(hidden_bits)
    w = widen_bf16(weight_bits)
    D = h.shape[-1]
    out = h.reshape(-1, D) @ w.T
    return out.reshape(h.shape[:-1] + (w.shape[0],))


def lm_head_target_bits(hidden_bits, weight_bits):
    """The target logits as the verification reads them: bfloat16 bit patterns."""
    return bf16_bits(round_bf16(lm_head_logits(hidden_bits, weight_bits)))
