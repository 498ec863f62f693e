"""Plain, slow, fp64 CPU oracle for batched speculative-decoding verification.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import it: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels,
headers, helpers or constant tables) and imports nothing from the package.

Sources the oracle follows (cited by page title and section):

* [TB] tbxsx.cn, "推测解码采样验证优化策略 —— 深度调研报告" (research report on
  sampling verification): section "3. 数学形式化" (formulas 1, 3, 4) and
  section "4. 实现逻辑" (the ``_sampling_verification`` pseudo-code).
* [NW] nickwang.xyz, "推测解码：草稿、验证与实际加速" (notes on drafting,
  verification and real speed-up): sections "候选已知，验证才能并行"
  (position/logit alignment, bonus row, EOS), "接受与拒绝怎样保住分布"
  (equations a(x) and r(x)), "算完三个 token 的全部概率" (worked example and its
  exact-fraction replay) and "好草稿也要算得便宜" (acceptance rate, E[N]).
* [BZ] bowenzhou.top, "投机采样" (notes): sections "机制：起草-验证-接受",
  "收益账" and "深入推导" (distribution-preservation identity).

``oracle.round_policy`` holds the round statistics and the adaptive draft
length ([TB] "4. 实现逻辑"; [NW] "好草稿也要算得便宜").  ``oracle.lm_head``
holds the target logits of the verification fused with the LM head ([TB]
"6. 扩展性与安全性").

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, exact rational arithmetic or brute force.
"""

from .specverify_oracle import (  # noqa: F401
    ACCEPT_FLAG_REL,
    CDF_FLAG_REL,
    TOPP_FLAG_ABS,
    PATH_ERROR,
    PATH_REJECT,
    PATH_BONUS,
    PATH_EOS,
    FLAG_NONE,
    FLAG_ACCEPT,
    FLAG_CDF,
    FLAG_TOPP,
    FLAG_EMPTY_RESIDUAL,
    widen_row,
    topk_threshold,
    processed_distribution,
    accept_prob,
    residual,
    icdf,
    verify,
    expected_tokens_per_round,
    acceptance_rate,
    acceptance_rates,
)
