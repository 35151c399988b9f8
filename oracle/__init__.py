"""Plain, slow CPU oracle for the drafter LM head and speculative verification.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.  The
product path (the HIP library and its Python binding) never imports it, and this package
never imports the product path.  The two share no code; they only receive the same seeded
inputs from the input generator module, which holds none of the method's arithmetic.

Everything is NumPy on the host, accumulated in float64.  bf16 inputs are decoded exactly
(bf16 -> fp32 -> fp64 is lossless).  Each function cites the passage of the source pages
it follows:

* "SlimSpec" write-up (mhpn.cn, "荷兰Nebius团队：给AI起草员瘦身"), sections 三 (low-rank
  head), 四 (acceptance ceiling), 一 (round structure).
* "SpecVocab" write-up (2kiu.com), sections 2.2.1-2.2.3 (scorer, top-k, exact logits)
  and 3.3 (verification keeps the full vocabulary).
* "投机解码讲人话" explainer (liuchunshan.com), sections "小模型起草，大模型批改" (greedy
  verification), "为什么答案不会变" (rejection sampling, residual, distribution
  preservation) and "这笔账划不划算，看一个数" (closed-form tokens per step, table for
  gamma = 4).
* "SpecTr-GBV" write-up (hypresin.com), "为什么重新设计推测解码的验证环节" and "第三步"
  (first rejection ends the block; residual next token; bonus token when all accepted).
* Phrase-level speculation page (kongchang.com), "更换单元：从 token 到短语" (candidates in a
  prefix tree verified in one pass, kept only where they equal the target's argmax).

Parity status: every function here is pinned by a CPU test against something other than
itself (library routines it does not call, brute force, closed forms, the pages' printed
table, Monte Carlo against exact distributions).  No function is "parity unpinned".
"""

from . import fp, philox, sampler, heads, verify, tree  # noqa: F401
