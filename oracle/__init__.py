"""CPU oracle for the speculative-decoding verify step -- TEST INFRASTRUCTURE.

This package is a plain, slow, deliberately obvious float64 restatement of
what the verify step computes.  It exists to check the GPU library and to be
timed as a CPU baseline.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(the HIP library and its Python binding) never does, and this package never
imports the product.

Pages followed (title, section):

* "投机推理算法的常见优化手段" (cnblogs) -- section on verifying the draft
  tree with a tree mask: flattening, the ancestor mask and its printed 6x6
  matrix, the per-node distribution P(i | ancestors(i)), level-by-level
  verification.  -> ``tree``, ``attention``, ``accept``.
* "【模型后训练与深度推理】9 推理加速：推测解码与级联推理" (CSDN) -- section
  7.1 (acceptance probability min(1, p/q), resampling from norm(max(0,p-q))),
  section 7.2 (expected emitted length).  -> ``accept``.
* guijiagi.com post on speculative decoding -- section on the mathematical
  basis (rejection sampling, stop at the first rejection) and section on KV
  cache management (roll back rejected tokens' KV).  -> ``accept``, ``kv``.
* "万字综述 10+ 种 LLM 投机采样推理加速方案" -- section 5.2 (tree-based
  parallel decoding equals sequence-based decoding), section 4.3 / 8.1
  (argmax sampling at temperature 0, longest matching prefix).
* "投机推理算法的常见优化手段" (cnblogs) -- draft-tree generation (EAGLE-2
  expansion of the most probable leaves) and dynamic draft length (ECHO's
  global budget and checkpoints).  -> ``draft``.
* "投机推理算法的常见优化手段" (cnblogs) tree-mask section, and the survey
  page's Medusa / EAGLE sections (the original LM head after the last layer)
  -- the target LM head that produces every tree row's logits.  -> ``lm_head``.

Readings of the pages where they are silent or garbled are listed in the
module that takes them.  Every function here is pinned by the CPU tests
against printed values, closed forms, library routines or brute force,
except where a module header says "parity unpinned".
"""
from . import philox, tree, attention, accept, kv, draft, lm_head  # noqa: F401
