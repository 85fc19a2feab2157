"""CPU oracle for DiffusionGemma-style block diffusion decoding.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It is a plain, slow,
float64 NumPy implementation of what the denoise step, the denoise loop and
the causal commit pass compute; it shares no code with the HIP library and
imports nothing from it.

What each function follows (pages: the four DiffusionGemma pages; sections
named by their headings):

* ``philox``   counter-based Philox4x32-10 (Salmon et al., "Parallel Random
  Numbers: As Easy as 1, 2, 3", SC 2011) for canvas initialisation and
  re-noising; uniform-state noise (zhichai.net 深度拆解, "统一状态扩散";
  DiffusionGemma解析, "整片并行去噪").
* ``numerics`` bfloat16 round-to-nearest-even and OCP E4M3FN decoding.
* ``model``    the backbone step (bidirectional attention over prompt KV plus
  canvas: DiffusionGemma解析 "整片并行去噪", zhichai.net "双向注意力"; MoE with
  128 experts, top-8 and a shared expert: zhichai.net "MoE 效率"), per-position
  entropy and argmax confidence, entropy-ranked commit and re-noising
  (DiffusionGemma解析 "整片并行去噪"; ipcmen.com "工作原理"), the 48-step cap
  (DiffusionGemma解析 "自适应停步机制"), and the causal append of a committed
  canvas to the KV cache (zhichai.net "Block-Autoregressive").

Parity pins live in ``tests/test_oracle_*.py``.  Unpinned: the pages' trained
statistics (about 12 steps per generation, 19.74 tokens per step) cannot be
reproduced with synthetic weights, so nothing here claims them.
"""
from . import numerics, philox, model  # noqa: F401
