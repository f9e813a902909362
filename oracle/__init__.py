"""CPU oracle of the DeepSeekMoE layer forward: TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import anything here.  The product path (the HIP library and
its Python binding) never imports, links or runs it.

Modules:
  e4m3  - E4M3FN codec and tile/block quantiser, written from the format's
          field definitions.
  moe   - routing (sigmoid affinity, bias-steered top-K, normalised gates,
          loads), SwiGLU experts, combine, bias rule and the expert-contiguous
          layout definition, all in fp64.

Every function is pinned by tests under `tests/` (test_oracle_*.py) against
brute force, closed forms, invariants or an independent library routine.
"""
from . import e4m3, moe  # noqa: F401
