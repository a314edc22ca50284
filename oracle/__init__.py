"""CPU fp64 oracle for the Mamba-2 SSD forward pass.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything
in this package. The product path (the HIP library and its Python binding)
never routes through it, and this package imports nothing from the product.

Two implementations, written independently of each other and of the HIP
kernels:

* ``ssd_sequential`` -- the token-by-token recurrence, the plain definition.
* ``ssd_chunked``    -- the chunk-wise "jump" evaluation through log-space
  cumulative decays, in natural ``exp`` (no base-2 rescaling).
* ``ssd_step``       -- one token of the recurrence for every sequence and
  head (the decode step), updating a given state.
* ``ssd_bwd_sequential`` / ``ssd_bwd_chunked`` -- every input's gradient
  (the backward pass), by reverse mode through the token recurrence and from
  the chunked form, independently of each other (``ssd_bwd.py``; pinned in
  ``tests/test_oracle_bwd.py``).
* ``s6_sequential`` -- the Mamba-1 selective scan (S6) token by token, the
  family's second member (``s6.py``; pinned in ``tests/test_oracle_s6.py``),
  and ``s6_bwd_sequential``, its every-input gradient by reverse mode through
  the same recurrence (pinned in ``tests/test_oracle_s6_bwd.py``).

Both upcast every input to float64 and never round to a narrower type.

Source: NVIDIA developer blog, "Accelerating Mamba-2 with high-performance
forward-pass kernels in NVIDIA CUDA Tile" (Korean edition, and its Chinese
copy on everytik.com), section "Mamba-2 architecture" and its equations and
Figs. 1-4; section "Kernel 1" for the chunk-local cumulative sum. Pins that
tie both functions to facts fixed outside this package live in
``tests/test_oracle_pins.py``; every function here is pinned there.
"""
from .ssd_seq import ssd_sequential, heads_to_groups
from .ssd_chunked import ssd_chunked
from .ssd_step import ssd_step
from .ssd_bwd import ssd_bwd_chunked, ssd_bwd_sequential
from .s6 import s6_bwd_sequential, s6_sequential

__all__ = ["ssd_sequential", "ssd_chunked", "ssd_step", "heads_to_groups", "ssd_bwd_sequential",
           "ssd_bwd_chunked", "s6_sequential", "s6_bwd_sequential"]
