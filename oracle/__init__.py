"""CPU oracle for prefix-tree-packed causal attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct reference implementations of what the GPU path
computes: the radix segment build and best-fit-decreasing row packing
(``oracle.packer``), the token-forest attention mask and tile classes
(``oracle.mask``), masked softmax attention in float64, forward and gradients
(``oracle.attention``), rotary embedding at tree positions (``oracle.rope``) and the
gated delta rule threaded along the token tree (``oracle.gdn``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the C-ABI library and
its Python binding) never imports it, and this package imports nothing from the
product: the two share no code.  The only shared module is the seeded input
generator ``workloads``, which holds none of the method's arithmetic.

Sources, cited in each function by page title and passage:
  [PTP]   "Prefix tree packing" post, furtherai.github.io/blog/posts/prefix-tree-packing
  [AReaL] "How to Configure Sequence Packing for Efficient GPU Utilization in AReaL"
  [AOM]   "ART-Optimized Megatron (AOM): 12x higher training throughput" (CoreWeave blog)

Parity status: every function here is pinned by a ``-m "not gpu"`` test against
something other than itself (worked examples printed on the pages, closed forms,
library routines, brute force, independent algorithms).  None is "parity unpinned".
"""
from . import packer, mask, attention, rope, gdn  # noqa: F401
