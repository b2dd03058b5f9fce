"""Plain CPU oracle for the ring / tree collectives.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constant generators) and does
not import it.

What it is: a literal, slow, step-by-step simulation of the schedules the pages
describe, written in NumPy on the host.  N logical ranks are N NumPy arrays.
Each simulated step first takes a copy of everything the ranks send (the
"send"), then applies every receive.  Floating point follows the dtype the
pages' per-hop ``+=`` implies (see ``numerics``); nothing is reordered, fused or
blocked beyond what the schedules state.

Sources (cited by page title and section):

* "第09讲：网络通信基础与集合通信 Collective 原语直觉" (Lecture 09, collective
  primitives), sections 3.1-3.9 (the primitives), 4.2-4.4 (ring), 5.2 (double
  binary tree), 7.1 (lab 1, the single-process ring simulation).
* "4. 通信模式：集合通信（AllReduce、AllGather等）原理与实现" (Chapter 4,
  communication patterns), sections 4.3.1 (ring pseudo-code) and 4.3.2 (tree).
* "从零实现集合通信" (Collectives from scratch), section "两趟实现 ring
  allreduce" (two-pass ring) and its per-primitive cost table.
* Lecture 09 sections 3.2-3.4 for Scatter, Gather and Reduce (each rank not
  named as receiving keeps its data), section 3.8 and lab 4 (section 7.4)
  for AllToAll.

Pins (what the oracle is checked against in ``tests/test_oracle_*.py``):
int32 brute force, hand-derived order-revealing fp32 examples, the worked
examples the pages print, an independently written 0-based schedule from the
Lecture 09 lab / Chapter 4 pseudo-code on rotated ranks, the exactly rounded
sum (``math.fsum``) within the recursive-summation bound, the pages' byte and
step counts, torch's CPU bfloat16 conversion, the order-free maximum and
minimum over the rank axis for MAX and MIN, the per-element fold order for
PROD, and planted mistakes that each of these must catch.  Two readings are this
package's own because the pages leave them open: the ragged chunk layout and
the double-tree shape and split.  No page value can fix them; the oracle's
implementation of each is pinned independently (chunks covering every element
once in rank order, int32 brute force on ragged shapes, the binomial recursion
evaluated directly on each half, the pages' n=3 and n=4 pairing examples and
the cost table's per-rank bytes).
"""

from .numerics import (  # noqa: F401
    DTYPES,
    ITEMSIZE,
    OPS,
    STORAGE,
    bf16_to_f32,
    combine,
    f32_to_bf16_rne,
)
from .collectives import (  # noqa: F401
    Result,
    alltoall,
    broadcast,
    ceil_log2,
    chunk_layout,
    gather,
    reduce,
    ring_allgather,
    ring_allreduce,
    ring_reduce_scatter,
    scatter,
    tree_allreduce,
)
