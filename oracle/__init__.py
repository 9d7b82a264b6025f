"""CPU oracle for the extended-EinSum / tensor-relational-algebra path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this
package; only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import, call or link it.  It shares no code, header,
table or helper with the HIP path.

Modules:
  ref       -- the definition: a nested-loop C implementation (einsum_ref.c,
               fp64/int64, OpenMP over output elements), a pure-Python brute
               force for tiny shapes, and a numpy full-index-space evaluator.
  tra_cpu   -- tensor-relational algebra taken literally: tensors cut into
               {key: sub-tensor} dictionaries by the partition rule, join of
               key-matched pairs, group-by aggregation, repartition, and the
               flat relation buffer layout.
  chooser   -- the communication cost model and an exhaustive search over
               partition vectors for small EinGraphs.
  mha       -- the multi-head-attention EinGraph evaluated in fp64.

Sources: the page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法"
(sections 2.1, 2.2, 3.1, 3.2) and, for the blocked GEMM, the page
"ColossalAI 2.5D 张量并行深度解析" (section on the 2.5D partitioning of Y = XA).
"""
