"""CPU oracle for one TMP shard of a transformer layer stack run through the
Oases overlapped schedule with fine-grained recomputation.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the tests, the graft smoke entry and the benchmark's
CPU-baseline leg do.  It shares no code with the GPU library; the one module
both sides use is ``gen`` (seeded inputs, no arithmetic of the method).

Source: "Oases: Efficient Large-Scale Model Training on Commodity Servers via
Overlapped and Automated Tensor Model Parallelism" (arXiv 2305.16121, HTML
version), Section IV (the overlapped training schedule, Eq. (1), Fig. 4,
Algorithm 1).  The layer arithmetic is the plain definition of a
Megatron-style column-parallel / row-parallel shard, written out in float64.

Modules:
  blocks    -- GeLU, causal attention, FFN / attention shard forward and
               backward, the AllReduce point (fp64)
  schedule  -- op lists of the four schedules and a step simulator that keeps
               only what each schedule stores
  sums      -- the AllReduce-point sum in the storage type, accumulated
               sequentially in float32 (the bit-exact reference for the GPU
               sum kernel)

Parity status: every function is pinned by tests under ``tests/`` marked
"not gpu" (closed forms, brute force, finite differences, invariants);
nothing here is "parity unpinned" except that the pages print no numeric
example, so no check compares against a value printed on the pages.
"""
