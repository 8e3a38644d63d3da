"""CPU oracle for blockwise causal attention, the log-sum-exp merge, the ring
and zigzag schedules and the Ulysses repacks.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: only the tests, the smoke check
of ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, constants or helpers with the HIP library; the only
common dependency is ``seeded_inputs`` (random draws, no arithmetic of the
method).

Pages followed (cited by title and section throughout):

* "上下文并行：Ring Attention 与 Ulysses" (Context parallelism: Ring
  Attention and Ulysses), AI-infra handbook, train/model/context -- the
  authority on what is computed.  Sections: "哪些运算可以直接切" (which
  operations split directly: ``attention()`` with offsets and LSE,
  ``make_qkv``), "Ulysses：在序列和头之间转置" (Ulysses: transposing between
  sequence and heads), "Ring Attention：KV 沿环传一圈" (Ring Attention: KV
  goes once around the ring), "之字形切分" (zigzag split) and "练习"
  (exercises: GQA with 32 query and 8 KV heads).
* "Sequence Parallel vs Context Parallel" blog (xxqk.cn), section 3.2
  "分布式softmax怎么合并" (how the distributed softmax is merged): the
  global-max form and the running (m, l, o) update.

Modules:

* ``attention``  -- the plain definition in float64 (numpy), the merge and
  the global-max route.
* ``schedules``  -- the splits, the work model, the ring loops and the
  Ulysses all-to-all on P virtual ranks (numpy).
* ``native``     -- ctypes binding of ``cp_oracle.c``: the same definition
  in plain C + OpenMP for rows of the large configurations.
"""
