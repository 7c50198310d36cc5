"""CPU oracle for GQLA decode attention -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct fp64 reference of what the
decode path computes.  It exists to check the HIP library, never to stand in
for it: only the test-suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it.  It shares no code with the
HIP path (``decode_attention_gqla_amd``) and imports nothing from it.

Sources (the GQLA pages: "GQLA: Group-Query Latent Attention for
Hardware-Adaptive Large Language Model Decoding", arXiv 2605.15250):

* paperlayer.ai summary, section 3 "Methods", bullet "Architecture": the latent
  ``c^KV_t`` is expanded into ``g`` grouped K/V representations of per-head
  dim ``d_h``; queries have ``h_q`` heads with decoupled-RoPE parts ``q^R_h``
  and one shared ``k^R``.
* same page, section 3, bullet "Two equivalent decoding paths": the GQA form
  materialises the ``g`` K/V groups; the MQA-absorb form folds the
  up-projections into Q/O and attends over the latent cache.
* gist.science technical summary, section 2 "Methodik", "Architektur": the
  up-projections ``W_UK``, ``W_UV`` are indexed by group instead of being
  replicated per query head.

Modules:

* ``gqla_ref`` -- numpy fp64: literal decode, absorb-form decode, GQA over a
  stored expanded cache, split partials, log-sum-exp merge, cache expansion
  (with bf16 round-to-nearest-even of its output), bf16 rounding.
* ``brute``    -- pure-Python scalar loops (math.fsum / math.exp) of the
  literal decode, for tiny inputs.

Parity status of each function is stated in its docstring; every function is
pinned by ``tests/test_oracle_*.py`` against brute force, a library routine,
closed forms or special cases.
"""
