"""fp64 CPU oracle for staged beam-search decode attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP library never routes through it, and it never imports
the HIP library: the two share no code. Only the seeded input generator
(``generative_recommendation_beam_amd.inputs``) feeds both.

Modules:
  attention  plain single-softmax attention over each beam's concatenated
             (prompt + generated-history) key sequence; stage special cases;
             log-sum-exp merge.
  append     reference semantics of the token-granular cache update.
  beam_topk  reference semantics of beam-search survivor selection (the n_out
             best candidates by score, index tie-break).
  cht        Feather's batch-forming structure by brute force (missing
             counts from direct token comparison).
  pool       process-pool driver used to time the oracle on many cores.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
a library special case (torch scaled_dot_product_attention in fp64 on CPU),
closed forms and invariants. No function is "parity unpinned".
"""
