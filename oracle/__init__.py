"""CPU oracle for int8-key / int4-value quantized-KV decode and verify attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the C-ABI library under
``decode_attention_quantized_kv_amd``) may import, call, link or execute
anything in this package. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.

What it computes (each module cites the passage it follows):

* ``oracle.codec``  -- the K8/V4 codec: per-token int8 keys with an fp16
  absmax scale, per-(token, 32-dim group) int4 values with an fp16 absmax
  scale, in plain fp32 numpy arithmetic, plus the paged cache byte layout.
* ``oracle.attention`` -- textbook softmax attention in fp64 over the
  dequantized cache, for one decode query per sequence and for a block of
  draft queries with causal masking among the drafts (speculative verify).

Sources: the codec is the one the blog post at blog.123qwe.co.kr/?p=3927
reports from the engine's load log in its section 5 (speculative decoding,
quantized KV and prefix sharing): a decode attention unit named
``attention_decode_k8v4``, keys at 8 bits, values at 4 bits in groups of 32
with an fp16 scale.  The Launch HN digest (trawling.dev/post/1715, section on
per-device tuning and performance claims) gives the same bit widths.  The
exact scale rule (symmetric absmax, round-half-even) is this repository's
reading of those passages, stated in ``oracle.codec``.

The oracle shares no code with the HIP path; the seeded input generators in
``workloads/`` serve both and hold none of the method's arithmetic.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants and hand-derived golden cases
(``tests/golden/``).  No function is "parity unpinned".
"""

from . import codec, attention  # noqa: F401
