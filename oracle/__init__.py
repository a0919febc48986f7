"""CPU oracle for Multi-head Latent Attention over a compressed latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports, links or calls it, and shares no code with it: the two meet only in
the seeded input generators of ``workloads``, which hold no attention
arithmetic.

Plain numpy, float64 unless a caller asks for float32 (the pages' own fp32
checks).  No blocking, fusion or reordering beyond what each definition states.

Sources (cited in each function by page title and section):
  * "MLA + KV cache (Tier 3 #5)" ticket: incremental decode must equal a full
    forward (Acceptance criteria); decode projects only the new token and
    attends over the cache (Description).
  * "ARCH-MLA. Multihead Latent Attention" tutorial: the KV-state ledger (Step 1,
    Step 4) and the experiment widths (5.1, 5.4).
  * modeldna "MLA" module: latent c of width kv_lora_rank plus a shared rope
    key, absorption of the up-projections (Under the hood); the Kimi-scale
    cache table.
  * softved article "Multi-Head Latent Attention": quantize the latent cache
    on top of MLA ("Practical Implementation Tips for MLA in LLM Serving");
    the FP8 row format is a reading (``fp8_cache``).
  * "GatedMLA" docs: projection geometry, per-head Q/K/V with the shared key
    broadcast, causal SDPA scaled over the full Q/K width (Projection
    geometry and stored weights; Build per-head Q, K and V; Observe logits,
    then compute causal attention; Output projection and optional gate).

Readings where the pages are silent:
  RoPE pairs element i with i + Dr/2 (half split), frequency theta^(-2i/Dr),
  angle = absolute 0-based position * frequency; RMSNorm eps = 1e-6 on the
  latent part only; W_DKV output order [c | k_pe]; per-head query order
  [nope | rope]; softmax scale 1/sqrt(Dn + Dr) multiplies the sum of both dot
  products; a cache row is rounded to the storage dtype when stored and later
  reads use the stored value.

Pins: every function is checked by ``tests/test_oracle_pins.py`` against
closed forms, invariants, a library routine (torch CPU SDPA), printed page
values (``tests/golden``) or brute-force loops.  The end-to-end numeric
outputs of the five workloads have no printed values on the pages; they are
pinned only through those identities.
"""
from .mla_oracle import *  # noqa: F401,F403
from .fp8_cache import *  # noqa: F401,F403
from . import ledger  # noqa: F401
