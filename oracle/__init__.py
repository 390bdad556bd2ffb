"""Float64 CPU oracle for sequence-sharded MLA decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plainly written
definition that the GPU library is checked against.  Only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its Python binding) never does, and this
package imports nothing from the product path.

What it computes, with the page each part follows:

* MLA decode attention with one shared latent KV head: every query head
  scores every attended token over 512 latent + 64 rope dimensions and
  averages the 512-d latent part (the values) with the softmax weights.
  Geometry from "GLM-5.2 vLLM Decode Context Parallelism", section
  "Understand the cache-copy opportunity" (64 query heads, latent rank 512,
  one effective latent KV head) and "The Final Verification: Confirming a
  200k Context Deployment on GLM-5", section "The Decision-Making Process
  Visible in the Reasoning" (512 latent + 64 rope per token).
* Per-shard partial attention that also returns the softmax log-sum-exp,
  and the LSE-weighted merge of the partials: "GLM-5.2 vLLM Decode Context
  Parallelism", sections "See why vLLM 0.26.0 fails" and "Frequently asked
  questions" (what DCP is; why DCP needs softmax LSE).
* Round-robin ownership of cache tokens by shard: "How vLLM Serves GLM-5.3
  with Million-Token Contexts on 16 H200s", section "The core design".
* Localisation of global sparse top-K indices to the owning shard, and the
  neutral (0, -inf) row of a shard that owns none of a row's selections:
  "GLM-5.2 vLLM Decode Context Parallelism", section "Separate the backend
  merge from stable".
* Writing new tokens into the sharded cache: the owning shard's slot of each
  token (a negative slot suppresses the cache write, never the query: "GLM-5.2
  vLLM Decode Context Parallelism", section "Keep the current-main
  correctness blocker visible") and the row it receives in the cache's
  storage format, with the fp8 codes chosen by a per-group scale and
  round-to-nearest-even (a reading; the pages give no quantiser).
* Top-K selection of the sparse indices from indexer scores over each query
  token's causal prefix, per shard and merged across shards ("GLM-5.2 vLLM
  Decode Context Parallelism", section "Understand the cache-copy
  opportunity": top-K of 2,048; "How vLLM Serves GLM-5.3 with Million-Token
  Contexts on 16 H200s", section "Why conventional TP and DP fall short").

Every function states the passage it follows.  Where the pages leave a step
open, the reading taken is stated at the function.

Pins (tests marked ``not gpu``): closed forms of softmax attention, the
partition invariant of the merge against an independent library attention
(torch scaled_dot_product_attention in float64) and scipy's logsumexp, the
OCP E4M3FN code table, exact rounding midpoints and torch's float8/bfloat16
casts for the codecs and encoders,
brute-force enumeration for the integer steps, and the tables the pages
print (copy geometry, head envelope, per-token byte counts).
"""

from . import codecs, sharding, attention, capacity, decode, kv_write, topk  # noqa: F401
