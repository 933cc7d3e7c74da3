"""fp64 CPU oracle for paged prefix-reuse attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of the package entry script and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library and
its Python binding) never calls it, and this package imports nothing from the
product: the two share no code.  The only module both sides consume is the
seeded input generator (``workloads``), which holds no attention arithmetic.

What it computes, and from which passages:

* A block pool of fixed 16-token blocks reached through per-sequence block tables
  whose prefix blocks may be shared copy-on-write (kvboost 0.6.0, section "CPU
  paged attention"; kvstream 0.1.0, "Why KVStream?" feature table and "Request
  lifecycle" step 3).
* New K/V written one slot per token into that pool (kvstream 0.1.0, "Why
  KVStream?" feature table, "Streaming KV allocation"; "Request lifecycle" step 2).
* A new chunk processed together with its cached prefix in one forward pass, so
  each chunk row attends to the whole cached prefix and causally to the chunk
  (kvboost 0.6.0, "How it works", step 5 "Forward pass"; "Flash Attention (CUDA)",
  the supported-properties table: causal masking).
* Decode as the one-query case of the same attention (kvboost 0.6.0, "CPU paged
  attention": only the decode loop changes; "How it works", step 5).

The attention itself is the plain definition: the full score row is built, its
maximum subtracted, exponentials normalised and V averaged with those weights,
all in float64 — no tiling, no online softmax, no split.  The pages fix fp16 and
bf16 inputs; the oracle decodes those 16-bit payloads exactly to float64.

Pins (tests marked ``not gpu``): brute force on tiny inputs with scalar Python
math; hand-derived closed forms under ``tests/golden``; rows of the softmax
summing to one; a single key returning its V; equal scores returning the mean
of V; block-permutation invariance; the reuse invariant (prefill over a cached
prefix equals full causal attention on those rows); decode equals a one-row
prefill; GQA equals MHA with repeated K/V; causality; the log-sum-exp merge of
key partitions; block copies leave every sequence's gathered tokens unchanged under
a remapped table.  The 8-bit pool (``oracle.quant``: per-channel K scales, per-token V
scales) is pinned by hand-derived codes under ``tests/golden`` (round half to even,
clamping, zero scales), the half-step error bound, and the reduction that decode over a
pool whose values are exactly what their codes stand for equals the 16-bit decode bit
for bit.  The softmax scale 1/sqrt(head_dim) is the conventional reading
(the tiny workload states it; the pages state no other): parity unpinned by the
pages for that convention beyond the tiny workload.
"""
from .attention import (  # noqa: F401
    decode_bits,
    write_kv,
    copy_blocks,
    gather_kv,
    attend,
    paged_prefill,
    paged_decode,
    lse_merge,
)
