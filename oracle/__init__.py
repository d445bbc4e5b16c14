"""fp64 CPU oracle for fused exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
imports nothing from the product path. The two share no code; only the seeded
input generator (``exact_io_aware_12_amd.inputs``, which holds no attention
arithmetic) feeds both, and the oracle does not even import that: it takes
plain float64 arrays.

What it computes, and from where (pages: "FlashAttention core principles"
lesson 1 = page 1; the aiworkagent interview answer on FlashAttention = page 2;
"FlashAttention and Triton", chapter 19 = page 3):

* ``attention_fwd`` -- the plain definition O = softmax(scale * Q K^T) V of
  page 1 section 1 and page 3 section 19.1, with the per-row logsumexp that
  page 1 section 5 keeps instead of P. Pages 2 ("exact, not approximate") and
  1 (section 4, "why the rescale is right") state that the fused method reaches
  exactly this result, so the oracle is the definition, not the algorithm.
* ``attention_bwd`` -- the gradient of that definition (page 1 section 5,
  softmax backward), with the row sum taken over the whole row.
* ``attention_tiled`` -- the online-softmax recurrence (page 1 sections 3-4,
  page 2 "2. Online Softmax", page 3 section 19.5 and the tiling simulator of
  section 19.12), used only to check that tiled and untiled agree.
* ``online_softmax_stream`` -- the same recurrence on one row of raw scores
  (the two-block example of page 3 section 19.5).
* ``attention_fwd_brute`` / ``attention_bwd_brute`` -- scalar loops, no BLAS,
  for tiny inputs.
* ``attention_decode`` -- the same definition with Nq query rows against Nk
  key/value rows (the KV-cache use that page 2's bonus points name); causal
  queries are the last Nq positions.

Every function has a pin in ``tests/test_oracle.py`` that does not re-type its
formula: closed forms, the worked example, invariants, brute force, central
finite differences and a library cross-check. No function is parity unpinned.
"""
from .attention import (  # noqa: F401
    attention_bwd,
    attention_decode,
    attention_bwd_brute,
    attention_fwd,
    attention_fwd_brute,
    attention_probs,
    attention_tiled,
    online_softmax_stream,
)
