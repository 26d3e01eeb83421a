"""Float64 CPU oracle for the routed MoE layer over block-quantised expert weights.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this package: only the tests, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library and imports
nothing from it; the two meet only through the seeded generator in ``synth``.

It is a plain, slow definition of what the layer computes, in NumPy float64:
  * ``formats``: E2M1 / E8M0 / E4M3 / bf16 decoding, MXFP4 and FP8-block dequantisation,
    and the OCP MX quantiser used for MX-quantised activations;
  * ``layer``: router logits, softmax / sigmoid scoring with top-k and renormalisation,
    the token-to-expert permutation, each expert's SwiGLU FFN, the shared expert with
    its gate, the LatentMoE projections and the weighted combine.

Every function cites the passage of the pages it follows.  Where the pages are silent,
the reading taken is stated in the docstring.  Each function is pinned by a CPU test
against something other than itself (a hand-derived table, a library routine, brute
force, a closed form or an invariant); there is no function here whose parity is
unpinned.
"""
from . import formats, layer  # noqa: F401
