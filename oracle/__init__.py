"""Plain CPU oracle for one Kimi-K3-shaped MXFP4 routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, the graft entry's smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path: it decodes the same bytes
with its own decoders, in float64 with numpy.

Sources (page title, section):
  * Deltafin README ("An experiment in running Kimi K3 (2.8T parameters) on
    one Apple Silicon Mac"), "How it works" and "Techniques / Compute":
    16 of 896 experts are read per MoE layer, and MXFP4 weights are decoded
    inside the product (dequant fused with the GEMV, e8m0 scale applied to
    the fp32 exponent); the dense weights kept as row-scaled int8 and
    expanded to fp32 by a fused convert-scale-copy kernel (spine.py).
  * Deltafin explainer (bhfrc.com, "Kimi K3 extreme deployment"), section 2.1:
    hidden 7168, 896 routed experts with 16 selected, 2 shared experts,
    MXFP4 weights with MXFP8 activations; section 5.1: the two shared
    experts' results are added after the routed experts.
  * kimi-k3-in-c note (curvesoft.net, "2.78T model in 8 GB"), byte
    accounting: 0.53125 bytes per MXFP4 weight (4-bit element plus one 8-bit
    exponent per 32 elements) and 17,547,264 bytes per expert.

Where the pages are silent (scoring function, tie rule, renormalisation,
activation, nibble order, MXFP8 quantiser), this oracle follows the readings
listed in the repository's design notes; each function names its reading.

Parity pins: every public function is pinned by tests under tests/ marked
"not gpu" (closed forms, library routines, brute force, invariants).  The
pages print no worked example of a layer output; the whole layer is pinned
against a result assembled by hand from exactly rounded router sums and
closed-form experts, and its parts individually.

Modules:
  formats -- E2M1, E8M0, E4M3, bf16 encodings and the MXFP4/MXFP8 codecs.
  record  -- the expert record layout (six tensors, contiguous).
  moe     -- router, expert FFN, shared experts, combine, RMSNorm, layer.
"""

from . import formats, record, moe  # noqa: F401
