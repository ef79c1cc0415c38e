"""fp64 CPU oracle of the gated delta rule.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, helpers, tables or pre/post-processing).

Sources (cited by page title and section):
  * "Gated Delta Networks: Improving Mamba2 with Delta Rule" (paper review),
    sections "Method", "Key idea", "Background", "Goal" -- the recurrence,
    its two limits and the test-time-SGD reading.
  * "Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
    Routing" (abstract) -- names the per-channel (Kimi-Delta-style) gate
    without defining it.
  * the GDN review's "Future work" and closing section -- name Householder-
    product transitions (several delta steps per token) without a formula.
  * "TreeWY: Speculative Verification for Gated DeltaNet Hybrids" (summary in
    the list of related papers) -- draft-tree verification with one
    triangular solve and a commit of the accepted state only.
  * "Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
    Routing" (abstract) and its related-paper entry "Gated DeltaNet-2:
    Decoupling Erase and Write in Linear Attention" -- name Gated
    DeltaNet-2's separate erase and write control without a formula.

Parity status per function is listed in ``gdn_oracle.__doc__``.
"""

from .gdn_oracle import (  # noqa: F401
    gdn_fwd,
    gdn_fwd_chain,
    gdn_decode,
    gdn_bwd,
    gdn_bwd_chain,
    gdn_chunked_bruteforce,
    gdn_sgd_form,
    delta_rule_ungated,
    deltaproduct_fwd,
    gdn_fwd_qknorm,
    l2_normalize,
    tree_fwd,
    tree_commit,
    tree_path,
    tree_wy_bruteforce,
    normwise_rel_err,
    gdn2_fwd,
    gdn2_fwd_chain,
    gdn2_decode,
    gdn2_chunked_bruteforce,
    short_conv,
    silu,
    conv_prologue,
    conv_prologue_bwd,
    gdn_fwd_conv,
)
