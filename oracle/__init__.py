"""FP64 CPU oracle of the GDN layer core.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it. The HIP library never does.

Parity status of each function (what pins it; the pins live in
``tests/test_oracle_pins.py``):

* ``round_to``          - checked against numpy float16 and torch float32->bf16.
* ``causal_conv_silu``  - library conv1d (groups=C), separate == concatenated,
                          identity taps give SiLU, causality, varlen reset.
* ``beta_and_g``        - closed-form special values, ranges.
* ``l2norm``            - norm identity, flag-off no-op, GQA replication.
* ``gated_delta_rule``  - T=1 closed form, scalar geometric-series closed form,
                          brute-force product of transition matrices (T<=8),
                          exact key/value retrieval, pure decay, chunked ==
                          sequential, varlen == separate runs, state handoff.
* ``gated_rmsnorm``     - library rms_norm and silu, gate 0, scale invariance.
* ``layer``             - composition of the above; concatenated conv equals
                          three separate convs end to end.
* ``decode_step``       - T steps from a zero cache and state equal ``layer``
                          over the T tokens (every output, and the final state
                          of ``gated_delta_rule``); the cache shift is exact;
                          a closed form for one step from a nonzero state.

``backward.py`` (first-order gradients of the gated norm, of the prologue and
of the gated delta rule, by float64 autograd of the plain forward) is pinned by finite differences and
closed forms in ``tests/test_oracle_backward_pins.py``.

No function is "parity unpinned", but the absolute values of the layer have no
printed worked example on the pages to check against.
"""
from .gdn import (beta_and_g, build, causal_conv_silu, decode_step,  # noqa: F401
                  default_threads, gated_delta_rule, gated_rmsnorm, l2norm, layer, round_to, silu,
                  softplus)
