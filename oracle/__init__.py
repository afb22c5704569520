"""Plain CPU oracle for the Beam sparse-MoE block.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this
package: only the tests, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` call it. It shares no code with the HIP
library under ``group_limited_routing_amd/``.

Everything here is slow, plain numpy in float64 (bf16 and fp32 inputs
upcast exactly), written from the statement of the block:

* Beam launch post ("Introducing Beam"), section "Mixture of Experts":
  sigmoid scores over all 256 experts, 8 groups of 32, keep the 4 groups
  with the best sum of their two top scores, take the top 8 experts inside
  them, no shared expert, combine with the normalised router weights and
  scale by 2.5; every expert is a SwiGLU MLP of intermediate size 2560.
* Same post, section "Residual Stream": the router and the SwiGLU product
  are computed in fp32.
* transformers model doc "Beam", section "Overview": a learned per-expert
  bias balances load in place of an auxiliary loss; ``n_group``,
  ``topk_group`` and ``routed_scaling_factor`` name the group count, the
  kept-group count and the output scale; router weights and expert bias are
  kept in fp32.
* Same doc, section "Notes": router logits are returned on request.

Readings of points the pages leave open (each is also listed in the design
notes): the bias enters the selection key only, never the weights; group
scores use the same biased key; groups are contiguous index blocks; ties go
to the lower index; experts outside the kept groups get a key of -inf; the
weights are divided by the sum of the selected sigmoid scores; no capacity
limit, every token gets exactly ``top_k`` experts.

Parity status: every function here is pinned by the CPU tests
(tests/test_oracle_*.py) except where its docstring says "parity unpinned".
"""

from .routing import sigmoid, group_scores, select_from_keys, route  # noqa: F401
from .experts import expert_ffn, forward, forward_tokens, dense_forward  # noqa: F401
from . import bf16  # noqa: F401
from . import e4m3  # noqa: F401
from . import mxfp4  # noqa: F401
from . import residual  # noqa: F401
from . import backward  # noqa: F401
