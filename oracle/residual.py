"""Oracle: the step after the MoE block in Beam's residual stream.

Test infrastructure only; see the package docstring.

Launch post ("Introducing Beam"), section "Residual Stream", and the
transformers model doc "Beam", section "Overview" (depth-scaled residual and
sandwich norm):

* every sublayer is wrapped in RMSNorm before and after ("sandwich"); the
  post-norm of the MoE block normalises its output;
* the input embedding is step 1; at step k a sublayer's (post-normalised)
  output enters the stream with weight 1/sqrt(k) while the existing stream is
  kept with weight sqrt((k-1)/k). The two squared weights sum to one, and
  after k steps the stream is the sum of all k contributions divided by
  sqrt(k);
* RMSNorm is computed in fp32 in the implementation (section "Residual
  Stream": normalisation is one of the fp32 islands).

Readings (the pages give no formula for RMSNorm's details): RMSNorm(v) =
v / sqrt(mean(v^2) + eps) * gain, the mean over the hidden dimension, with a
learned per-channel gain and a small eps (a parameter; 1e-6 where a default is
needed). Parity of eps's value and of the gain's placement is unpinned (the
pages fix neither); the rest is pinned by tests/test_oracle_residual.py.
"""

import numpy as np


def rms_norm(v, gain, eps):
    """Row-wise RMSNorm of a [T, H] array (float64)."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def step_weights(k):
    """(weight of the existing stream, weight of the new contribution) at step k >= 2."""
    return np.sqrt((k - 1.0) / k), 1.0 / np.sqrt(k)


def residual_update(stream_in, block_out, gain, eps, k):
    """The stream after step k, whose sublayer output is ``block_out``:
    sqrt((k-1)/k) * stream_in + RMSNorm(block_out) / sqrt(k)."""
    keep, add = step_weights(k)
    return keep * np.asarray(stream_in, dtype=np.float64) + add * rms_norm(block_out, gain, eps)
