"""Oracle: bf16 storage of an fp32 value (float64 in and out, numpy).

Test infrastructure only; see the package docstring.

Beam launch post, "Residual Stream": the SwiGLU product is an fp32 island;
the intermediate h that leaves it is stored as bf16 before the down
projection reads it (the storage reading of the design notes). With
quantised experts the per-row E4M3 quantisation then starts from those
stored values.

bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of
an IEEE binary32 value. The value is first rounded to binary32 (round to
nearest even), then to the nearest bf16 with ties to the even bf16 (the
lowest kept fraction bit 0): add 0x7FFF plus that bit to the 32-bit pattern
and clear the low 16 bits. Values here are finite; overflow past the
largest bf16 gives infinity as the definition does.
"""

import numpy as np


def round_to_bf16(v):
    """The bf16 value nearest fp32(v) (ties to even), as float64."""
    f32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    bits = f32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return rounded.view(np.float32).astype(np.float64)
