"""Oracle INT8 quantiser for the INT8 KV-cache variant.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The paper mentions INT8 only as quantised *model* inference (LongLive: Real-time
Interactive Long Video Generation, Abstract and §5 "Conclusion": model size
2.7 GB to 1.4 GB); it gives no KV-cache scheme.  The variant built here is the
plainest symmetric one: per token and per head, over the head dimension,

    a = max |x|                       (float32, exact)
    s = fl32(a / 127)                 (IEEE float32 division)
    q = clamp(rne(fl32(x / s)), -127, 127)   (round half to even)
    a == 0  ->  s = 0, q = 0

and the dequantised value is q * s, formed exactly in float64.  Every step that
decides an integer is taken in float32, the precision the scheme is stated in.
"""

import numpy as np


def quantize_int8(x):
    """x: float32 [..., D] -> (q int8 [..., D], s float32 [...])."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("the quantiser is defined on float32 inputs")
    a = np.max(np.abs(x), axis=-1)                        # float32, exact
    s = (a / np.float32(127.0)).astype(np.float32)       # IEEE float32 division
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    r = (x / safe[..., None]).astype(np.float32)          # IEEE float32 division
    q = np.clip(np.rint(r), -127, 127)                    # rint: half to even
    q = np.where(s[..., None] == 0, 0, q).astype(np.int8)
    return q, s


def dequantize_int8(q, s):
    """Exact dequantisation in float64: q * s."""
    return q.astype(np.float64) * np.asarray(s, dtype=np.float64)[..., None]
