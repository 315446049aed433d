"""CPU oracle for sink + short-window KV-cache attention (LongLive).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
anything in this package: only the tests, the package smoke check and the
benchmark's ``cpu_baseline`` leg may use it.

The oracle is a plain, slow, float64 restatement of what the method computes,
written from the paper "LongLive: Real-time Interactive Long Video Generation":

* ``attention``  -- masked softmax attention with an explicit frame mask
  (frame sink + short rolling window, causal across chunks), and the text
  cross-attention.
* ``cache_model`` -- which chunks the cache holds after every append, which
  window chunks a KV-recache rewrites, and the full token history a layer has
  seen (with recache payloads applied).
* ``quant``       -- the per-token, per-head symmetric INT8 quantiser used by
  the INT8 KV-cache variant, in float32 as the variant defines it.
* ``linear_attention`` -- the linear-attention variant over the same key set
  (feature map max(x, 0), normalised weighted sum), pairwise form.

It shares no code with the HIP path; the only module both sides use is the
seeded input generator, which holds none of the method's arithmetic.
"""

from .attention import (allowed_frames, frame_mask, masked_attention,
                        sink_window_attention, cross_attention, window_reencode_attention,
                        sink_window_attention_grad)
from .cache_model import (CacheGeometry, slot_of_chunk, DequeCacheModel,
                          resident_window_chunks, LayerHistory)
from .quant import quantize_int8, dequantize_int8
from .linear_attention import (LINEAR_EPS, feature_map, linear_masked_attention,
                               linear_sink_window_attention)

__all__ = [
    "allowed_frames", "frame_mask", "masked_attention", "sink_window_attention",
    "cross_attention", "window_reencode_attention", "sink_window_attention_grad",
    "CacheGeometry", "slot_of_chunk", "DequeCacheModel",
    "resident_window_chunks", "LayerHistory", "quantize_int8", "dequantize_int8",
    "LINEAR_EPS", "feature_map", "linear_masked_attention", "linear_sink_window_attention",
]
