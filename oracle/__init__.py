"""CPU oracle for the KIVI grouped KV-cache codec.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
anything in this package; only the test-suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

Two tiers, written independently of each other and of the HIP path:

* :mod:`oracle.kivi_ref`   -- vectorised numpy in explicit float32/float16.
* :mod:`oracle.kivi_exact` -- pure Python on exact rationals with a
  hand-written round-to-nearest-even into the binary16/binary32 formats,
  for tiny inputs.  It pins the numpy tier's use of hardware rounding.
* :mod:`oracle.attention_ref` -- float64 decode-phase attention of one query
  token per head over the dequantized prefix plus the fp16 residual.
* :mod:`oracle.fp8_ref` -- FP8 (E4M3) keys of the k8v4 layout, by nearest
  value over the listed code points.
* :mod:`oracle.layer_mix_ref` -- per-layer bit mixes: the protected boundary
  layers of a model, and layer-by-layer coding of a mixed cache.

Sources (titles of the pages the method is taken from):

* CacheForge README, "How it works": keys are quantized per channel, values
  per token, and the newest tokens are not quantized; the
  "Example" section names the knobs ``k_bits``, ``v_bits``, ``group_size``
  and ``residual_length`` (recent fp16 tokens), defaults 2/2/32/128.
* CacheSeek pull request #4 "Feature(quantization): add KIVI KV-cache
  quantization for exact-prefix reuse", description: KIVI encode/decode with
  grouped statistics, padding, and packing of the codes into int32 words;
  compact ``qdata``/``scale``/``offset`` payload.
* vLLM ``turboquant/config.py``, ``TurboQuantConfig`` docstring (a b-bit
  code has 2**b levels, stated there for 3 and 4 bits) and ``value_packed_size``
  (a per-vector uniform value code costs ceil(D*b/8) bytes plus an fp16
  scale and an fp16 zero).

The pages print no formula for the statistics or the rounding; the readings
used here are stated in each function's docstring.
"""

from . import attention_ref, fp8_ref, kivi_exact, kivi_ref, layer_mix_ref  # noqa: F401
