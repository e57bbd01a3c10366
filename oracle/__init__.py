"""CPU oracle for the TurboQuant-style KV codec: TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy/SciPy implementation of what the codec computes,
written step by step from the pages' description of the method.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the library (``kv_cache_vector_05_amd``) never does, and the oracle never
imports the library.  The two share no code: the only common module is
``synth``, which generates seeded inputs and holds none of the method's
arithmetic.

Sources (cited by page title and section):

* "FibQuant: Quantizacao Vetorial Universal para Compressao de KV-Cache de
  Acesso Aleatorio" (gist.science summary), referred to as the FibQuant
  summary: section 1 (fixed-address random-access records; the
  normalise-rotate-quantise interface: store the norm, shared Haar rotation,
  per-coordinate Lloyd-Max table), section 2.1 (the normalised, rotated vector
  is uniform on the sphere, so a coordinate follows the spherical-Beta law and
  one offline table serves every input), section 2.3 (encoder: norm, rotate
  the unit vector; decoder: look up, inverse rotation, scale by the norm).
* "TurboQuant: Compressao Avancada da Google para Cache KV ..." (iaemfoco
  post), section "TurboQuant: Uma Nova Abordagem": the randomized Hadamard
  transform and the quantized Johnson-Lindenstrauss step that removes the
  inner-product bias.
* "Compressao KV eficaz com TurboQuant" (itstec post), section "Por dentro do
  processo de compressao KV": random rotation gives each coordinate a Beta
  law; MSE-optimal quantisers bias inner products; the residual is sketched by
  a JL transform reduced to sign bits, giving an unbiased estimator.
* "TurboESM: Ultra-Efficient 3-Bit KV Cache Quantization ..." (gist.science
  summary), technical summary section 2: RoPE is applied before the orthogonal
  rotation; 8-entry Lloyd-Max tables; a 1-bit sign of the residual; a fused
  decode kernel with online softmax.
* "Google acelera LLMs em 8 vezes" (tambur post): attention logits computed
  directly from quantised keys.

Parity status of each function is stated in its docstring; every function is
pinned by the CPU tests in ``tests/test_oracle_*.py`` except where a
docstring says "parity unpinned".
"""
from . import rng, lloyd_max, rotation, rope, codec, estimator, calibration, paging, fibquant  # noqa: F401
from .codec import Codebook, make_codebook, encode, dequant  # noqa: F401
