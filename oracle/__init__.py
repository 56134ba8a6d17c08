"""Plain, slow, fp64 CPU oracle for the online KV vector quantizer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
C ABI or the Python binding) may import, call or link anything here; only the
test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path: the seeded
synthetic-input generators live in ``synthetic.py`` and hold none of the
method's arithmetic.

Source of the method: the page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배
절약 구현 방법" (a2a-mcp.org), sections
  * "TurboQuant 작동 방식" (two-stage online algorithm),
  * "1단계: 무작위 회전 + PolarQuant 압축" (seeded random orthogonal rotation
    from the QR factorisation of a Gaussian matrix; rotated coordinates follow
    Beta((d-1)/2, (d-1)/2) on [-1, 1]; vectors are normalised; a Lloyd-Max
    quantiser optimal for that law maps every coordinate to a few bits),
  * "2단계: QJL 잔차 보정" (one sign bit of a Gaussian projection of the
    stage-1 residual removes the inner-product bias),
  * the same section's closing paragraphs (logits straight from the indices
    against a query rotated once; reconstruction cosine about 0.983 at 3 bits),
  * "TurboQuant 구현 방법" (codebooks precomputed per hidden size and bit
    width; the query is pre-rotated once).

Modules
  splitmix   SplitMix64 counter generator, uniforms, Box-Muller normals.
  rotation   Haar rotation Pi, QJL matrix S and M = S Pi^T.
  codebook   Lloyd-Max codebook for the Beta coordinate law (closed-form
             cell integrals through the regularised incomplete beta).
  quantizer  quantise (MSE / inner-product mode), bit-plane packing,
             dequantise, attention logits, top-k search, recall.
  attention  decode attention output softmax(l) . V_hat over a quantised
             value cache.
  decode     decode step with append: quantise the new key of every stream
             into the cache at a token position, logits over the prefix.
  polar      PolarQuant variant of stage 1: recursive polar transform of the
             rotated unit vector, Lloyd-Max codebooks of the angle laws,
             packing and reconstruction.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
textbook special cases, brute force or invariants.  Points the page leaves
open are read as stated in each module's docstring.
"""

from . import splitmix, rotation, codebook, quantizer, attention, decode, polar  # noqa: F401
