"""Reference oracle for the packed quantized linear layer Y = X . W_hat^T.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The library never calls
it, and it shares no code, table or constant with the library: every format
rule below is written out here a second time, from the source pages and the
readings recorded with the design notes.

Sources (three "Makale Bülteni" newsletter pages):

* the SpQR bulletin ("Makale Bülteni — SpQR"): a dense low-precision matrix
  plus a sparse fp16 outlier matrix holding about 1% of the weights; the rest
  in 3 bits with groups of 16 and bi-level (themselves quantized) statistics;
  3.36-4.75 bits per parameter.  Section "İddia ve Gerçeklik" (claim and
  reality).
* the GPTQ bulletin ("Makale Bülteni — GPTQ"): 4-bit weights quantized in
  blocks such as groups of 128; round-to-nearest is the baseline.  Sections
  lead and "İddia ve Gerçeklik".
* the SmoothQuant bulletin ("Makale Bülteni — SmoothQuant"): the identity
  Y = (X diag(s)^-1)(diag(s) W), per-token int8 activations, per-channel int8
  weights, alpha about 0.8-0.85, maxima from calibration samples.  Section
  "İddia ve Gerçeklik".

Two forms, sharing nothing with the library: the numpy modules below (format
encoders, decoders and fp64 forwards), and plain C++17 forwards in
qlin_oracle.cpp (fp64 decode + fp64 dot products per output row, OpenMP over
rows; int64 accumulation for W8A8), compiled on its own by the host compiler
and loaded through ``oracle.cref``.  Each is pinned against hand-worked values,
grid points, brute force and textbook routines (tests/test_oracle_*.py).

Precision: encoders run in fp32 in the written operation order (numpy float32
arithmetic is IEEE round-to-nearest-even, element by element, with no fused
multiply-add); decoders and forwards run in fp64.

Parity status: the layouts (bit positions of codes and statistics) are this
library's own readings where the pages are silent, so they are pinned only by
the round-trip tests, not by any value on the pages ("parity unpinned" for the
byte layout as such).
"""
from . import dense, gptq, metrics, smoothquant, spqr, w4  # noqa: F401
