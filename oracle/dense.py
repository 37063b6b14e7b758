"""Oracle for the dense fp16 layer Y = X . W^T, the 16-bit baseline.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages measure every format against 16-bit inference: the SpQR and
SmoothQuant bulletins ("İddia ve Gerçeklik") quote their speedups over it, and
the GPTQ bulletin ("İddia ve Gerçeklik") and the SmoothQuant bulletin
("Ticari Etki") describe the weight-only gain fading against it as the batch
grows.  The layer has a plain definition, written out here: every fp16 input
is exact in fp64, and the product sums in fp64.

Readings where the pages are silent: X fp16 [M][K] and W fp16 [N][K], both
row-major (W stored out x in, as the quantized formats store it).
"""
from __future__ import annotations

import numpy as np


def forward(X, W):
    """fp64 Y [M][N] = X . W^T for fp16 X [M][K] and W [N][K]."""
    X = np.asarray(X)
    W = np.asarray(W)
    assert X.dtype == np.float16 and W.dtype == np.float16, "fp16 operands"
    assert X.ndim == 2 and W.ndim == 2 and X.shape[1] == W.shape[1], "X [M][K], W [N][K]"
    return X.astype(np.float64) @ W.astype(np.float64).T


def forward_cols(X, W, cols):
    """The columns `cols` of forward(X, W), from those rows of W only."""
    return forward(X, np.asarray(W)[np.asarray(cols)])
