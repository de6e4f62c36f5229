"""The test plumbing on the CPU: the threaded evaluation of the row oracle
returns what the row oracle returns for the same rows."""

import numpy as np
import torch

import gpu_helpers as H
from oracle import reference as orc


def test_threaded_row_oracle_equals_the_row_oracle():
    g = torch.Generator().manual_seed(3)
    S, Hq, Hkv, D = 300, 8, 2, 32
    q = torch.randn(S, Hq, D, generator=g).bfloat16()
    k = torch.randn(S, Hkv, D, generator=g).bfloat16()
    v = torch.randn(S, Hkv, D, generator=g).bfloat16()
    cu = np.array([0, 7, 150, 151, 300])
    rows = np.array([0, 5, 6, 7, 8, 100, 149, 150, 151, 152, 250, 299])
    Ow, Lw = orc.rope_attention_rows(q, k, v, rows, cu)
    Ot, Lt = H.oracle_rows_threaded(q, k, v, rows, cu, 500000.0, n_threads=4, chunk=5)
    assert Ot.shape == Ow.shape and Lt.shape == Lw.shape
    assert np.max(np.abs(Ot - Ow)) < 1e-12 and np.max(np.abs(Lt - Lw)) < 1e-12
