"""csa_index_topk_noalloc (static scratch, no workspace) against csa_index_topk
on two calls in a row, the second smaller: indices and scores must be equal
bit for bit (the same kernels over the same inputs), and the small call must
equal the oracle exactly on grid inputs."""
import numpy as np
import pytest
import torch

import oracle
from helpers import both

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_sparse_kv_compress_amd as csa
else:
    csa = None


def _pair(q, kk, m, k, w, n_ctx):
    B, T = q.shape[:2]
    idx_a = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
    sc_a = torch.full((B, T, k), 3.0, dtype=torch.float32, device="cuda")
    csa.csa_index_topk_noalloc(q, kk, m, k, w_idx=w, n_ctx=n_ctx, idx=idx_a, out_score=sc_a)
    idx_b, sc_b = csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=n_ctx, want_scores=True)
    torch.cuda.synchronize()
    return idx_a, sc_a, idx_b, sc_b


def test_noalloc_equals_workspace_call_twice():
    assert csa.csa_index_topk_noalloc_max_bytes() == 32 << 20
    HI, dI, m = 64, 128, 4
    # call 1: the 1M-token decode shape, 16 sequences (single-pass plan)
    B, L, k = 16, 250000, 1024
    n_ctx = m * L
    q, _ = both((B, 1, HI, dI), 61, "q_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    kk, _ = both((B, L, dI), 61, "k_idx", dtype=torch.bfloat16, scale=dI ** -0.5)
    w, _ = both((B, 1, HI), 61, "w_idx", dtype=torch.float32, scale=HI ** -0.5)
    idx_a, sc_a, idx_b, sc_b = _pair(q, kk, m, k, w, n_ctx)
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(sc_a.view(torch.int32), sc_b.view(torch.int32))
    del q, kk, w
    # call 2: smaller (6 query rows over 30,001 entries: scores then top-k in
    # row groups), grid inputs so every score is exact
    B, T, L, k = 2, 3, 30001, 512
    n_ctx = m * L - 1
    q, q_c = both((B, T, HI, dI), 62, "q_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    kk, k_c = both((B, L, dI), 62, "k_idx", dtype=torch.bfloat16, kind="grid", scale=2.0 ** -4)
    idx_a, sc_a, idx_b, sc_b = _pair(q, kk, m, k, None, n_ctx)
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(sc_a.view(torch.int32), sc_b.view(torch.int32))
    want, _ = oracle.index_topk(q_c, k_c, m, k, n_ctx=n_ctx)
    assert np.array_equal(idx_a.cpu().numpy(), want)
