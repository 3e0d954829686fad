"""TT with fewer than three cores as the three-core case with unit trailing cores: a
two-core table W[i1 p2 + i2] = vec(G1[i1] G2[i2]) (ranks (R1), q = (q1, q2)) is run as
p = (p1, p2, 1), q = (q1, q2, 1), ranks = (R1, 1) with a third core equal to 1.  The
GPU forward and SGD step are compared with the two-core definition written out in
numpy (fp64) -- not with the three-core oracle.  (The unit core receives its own update
too; a caller training a two-core model resets it, or uses the gradient variant and
ignores its gradient.)"""
import numpy as np
import pytest
import torch

from tensor_train_compressed_ttembeddingbag_amd import abi
from helpers import TOL, rel_err

pytestmark = pytest.mark.gpu


def test_two_core_table_forward_and_sgd():
    print("case two-core", flush=True)
    rng = np.random.Generator(np.random.PCG64(61))
    p1, p2, q1, q2, R = 13, 11, 4, 8, 24
    E, D, B = p1 * p2, q1 * q2, 40
    G1 = (rng.standard_normal((p1, q1, R)) * 0.3).astype(np.float32)   # [i1][j1][r]
    G2 = (rng.standard_normal((p2, R, q2)) * 0.3).astype(np.float32)   # [i2][r][j2]
    lens = rng.integers(0, 9, B)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    idx = rng.integers(0, E, off[-1]).astype(np.int64)
    w = rng.random(off[-1]).astype(np.float32)
    dY = rng.standard_normal((B, D)).astype(np.float32)
    # two-core definition: W[i][j1 q2 + j2] = sum_r G1[i1][j1][r] G2[i2][r][j2]
    Wd = np.einsum("ajr,brk->abjk", G1.astype(np.float64), G2.astype(np.float64)).reshape(E, D)
    Yref = np.zeros((B, D))
    for b in range(B):
        for n in range(off[b], off[b + 1]):
            Yref[b] += w[n] * Wd[idx[n]]
    # the same table as three cores: slice-major G1 [p1][1][q1][R], G2 [p2][R][q2][1], G3 = 1
    cores = [torch.from_numpy(G1.reshape(-1).copy()).cuda(),
             torch.from_numpy(G2.reshape(-1).copy()).cuda(),
             torch.ones(1, device="cuda")]
    desc = abi.make_desc((p1, p2, 1), (q1, q2, 1), (R, 1), E)
    d_idx, d_off = torch.from_numpy(idx).cuda(), torch.from_numpy(off).cuda()
    d_w, d_dY = torch.from_numpy(w).cuda(), torch.from_numpy(dY).cuda()
    Y = abi.tt_bag_forward(desc, cores, d_idx, d_off, B, d_w).cpu().numpy()
    assert rel_err(Y, Yref) <= TOL
    lr = 0.05
    abi.tt_bag_backward_sgd(desc, cores, d_idx, d_off, B, d_dY, lr, d_w)
    torch.cuda.synchronize()
    # gradients of the two-core definition
    g1, g2 = np.zeros(G1.shape), np.zeros(G2.shape)
    for b in range(B):
        for n in range(off[b], off[b + 1]):
            i1, i2 = divmod(int(idx[n]), p2)
            gr = w[n] * dY[b].astype(np.float64).reshape(q1, q2)
            g1[i1] += gr @ G2[i2].astype(np.float64).T
            g2[i2] += G1[i1].astype(np.float64).T @ gr
    n1 = cores[0].cpu().numpy().reshape(G1.shape).astype(np.float64)
    n2 = cores[1].cpu().numpy().reshape(G2.shape).astype(np.float64)
    assert rel_err(n1 - G1, -lr * g1) <= TOL
    assert rel_err(n2 - G2, -lr * g2) <= TOL
