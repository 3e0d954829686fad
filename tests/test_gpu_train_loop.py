"""The training loop the benchmark times (loop.TrainLoop: the grouping of batch i+1 on a
second stream during the backward of batch i, two alternating workspaces, event ordering),
at the full readme and table-batched sizes: every step's pooled forward and core update
against the oracle evaluated at the cores that step started from."""
import numpy as np
import pytest
import torch

import oracle
from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W
from tensor_train_compressed_ttembeddingbag_amd.loop import TrainLoop
from helpers import TOL, gpu_cores, host_cores, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name, steps", [("readme", 3), ("multitable", 2)])
def test_pipelined_loop_matches_oracle(name, steps):
    print("case train loop", name, steps, flush=True)
    wl = W.WORKLOADS[name]
    T, B = wl.num_tables, wl.bags_per_table
    cores = W.make_cores(wl)
    g = gpu_cores(wl, cores)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, T)
    host_batches = [W.make_batch(wl, k) for k in range(2)]  # cycled, as the benchmark does
    out = torch.empty(T * B, wl.D, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    loop = TrainLoop(desc, g, [to_dev(b) for b in host_batches], B, wl.lr, out, status)
    snaps, ys = [[x.clone() for x in g]], []
    for _ in range(steps):
        loop.step()
        # both copies run on the main stream: after forward i / backward i, before step i+1
        ys.append(out.clone())
        snaps.append([x.clone() for x in g])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for i in range(steps):
        b = host_batches[i % 2]
        start, end = host_cores(wl, snaps[i]), host_cores(wl, snaps[i + 1])
        yref = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"], b["offsets"], B,
                              per_sample_weights=b["per_sample_weights"])
        assert rel_err(ys[i].cpu().numpy(), yref) <= TOL, i
        grads, touched, _, _ = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, start, b["indices"],
                                               b["offsets"], B, b["grad_out"],
                                               per_sample_weights=b["per_sample_weights"])
        for t in range(T):
            for k in range(3):
                delta = end[t][k].astype(np.float64) - start[t][k].astype(np.float64)
                assert rel_err(delta, -wl.lr * grads[t][k]) <= TOL, (i, t, k)
                m = ~touched[t][k].astype(bool)
                assert np.array_equal(end[t][k][:, m], start[t][k][:, m]), (i, t, k)
