"""tt_bag_forward_static (the forward that allocates nothing: the grouping and the forward
run in the library's static per-GPU scratch array) against tt_bag_forward with a caller
workspace, through the C ABI: two calls in a row, the second with a smaller batch, then
other shapes (weights, several tables), and the rejection of a batch too large for the
array.  The pooled outputs agree up to the order of the forward's fp32 atomics, and both
match the oracle."""
import numpy as np
import pytest
import torch

import oracle
from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W
from helpers import TOL, gpu_cores, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _both(wl, cores, b):
    g = gpu_cores(wl, cores)
    d = to_dev(b)
    B = b["num_bags"]
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, wl.num_tables)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = abi.tt_bag_forward(desc, g, d["indices"], d["offsets"], B, d["per_sample_weights"],
                             dev_status=st)
    out = torch.full_like(ref, float("nan"))
    got = abi.tt_bag_forward_static(desc, g, d["indices"], d["offsets"], B,
                                    d["per_sample_weights"], out=out, dev_status=st)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert int(st.item()) == 0
    return got.cpu().numpy(), ref.cpu().numpy()


def test_static_forward_matches_the_workspace_forward_twice_in_a_row():
    """Two calls in a row on the same GPU, the second with a smaller batch (the scratch
    keeps the first call's contents), each against tt_bag_forward and the oracle."""
    wl = W.WORKLOADS["readme"]
    cores = W.make_cores(wl)
    for B in (512, 37):
        print("case static forward readme bags", B, flush=True)
        b = W.make_batch(wl, 11, bags_per_table=B)
        got, ref = _both(wl, cores, b)
        assert rel_err(got, ref) <= 1e-6
        Yo = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, cores, b["indices"], b["offsets"], B)
        assert rel_err(got, Yo) <= TOL


def test_static_forward_other_shapes():
    for wl in (W.custom("weighted q1=4 r=32", p=(7, 9, 5), q=(4, 4, 4), ranks=(32, 32),
                        bags_per_table=40, lengths=("uniform", 0, 9), init_std=0.2,
                        weighted=True),
               W.custom("three tables", p=(6, 5, 4), q=(4, 2, 3), ranks=(16, 12), num_tables=3,
                        bags_per_table=20, lengths=("uniform", 1, 8), init_std=0.3),
               W.WORKLOADS["tiny"]):
        print("case static forward", wl.name, flush=True)
        cores = W.make_cores(wl)
        b = W.make_batch(wl, 2)
        got, ref = _both(wl, cores, b)
        assert rel_err(got, ref) <= 1e-6
        Yo = oracle.forward(wl.p, wl.q, wl.ranks, wl.E, cores, b["indices"], b["offsets"],
                            b["num_bags"], per_sample_weights=b["per_sample_weights"])
        assert rel_err(got, Yo) <= TOL


def test_static_forward_rejects_a_batch_beyond_its_scratch():
    """About 80 bytes of scratch per index: 120,000 indices of the README shape need more
    than TT_STATIC_SCRATCH_BYTES, so the call is refused on the host (TT_EWORKSPACE) and
    out keeps its contents."""
    wl = W.WORKLOADS["readme"]
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    B, L = 6000, 20
    idx = torch.zeros(B * L, dtype=torch.int64, device="cuda")
    off = torch.arange(0, B * L + 1, L, dtype=torch.int64, device="cuda")
    g = [torch.zeros(n, device="cuda") for n in abi._core_numels(desc)]
    out = torch.full((B, wl.D), 3.0, device="cuda")
    with pytest.raises(abi.TTError) as e:
        abi.tt_bag_forward_static(desc, g, idx, off, B, out=out)
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
