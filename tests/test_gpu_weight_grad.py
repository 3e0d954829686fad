"""GPU parity of the gradient with respect to the per-sample weights
(tt_bag_weight_grad) against the oracle's dL/dw: every element within 1e-4 of the
oracle (per tensor), misses and cache hits, sum and mean pooling, skipped elements
zero, planned call equal to the stateless one bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from tensor_train_compressed_ttembeddingbag_amd import abi, workloads as W
from helpers import TOL, gpu_cores, rel_err, to_dev
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

CASES = [w for w in SMALL if w.D <= 512]


def _check(wl, b, pooling=0, cache=None, K=0, slots_np=None, rows_np=None):
    cores = W.make_cores(wl)
    g = gpu_cores(wl, cores)
    d = to_dev(b)
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E, wl.num_tables, pooling=pooling)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((d["indices"].numel(),), float("nan"), device="cuda")
    ws = abi.workspace(desc, d["indices"].numel(), b["num_bags"], K)
    abi.tt_bag_weight_grad(desc, g, d["indices"], d["offsets"], b["num_bags"], d["grad_out"],
                           per_sample_weights=d["per_sample_weights"], cache=cache, out=out,
                           ws=ws, dev_status=st)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.isnan(got).any()
    ref = oracle.backward(wl.p, wl.q, wl.ranks, wl.E, cores, b["indices"], b["offsets"],
                          b["num_bags"], b["grad_out"], per_sample_weights=b["per_sample_weights"],
                          slots=slots_np, cache_size=K, pooling=pooling, cache_rows=rows_np,
                          weight_grad=True)[4]
    assert rel_err(got, ref) <= TOL, rel_err(got, ref)
    return desc, g, d, got, st


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
@pytest.mark.parametrize("pooling", [0, 1], ids=["sum", "mean"])
def test_weight_grad_small_shapes(wl, pooling):
    print("case wgrad", wl.name, pooling, flush=True)
    _check(wl, W.make_batch(wl, 0), pooling)


def test_weight_grad_readme_and_planned():
    print("case wgrad readme", flush=True)
    wl = W.WORKLOADS["readme"]
    b = W.make_batch(wl, 0)
    desc, g, d, got, _ = _check(wl, b)
    ws = abi.tt_bag_plan(desc, d["indices"], d["offsets"], b["num_bags"])
    again = abi.tt_bag_weight_grad(desc, g, d["indices"], d["offsets"], b["num_bags"],
                                   d["grad_out"], ws=ws, planned=True)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy().view(np.uint32), got.view(np.uint32))


def test_weight_grad_with_cache_hits_and_skipped_elements():
    print("case wgrad cache", flush=True)
    wl = W.custom("cache", p=(20, 22, 25), q=(4, 4, 4), ranks=(32, 32), bags_per_table=300,
                  lengths=("uniform", 1, 20), dist=("zipf", 1.2), init_std=1 / 32 ** 0.5,
                  lr=0.01, weighted=True)
    K = 512
    desc = abi.make_desc(wl.p, wl.q, wl.ranks, wl.E)
    cache = abi.Cache(desc, K, 1 << 14)
    cache.lookup(torch.from_numpy(W.make_batch(wl, 100)["indices"]).cuda(), count_freq=True)
    rows = torch.zeros(K, wl.D, device="cuda")
    cache.populate(gpu_cores(wl, W.make_cores(wl)), rows)
    rows += 0.125  # rows that differ from the TT rows (trained)
    b = W.make_batch(wl, 0)
    slots = cache.lookup(torch.from_numpy(b["indices"]).cuda(), count_freq=False)
    sl = slots.cpu().numpy()
    assert (sl >= 0).any() and (sl < 0).any()
    for pooling in (0, 1):
        _check(wl, b, pooling, cache=(slots, rows), K=K, slots_np=sl, rows_np=rows.cpu().numpy())
    # an invalid index is skipped: its gradient is 0 and the status says so
    bad = dict(b)
    bad["indices"] = b["indices"].copy()
    bad["indices"][3] = wl.E + 7
    d = to_dev(bad)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = abi.tt_bag_weight_grad(desc, gpu_cores(wl, W.make_cores(wl)), d["indices"], d["offsets"],
                                 b["num_bags"], d["grad_out"], dev_status=st)
    torch.cuda.synchronize()
    assert out[3].item() == 0.0 and int(st.item()) & abi.TT_DEV_BAD_INDEX
    cache.close()
