"""Host-side pieces of the benchmark (no GPU needed): the CPU oracle baseline runs on a
valid sample of every workload kind -- one table, several tables (table 0's bags),
per-sample weights, four cores -- on one core and on all usable cores, and reports what
it ran."""
import pytest

import bench
from tensor_train_compressed_ttembeddingbag_amd import workloads as W


@pytest.mark.parametrize("name", ["tiny", "multitable", "skewed", "readme4"])
def test_cpu_baseline_runs_on_a_valid_sample(name):
    wl = W.WORKLOADS[name]
    r = bench.cpu_baseline(wl, W.make_cores(wl), 0.05)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["value_1core"] > 0
    assert r["cores"] == bench._host_threads() and r["cores_1core"] == 1
    assert len(r["runs_us_per_nnz"]["1"]) == 5 and len(r["runs_us_per_nnz"][str(r["cores"])]) == 5
    assert r["cpu_model"]
    if wl.num_tables > 1:
        assert "of table 0 of %d" % wl.num_tables in r["sample"]
