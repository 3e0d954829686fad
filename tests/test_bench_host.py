"""Host-side pieces of the benchmark (no GPU needed): the CPU oracle baseline runs on a
valid sample of every workload kind -- one table, several tables (table 0's bags),
per-sample weights, four cores -- and reports what it ran."""
import pytest

import bench
from tensor_train_compressed_ttembeddingbag_amd import workloads as W


@pytest.mark.parametrize("name", ["tiny", "multitable", "skewed", "readme4"])
def test_cpu_baseline_runs_on_a_valid_sample(name):
    wl = W.WORKLOADS[name]
    r = bench.cpu_baseline(wl, W.make_cores(wl), 0.05)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    if wl.num_tables > 1:
        assert "of table 0 of %d" % wl.num_tables in r["sample"]
