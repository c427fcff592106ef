"""The committed measurement records match the sources they describe.

`bench.py` reports the forward kernel's HBM traffic from the rocprofv3 counter
record of its workload (profiles/traffic_attn_fwd_<workload>.json), and only
while the record's kernel-source hash equals the tree's: a kernel edit without
new counter runs would silently turn the benchmark line's `traffic` into null.
"""
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WORKLOADS = ["sparse", "sparse_mask", "mha", "gqa", "varlen_d64", "varlen_d128", "varlen_d256"]


@pytest.mark.parametrize("workload", WORKLOADS)
def test_traffic_record_is_of_this_kernel(workload):
    rec = json.load(open(os.path.join(ROOT, "profiles", f"traffic_attn_fwd_{workload}.json")))
    assert rec["workload_name"] == workload
    assert rec["kernel_src_sha256_16"] == bench.kernel_hash(), (
        "the forward kernel changed since its counters were taken: re-run the rocprofv3 FETCH_SIZE / "
        "WRITE_SIZE passes for this workload")
    # the summary it points to was made from the same kernel source
    summary = open(os.path.join(ROOT, rec["source"])).read()
    assert bench.kernel_hash() in summary
    assert rec["bytes_per_launch"] > rec["algorithmic_bytes"] > 0


def test_headline_traffic_is_reported():
    assert bench.measured_traffic("sparse") is not None
