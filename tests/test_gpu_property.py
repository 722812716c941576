"""Property tier on the GPU: random cases at the supported geometry (query groups {1, 2, 4, 8, 32}, block
sizes {16, 32}, head_dim {64, 128}, q_len from 0 to chunk size, random block permutations, shared first
blocks) through write + attention, against the oracle, under both bf16 row-tile kinds with automatic or
short forced partitions, and on the float32 path.  A fixed number of derandomised examples without
shrinking: reproducible, and the first failure ends the test."""

import pytest
import torch
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import oracle
import paged_kv_cache_229_amd as pkv
from gpu_util import DeviceWorkload, check_close, log, out_f64
from property_cases import gpu_case
from workloads import BF16, FP32

pytestmark = pytest.mark.gpu


def _settings(n):
    return settings(max_examples=n, deadline=None, derandomize=True, database=None,
                    phases=[Phase.explicit, Phase.generate],
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large,
                                           HealthCheck.function_scoped_fixture])


def _run(w, kind, partition):
    log(f"property case kind={kind} P={partition}: {w.description}")
    pkv.set_tuning(partition, 0, kind)
    try:
        dw = DeviceWorkload(w)
        out = dw.run_step(0)
        torch.cuda.synchronize()
    finally:
        pkv.set_tuning(0, 0, 0)
    _, _, ref = oracle.run_step(w.k_pool, w.v_pool, w.block_tables, w.steps[0], w.scale, w.dtype)
    check_close(out_f64(out), ref, w.dtype, f"property kind={kind} P={partition}")


@_settings(60)
@given(gpu_case(BF16), st.sampled_from([1, 2]), st.sampled_from([0, 0, 64, 256]))
def test_property_bf16(w, kind, partition):
    _run(w, kind, partition)


@_settings(20)
@given(gpu_case(FP32))
def test_property_fp32(w):
    _run(w, 0, 0)
