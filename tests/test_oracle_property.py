"""Property tier on the CPU: random tiny cases (random block permutations, shared first blocks, MHA, GQA
and MQA, q_len 0 included) of the oracle against scalar brute force that reads every key from its own
(block, offset) slot, in float32 and bf16 storage.  A fixed number of derandomised examples, no shrinking,
so the run is reproducible and stops at the first failure."""

import numpy as np
from hypothesis import HealthCheck, Phase, given, settings

import oracle.paged_kv as O
from oracle_pins import _brute_force
from property_cases import tiny_case
from workloads import BF16, FP32

_SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                     phases=[Phase.explicit, Phase.generate],
                     suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _check(w):
    st = w.steps[0]
    kp, vp = O.kv_write(w.k_pool, w.v_pool, st.k_new, st.v_new, st.slot_mapping)
    out = O.paged_attention(st.q, kp, vp, w.block_tables, st.context_lens, st.query_start_loc, w.scale,
                            w.dtype)
    ref = _brute_force(w, kp, vp, st, w.scale)
    assert np.max(np.abs(out - ref), initial=0.0) <= 1e-12, w.description


@_SETTINGS
@given(tiny_case(FP32))
def test_oracle_matches_brute_force_fp32(w):
    _check(w)


@_SETTINGS
@given(tiny_case(BF16))
def test_oracle_matches_brute_force_bf16(w):
    _check(w)
