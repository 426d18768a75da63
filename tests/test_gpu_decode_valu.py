"""GPU parity of kvq_decode_attention_valu (the VALU-only comparison kernel) against the
fp64 CPU oracle, on the same cases and with the same bar as kvq_decode_attention."""
import pytest

from bit_kv_cache_pack_amd import kvq as K

from test_gpu_decode import CASES, _full, _run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}h{}_B{}_{}x{}_P{}_R{}_S{}".format(*c))
def test_valu_decode_small(oracle_mod, case):
    bits, hybrid, B, Hq, Hkv, n_packed, n_res, S_ = case
    _run(oracle_mod, bits, hybrid, B, Hq, Hkv, n_packed, n_res, S_, seed=sum(case),
         entry=K.kvq_decode_attention_valu)


@pytest.mark.parametrize("dist,scale", [("t5", 1.0), ("normal", 4.0)])
def test_valu_decode_value_ranges(oracle_mod, dist, scale):
    _run(oracle_mod, 4, False, 1, 8, 2, 640, 128, 5, dist=dist, scale=scale, seed=7,
         entry=K.kvq_decode_attention_valu)
    _run(oracle_mod, 3, False, 1, 8, 2, 640, 128, 5, dist=dist, scale=scale, seed=8,
         entry=K.kvq_decode_attention_valu)


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama8b_32k"])
def test_valu_decode_full_workload(oracle_mod, name):
    _full(oracle_mod, name, entry=K.kvq_decode_attention_valu)
