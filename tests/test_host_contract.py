"""Host-side contract checks that need no GPU: the benchmark refuses more than one GPU with
a message, the binding fails loudly when the HIP library is missing (there is no CPU
fallback), and the synthetic workloads have the sizes the benchmark reports."""
import os
import subprocess
import sys

import pytest

import synth_inputs as S
from bit_kv_cache_pack_amd import kvq as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(K, "_lib", None)
    monkeypatch.setattr(K, "LIB_PATH", str(tmp_path / "missing" / "libkvq.so"))
    with pytest.raises(ImportError, match="build it"):
        K.lib()


def test_workload_bytes():
    wl = S.WORKLOADS["llama8b_32k"]
    # 8 rows x 32640 packed tokens x 2 x (64 B codes + 16 B scale/zero) + 128 fp16 tokens x 2
    assert wl.step_bytes() == 8 * (32640 * 160 + 128 * 512) == 42303488
    assert S.WORKLOADS["tiny"].step_bytes() == 2 * (896 * 160 + 128 * 512)
    pw = S.PAGED_WORKLOADS["paged_ragged_b16"]
    assert pw.kv_bytes_per_token_head() == 160 and pw.gq == 4
