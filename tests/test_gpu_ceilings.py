"""The device-ceiling microbenchmarks (moe_ceilings) run and report rates
inside what the device can physically do: a streaming read below the 8 TB/s
HBM peak and fp16 MFMA below its 2.5 PFLOP/s dense peak."""
import json
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "bit_quantized_expert_router_amd", "moe_ceilings")


@pytest.mark.gpu
def test_ceilings_program():
    assert os.path.exists(EXE), "moe_ceilings is not built"
    print("running moe_ceilings", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr
    d = json.loads(r.stdout.strip().splitlines()[-1])
    print(d)
    assert 1000.0 < d["stream_read_GBps"] < 8000.0
    assert 3.0 < d["burst_24MiB_us"] < 100.0          # 24 MiB takes 3 us even at the 8 TB/s peak
    assert 0.0 < d["empty_kernel_us_graph"] < 50.0
    assert 0.0 < d["empty_kernel_us_eager"] < 50.0
    assert 100.0 < d["mfma_f16_TFLOPs"] < 2600.0
    assert d["dequant_mfma_Tweights_per_s"] > 0.0
