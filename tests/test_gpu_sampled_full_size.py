"""Parity at the full workload sizes, in the launch configuration the
benchmark times (all shards in one launch, then the merge), checked on
sampled requests that the float64 oracle evaluates one by one."""
import numpy as np
import pytest

import workload
from gpu_cases import compare, run_gpu, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("name,requests", [
    ("dense_bf16_32k", [0, 17, 31]),
    ("dense_fp8_mixed", None),        # shortest, longest and one more request
    ("long_fp8_1m", [2]),
    ("sparse_fp8_topk2048", [0, 77, 127]),
])
def test_full_size_sampled(name, requests):
    sp = workload.SPECS[name]
    say(f"full-size {name}: generating")
    x = workload.generate(sp)
    if requests is None:
        L = x.context_lens
        requests = sorted({int(np.argmin(L)), int(np.argmax(L)), 5})
    say(f"full-size {name}: running the GPU step")
    _, step = run_gpu(x)
    say(f"full-size {name}: oracle on requests {requests}")
    compare(x, step, requests=requests)
