"""The accuracy measurement end to end on the GPU (selection through the C
ABI, exact references in host float64): plans that read every channel fully
select identically, and the tiny workload's planted keys carry the
attention, so a plan that finds them has near-zero output error."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def test_accuracy_tiny():
    need_gpu()
    from sparse_attention_key_amd import accuracy as A

    w = wl.WORKLOADS["tiny"]
    say("accuracy tiny")
    res = A.evaluate(w, ["B512", "r128", "B48", "B8"], [0])
    assert res["B512"]["recall"] == res["r128"]["recall"]
    assert res["B512"]["error"] == res["r128"]["error"]
    assert res["B512"]["recall"] >= 0.8
    assert res["B48"]["error"] < 1e-6  # the 64 planted keys dominate every head's attention
    for v in res.values():
        assert np.isfinite(v["error"]) and 0.0 <= v["error"] <= 2.0
        assert 0.0 <= v["recall"] <= 1.0
