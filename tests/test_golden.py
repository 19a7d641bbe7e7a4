"""Stored small-case outputs (tests/golden/oracle_small_cases.json, written by
tests/golden/make_golden.py from the CPU fp64 oracle only).

The CPU test pins the oracle against its stored outputs (any change to its
arithmetic shows up here and must be justified); the GPU test compares the HIP
path with the stored values directly, at the usual bar (max-abs <= 1e-2,
relative L2 <= 2e-3; fp32 inputs also relative L2 <= 1e-5)."""
import json
import os

import numpy as np
import pytest

from tests.golden import make_golden as mg

with open(os.path.join(os.path.dirname(mg.__file__), "oracle_small_cases.json")) as f:
    GOLDEN = json.load(f)["cases"]


def stored(name):
    c = GOLDEN[name]
    return np.array(c["out"], dtype=np.float64).reshape(c["shape"])


@pytest.mark.parametrize("name", sorted(mg.CASES))
def test_oracle_reproduces_stored_outputs(name):
    case = mg.CASES[name]
    assert GOLDEN[name]["args"] == json.loads(json.dumps(case))
    ref = mg.expected(case, mg.build(case))
    np.testing.assert_allclose(ref, stored(name), rtol=1e-8, atol=1e-12)


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(mg.CASES))
def test_hip_matches_stored_outputs(name):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from tests.gpu_util import DeviceBatch, assert_parity, host

    case = mg.CASES[name]
    bt = mg.build(case)
    dev = DeviceBatch(bt)
    if case["mode"] == "decode":
        got = dev.decode(0)
    elif case["mode"] == "causal":
        got = dev.mixed(0)
    else:
        got = dev.cross(0)
    assert_parity(host(got), stored(name), bt.dtype, f"golden {name}")
