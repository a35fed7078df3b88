"""The hand-derived closed-form cases of tests/golden/powers_of_two.json run on
the GPU, through the C ABI, with no oracle in between.

Each case is zero-padded to the head size (extra zero columns change no dot
product and add zero output columns), uses scale = ln 2 so that every weight
is 2^n for an integer n, and is compared with the exact fractions and logs
the fixture states.  The inputs are small integers, exact in both 16-bit
types; O is rounded to the input type at the end, so the bar is the usual
max |dO| <= 2e-2 and |dLSE| <= 1e-3.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import dense_attention_amd as da

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "powers_of_two.json")


def _ln(s):
    assert s.startswith("ln(") and s.endswith(")")
    return math.log(float(Fraction(s[3:-1])))


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    da.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("variant", ["default", "all"])
def test_golden_fractions_on_gpu(D, dtype, variant):
    with open(GOLDEN) as f:
        g = json.load(f)
    assert g["scale"] == "ln2"
    code = da.ATTN_F16 if dtype == torch.float16 else da.ATTN_BF16
    ids = [0] if variant == "default" else \
        [v["id"] for v in da.attn_variants() if v["head_dim"] == D and v["dtype"] == code]
    for case in g["cases"]:
        q, k, v = (np.array(case[n], dtype=np.float64) for n in ("q", "k", "v"))
        exp_o = np.array([[float(Fraction(x)) for x in row] for row in case["expected_o"]])
        exp_l = np.array([_ln(x) for x in case["expected_lse"]])

        def pad(a):
            out = np.zeros((a.shape[0], D))
            out[:, : a.shape[1]] = a
            return torch.tensor(out, dtype=dtype).reshape(1, 1, a.shape[0], D).cuda()

        qd, kd, vd = pad(q), pad(k), pad(v)
        for var in ids:
            o, lse = da.attn_fwd_strided(qd, kd, vd, scale=math.log(2.0), variant=var)
            torch.cuda.synchronize()
            go = o[0, 0].cpu().double().numpy()
            gl = lse[0, 0].cpu().double().numpy()
            assert np.all(go[:, exp_o.shape[1]:] == 0), (case["name"], var)
            err = np.abs(go[:, : exp_o.shape[1]] - exp_o).max()
            lerr = np.abs(gl - exp_l).max()
            assert err <= 2e-2 and lerr <= 1e-3, (case["name"], var, err, lerr)
