"""Bit-exact decode through the matmul.  With an integer LUT (lut[s] = (s mod 251) - 125,
exact in fp16 and bf16), unit scales and one-hot activation rows, each output equals one
decoded weight exactly; both arms must reproduce the oracle's decode bit for bit, including
weights whose window wraps past the row end."""
import numpy as np
import pytest

import trellis_quantized_moe_expert_amd as q
from gpu_util import say
from oracle import trellis

pytestmark = pytest.mark.gpu


def integer_lut():
    s = np.arange(65536)
    return ((s % 251) - 125).astype(np.float16)


@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
@pytest.mark.parametrize("rows,cols", [(32, 128), (48, 384), (16, 256)])
def test_decode_bitexact_one_hot(arm, rows, cols):
    import torch
    rng = np.random.default_rng(rows * cols + arm)
    E = 3
    codes = rng.integers(0, 256, size=(E, rows, cols // 4), dtype=np.uint8)
    lut = integer_lut()
    scales = np.ones((E, rows), np.float16)
    # one-hot rows: columns cover the start, the wrap region and random positions
    cols_hot = [0, 1, 7, cols - 8, cols - 7, cols - 1] + rng.integers(0, cols, 60).tolist()
    P = len(cols_hot)
    a = np.zeros((P, cols), np.float32)
    a[np.arange(P), cols_hot] = 1.0
    a_bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    # units: ragged lengths over three experts
    units, s, e = [], 0, 0
    for L in (1, 5, 16, 17, 3, 24):
        units.append((e % E, s, L)); s += L; e += 1
    assert s == P
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    y = torch.full((P, rows), float("nan"), dtype=torch.float32, device="cuda:0")
    plan = q.qtip_moe_plan(q.make_desc(E, 1, 128, 128, 1), 0)
    say(f"decode one-hot arm={arm} rows={rows} cols={cols} units={units}")
    q.qtip_expert_matmul(plan, arm, dev(codes), dev(scales.view(np.int16)), dev(lut.view(np.int16)), E, rows, cols,
                         dev(a_bits.view(np.int16)), P, dev(np.array(units, np.int32)), len(units), y)
    torch.cuda.synchronize()
    q.qtip_moe_plan_destroy(plan)
    got = y.cpu().numpy()
    for (ex, st, L) in units:
        w = trellis.decode_declared(trellis.stored_rows(codes[ex]), lut)  # [rows, cols]
        for i in range(L):
            expect = w[:, cols_hot[st + i]]
            assert np.array_equal(got[st + i], expect.astype(np.float32)), (ex, st + i, cols_hot[st + i])
