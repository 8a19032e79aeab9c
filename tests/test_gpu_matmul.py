"""One trellis matrix times binned rows (qtip_expert_matmul) vs the oracle's declared-mode
decode and an fp64 product, on both arms; plus unit validation on the device (a bad unit is
skipped, never read out of bounds)."""
import numpy as np
import pytest

import trellis_quantized_moe_expert_amd as q
from gpu_util import say
from oracle import numerics, trellis

pytestmark = pytest.mark.gpu


def run(arm, codes, scales, lut, a_bits, units, rows, cols, fill=np.nan):
    import torch
    E = codes.shape[0]
    P = a_bits.shape[0]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    y = torch.full((P, rows), fill, dtype=torch.float32, device="cuda:0")
    plan = q.qtip_moe_plan(q.make_desc(E, 1, 128, 128, 1), 0)
    q.qtip_expert_matmul(plan, arm, dev(codes), dev(scales.view(np.int16)), dev(lut.view(np.int16)), E, rows, cols,
                         dev(a_bits.view(np.int16)), P, dev(np.array(units, np.int32).reshape(-1, 3)), len(units), y)
    torch.cuda.synchronize()
    q.qtip_moe_plan_destroy(plan)
    return y.cpu().numpy()


def oracle_y(codes, scales, lut, a_bits, units, rows):
    P = a_bits.shape[0]
    y = np.full((P, rows), np.nan)
    a = numerics.bf16_bits_to_f64(a_bits)
    for (e, s, L) in units:
        w = trellis.decode_declared(trellis.stored_rows(codes[e]), lut)
        y[s:s + L] = (a[s:s + L] @ w.T) * scales[e].astype(np.float64)[None, :]
    return y


@pytest.mark.parametrize("arm", [q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED])
@pytest.mark.parametrize("rows,cols,lens", [(64, 512, (1, 2, 16, 64, 33, 7)), (128, 2048, (64, 64, 3)),
                                            (4096, 2048, (5,)), (2048, 4096, (20, 1))])
def test_matmul_random_vs_oracle(arm, rows, cols, lens):
    rng = np.random.default_rng(rows + cols + arm)
    E = 3
    codes = rng.integers(0, 256, size=(E, rows, cols // 4), dtype=np.uint8)
    scales = rng.uniform(0.01, 0.05, size=(E, rows)).astype(np.float16)
    lut = rng.standard_normal(65536).astype(np.float16)
    P = sum(lens)
    a_bits = (rng.standard_normal((P, cols)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    units, s = [], 0
    for i, L in enumerate(lens):
        units.append((i % E, s, L)); s += L
    say(f"matmul arm={arm} rows={rows} cols={cols} lens={lens}")
    got = run(arm, codes, scales, lut, a_bits, units, rows, cols)
    ref = oracle_y(codes, scales, lut, a_bits, units, rows)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 2e-5, err


def test_invalid_units_are_skipped_not_read():
    rng = np.random.default_rng(1)
    E, rows, cols = 2, 32, 256
    codes = rng.integers(0, 256, size=(E, rows, cols // 4), dtype=np.uint8)
    scales = np.ones((E, rows), np.float16)
    lut = rng.standard_normal(65536).astype(np.float16)
    a_bits = (rng.standard_normal((20, cols)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    units = [(0, 0, 4), (5, 4, 4), (1, -1, 2), (1, 8, 65), (1, 18, 3), (1, 8, 0), (1, 10, 10)]
    say("matmul invalid units")
    for arm in (q.QTIP_ARM_GEMV, q.QTIP_ARM_GROUPED):
        got = run(arm, codes, scales, lut, a_bits, units, rows, cols, fill=-123.0)
        ref = oracle_y(codes, scales, lut, a_bits, [units[0], units[6]], rows)
        assert np.allclose(got[0:4], ref[0:4], rtol=2e-5, atol=1e-5)
        assert np.allclose(got[10:20], ref[10:20], rtol=2e-5, atol=1e-5)
        assert np.all(got[4:10] == -123.0)          # rows only invalid units cover stay untouched
