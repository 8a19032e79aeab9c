"""CPU-side checks of the HIP library: it loads, exports every declared entry point, and its
host logic (plan validation, the closed-form predicate, argument errors) behaves as documented.
No test here launches GPU work."""
import ctypes
import os
import re

import pytest

import trellis_quantized_moe_expert_amd as q
from oracle import fill

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
V4 = dict(num_experts=256, top_k=6, hidden=4096, inter=2048, max_tokens=1024)


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qtip_moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qtip_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 17
    lib = q.lib()
    for name in names:
        assert hasattr(lib, name), name


def test_plan_for_arch_accepts_gfx950_and_reports_schedule():
    # dispatch_tile_m=16 reproduces the pages' sm80 gate exactly
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, dispatch_tile_m=16), "gfx950:sramecc+:xnack-")
    info = q.qtip_moe_plan_info(plan)
    assert info["tile_m"] == 16
    assert info["min_tokens_grouped"] == 683
    assert info["workspace_bytes"] > 1024 * 6 * (4096 * 4 + 2048 * 2)
    assert q.qtip_moe_select_arm(plan, 682) == q.QTIP_ARM_GEMV
    assert q.qtip_moe_select_arm(plan, 683) == q.QTIP_ARM_GROUPED
    assert q.qtip_moe_select_arm(plan, 8) == q.QTIP_ARM_GEMV
    line = q.qtip_moe_engaged_line(plan, 1572)
    assert "grouped" in line and "230.3%" in line and "36.84" in line and "683" in line
    q.qtip_moe_plan_destroy(plan)


@pytest.mark.parametrize("thr,expect", [(32, 1366), (64, 2731), (16, 683)])
def test_dispatch_threshold_drives_the_predicate(thr, expect):
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, dispatch_tile_m=thr), "gfx950")
    assert q.qtip_moe_plan_info(plan)["min_tokens_grouped"] == expect == fill.min_tokens_grouped(6, 256, thr)
    # below the grouped flip: the fused GEMV, or the dequantize arm once the fill reaches the
    # traffic ratio (16) under a higher grouped threshold
    below = {"gemv": q.QTIP_ARM_GEMV, "dequant": q.QTIP_ARM_DEQUANT}[fill.select_arm(expect - 1, 6, 256, thr)]
    assert q.qtip_moe_select_arm(plan, expect - 1) == below
    assert below == (q.QTIP_ARM_DEQUANT if thr > 16 else q.QTIP_ARM_GEMV)
    assert q.qtip_moe_select_arm(plan, expect) == q.QTIP_ARM_GROUPED
    q.qtip_moe_plan_destroy(plan)


ARM_CODE = {"gemv": q.QTIP_ARM_GEMV, "grouped": q.QTIP_ARM_GROUPED, "dequant": q.QTIP_ARM_DEQUANT}


def test_three_arm_closed_form_matches_the_oracle():
    for k, E in [(6, 256), (2, 8), (8, 128), (1, 4), (6, 64)]:
        for tm in (1, 16, 32, 64):
            for ratio in (8, 16, 32):
                for n in (1, 8, 9, 20, 100, 300, 683, 1000, 1500, 3000):
                    assert q.qtip_fill_select_arm(n, k, E, tm, ratio) == ARM_CODE[fill.select_arm(n, k, E, tm, ratio)]
    assert q.qtip_fill_select_arm(0, 6, 256, 16, 16) == -1
    assert q.qtip_fill_select_arm(9, 6, 256, 16, 0) == -1


@pytest.mark.parametrize("k,E", [(6, 256), (2, 8), (8, 128), (1, 4), (6, 64), (8, 256)])
def test_default_boundaries_leave_no_dequantize_window(k, E):
    for thr in (0, 16):
        plan = q.qtip_moe_plan_for_arch(q.make_desc(E, k, 256, 128, 4096, dispatch_tile_m=thr), "gfx950")
        assert q.qtip_moe_dequant_range(plan) == (0, 0)
        assert all(q.qtip_moe_select_arm(plan, n) != q.QTIP_ARM_DEQUANT for n in range(1, 4097, 7))
        q.qtip_moe_plan_destroy(plan)


def test_a_window_is_reported_and_sized():
    base = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    ws0 = q.qtip_moe_plan_info(base)["workspace_bytes"]
    q.qtip_moe_plan_destroy(base)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, dispatch_tile_m=32), "gfx950")
    lo, hi = q.qtip_moe_dequant_range(plan)
    assert (lo, hi) == (fill.min_tokens_grouped(6, 256, 16), 1025)      # grouped flip (1366) is past max_tokens
    assert fill.dequant_tokens(6, 256, 32, 16, 1024) == list(range(lo, hi))
    assert q.qtip_moe_select_arm(plan, lo) == q.QTIP_ARM_DEQUANT and q.qtip_moe_select_arm(plan, lo - 1) == q.QTIP_ARM_GEMV
    dense = 3 * 256 * 4096 * 2048 * 2
    assert q.qtip_moe_plan_info(plan)["workspace_bytes"] >= ws0 + dense
    q.qtip_moe_plan_destroy(plan)
    pinned = q.qtip_moe_plan_for_arch(q.make_desc(**V4, arm_override=q.QTIP_ARM_DEQUANT), "gfx950")
    assert q.qtip_moe_select_arm(pinned, 32) == q.QTIP_ARM_DEQUANT
    rows = q.qtip_moe_plan_for_arch(q.make_desc(**V4, act_layout=q.QTIP_ACT_ROWS), "gfx950")
    assert q.qtip_moe_plan_info(pinned)["workspace_bytes"] >= q.qtip_moe_plan_info(rows)["workspace_bytes"] + dense
    q.qtip_moe_plan_destroy(rows)
    sch = q.qtip_moe_plan_schedule(pinned, 32)
    assert sch["arm"] == q.QTIP_ARM_DEQUANT and sch["gate_up"]["waves_per_workgroup"] == 16
    q.qtip_moe_plan_destroy(pinned)
    with pytest.raises(q.QtipError):
        q.qtip_moe_plan_for_arch(q.make_desc(**V4, dequant_traffic_ratio=-1), "gfx950")


def test_dequantize_argument_errors_return_before_any_launch():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    w = q.qtip_moe_weights(256, 256, 256, 256, 256, 256, 256)
    lib = q.lib()
    dq = lambda m, e, out: lib.qtip_moe_dequantize(plan, ctypes.byref(w), m, e, out, None)
    assert dq(3, 0, 256) == q.QTIP_ERR_INVALID_ARG
    assert dq(-1, 0, 256) == q.QTIP_ERR_INVALID_ARG
    assert dq(0, 256, 256) == q.QTIP_ERR_INVALID_ARG
    assert dq(0, -1, 256) == q.QTIP_ERR_INVALID_ARG
    assert dq(0, 0, None) == q.QTIP_ERR_INVALID_ARG
    assert dq(0, 0, 264) == q.QTIP_ERR_INVALID_ARG                # misaligned output
    w.codes_down = 260
    assert dq(2, 0, 256) == q.QTIP_ERR_INVALID_ARG                # misaligned codes
    q.qtip_moe_plan_destroy(plan)


def test_default_dispatch_threshold_is_the_rederived_value():
    # one pair per woken expert and the measured floor of each rung: the grouped arm from 8 tokens
    # (bitshift) and from 5 (LUT rung), the measured crossovers
    for rung, floor in ((q.QTIP_RUNG_BITSHIFT, 7), (q.QTIP_RUNG_LUT, 4)):
        plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, rung=rung), "gfx950")
        assert q.qtip_moe_plan_info(plan)["min_tokens_grouped"] == floor + 1 == \
            fill.min_tokens_grouped(6, 256, 1, floor=floor)
        assert q.qtip_moe_select_arm(plan, floor) == q.QTIP_ARM_GEMV
        assert q.qtip_moe_select_arm(plan, floor + 1) == q.QTIP_ARM_GROUPED
        line = q.qtip_moe_engaged_line(plan, 32)
        assert "threshold 1 pairs" in line and f"GEMV up to {floor} tokens" in line
        q.qtip_moe_plan_destroy(plan)
    assert (q.QTIP_DEFAULT_DECODE_FLOOR_BITSHIFT, q.QTIP_DEFAULT_DECODE_FLOOR_LUT) == (7, 4)
    # the pages' floor, 8, as a plan field
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, decode_floor=8), "gfx950")
    assert q.qtip_moe_plan_info(plan)["min_tokens_grouped"] == 9 == fill.min_tokens_grouped(6, 256, 1)
    assert q.qtip_moe_select_arm(plan, 8) == q.QTIP_ARM_GEMV and q.qtip_moe_select_arm(plan, 9) == q.QTIP_ARM_GROUPED
    q.qtip_moe_plan_destroy(plan)


@pytest.mark.parametrize("floor", [1, 2, 4, 8, 16, 100])
def test_decode_floor_field_moves_the_switch(floor):
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, decode_floor=floor), "gfx950")
    for n in range(1, 130):
        want = {"gemv": q.QTIP_ARM_GEMV, "grouped": q.QTIP_ARM_GROUPED}[fill.select_arm(n, 6, 256, 1, floor=floor)]
        assert q.qtip_moe_select_arm(plan, n) == want, (floor, n)
    assert q.qtip_moe_plan_info(plan)["min_tokens_grouped"] == floor + 1
    q.qtip_moe_plan_destroy(plan)
    with pytest.raises(q.QtipError):
        q.qtip_moe_plan_for_arch(q.make_desc(**V4, decode_floor=-1), "gfx950")


@pytest.mark.parametrize("tile_m", [16, 32, 64])
def test_tile_m_is_reported_and_drives_the_tile_fill(tile_m):
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, tile_m=tile_m), "gfx950")
    assert q.qtip_moe_plan_info(plan)["tile_m"] == tile_m
    pct = 100 * fill.pairs_per_woken_expert(1024, 6, 256) / tile_m
    assert f"{pct:.1f}%" in q.qtip_moe_engaged_line(plan, 1024)
    q.qtip_moe_plan_destroy(plan)


def test_override_pins_the_arm():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, arm_override=q.QTIP_ARM_GROUPED), "gfx950")
    assert q.qtip_moe_select_arm(plan, 1) == q.QTIP_ARM_GROUPED
    assert "pinned" in q.qtip_moe_engaged_line(plan, 1)
    q.qtip_moe_plan_destroy(plan)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, arm_override=q.QTIP_ARM_GEMV), "gfx950")
    assert q.qtip_moe_select_arm(plan, 5000) == q.QTIP_ARM_GEMV
    q.qtip_moe_plan_destroy(plan)


@pytest.mark.parametrize("arch", ["gfx942", "gfx90a", "gfx9500", "sm_90", ""])
def test_unsupported_arch_is_refused(arch):
    with pytest.raises(q.QtipError) as ei:
        q.qtip_moe_plan_for_arch(q.make_desc(**V4), arch)
    assert ei.value.status == q.QTIP_ERR_NOT_SUPPORTED


@pytest.mark.parametrize("bad", [dict(num_experts=0), dict(top_k=0), dict(top_k=300), dict(hidden=4000),
                                 dict(inter=64), dict(max_tokens=0), dict(arm_override=7), dict(out_dtype=3),
                                 dict(tile_m=8), dict(num_experts=2048, top_k=6), dict(top_k=33),
                                 dict(dispatch_tile_m=-1), dict(dispatch_tile_m=2000)])
def test_invalid_desc_is_refused(bad):
    with pytest.raises(q.QtipError) as ei:
        q.qtip_moe_plan_for_arch(q.make_desc(**{**V4, **bad}), "gfx950")
    assert ei.value.status == q.QTIP_ERR_INVALID_ARG


def test_unknown_variant_warns_and_keeps_default(capfd):
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, variant=12), "gfx950")
    assert "unknown kernel variant 12" in capfd.readouterr().err
    q.qtip_moe_plan_destroy(plan)


def test_fill_functions_match_the_pages_and_the_oracle():
    assert f"{q.qtip_fill_woken_experts(32, 6, 256):.1f}" == "136.1"
    assert f"{q.qtip_fill_pairs_per_woken_expert(128, 6, 256):.2f}" == "3.15"
    assert f"{q.qtip_fill_pairs_per_woken_expert(683, 6, 256):.2f}" == "16.01"
    assert q.qtip_fill_min_tokens(6, 256, 16) == 683
    for n in (1, 8, 9, 32, 512, 682, 683, 1024, 1572, 2000):
        assert q.qtip_fill_select_grouped(n, 6, 256, 16) == int(fill.select_grouped(n, 6, 256, 16))
        assert q.qtip_fill_pairs_per_woken_expert(n, 6, 256) == pytest.approx(fill.pairs_per_woken_expert(n, 6, 256), rel=1e-12)
    for k, E in [(1, 4), (2, 8), (6, 64), (8, 256), (6, 8), (1, 1024)]:
        for tm in (16, 32, 64):
            assert q.qtip_fill_min_tokens(k, E, tm) == fill.min_tokens_grouped(k, E, tm)
    assert q.qtip_fill_select_grouped(0, 6, 256, 16) == -1
    assert q.qtip_fill_min_tokens(7, 6, 16) == -1


def test_forward_argument_errors_return_before_any_launch():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    ws = q.qtip_moe_plan_info(plan)["workspace_bytes"]
    w = q.qtip_moe_weights(256, 256, 256, 256, 256, 256, 256)
    lib = q.lib()
    fwd = lambda wp, x, lg, n, out, wsp, wsb: lib.qtip_moe_forward(plan, wp, x, lg, n, out, wsp, wsb, None)
    W = ctypes.byref(w)
    assert fwd(W, 256, 256, 0, 256, 256, ws) == q.QTIP_ERR_INVALID_CONFIG          # empty launch
    assert fwd(W, 256, 256, -3, 256, 256, ws) == q.QTIP_ERR_INVALID_CONFIG
    assert fwd(W, 256, 256, 1025, 256, 256, ws) == q.QTIP_ERR_INVALID_CONFIG       # above max_tokens
    assert fwd(W, None, 256, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG
    assert fwd(None, 256, 256, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG
    assert fwd(W, 256, 256, 4, 256, 256, ws - 1) == q.QTIP_ERR_INVALID_ARG         # workspace too small
    assert fwd(W, 256, 256, 4, 256, 384, ws) == q.QTIP_ERR_INVALID_ARG             # misaligned workspace
    assert fwd(W, 264, 256, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG             # misaligned x
    w.lut = None
    assert fwd(W, 256, 256, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG
    assert "NULL weight" in q.last_error_detail()
    assert lib.qtip_expert_matmul(plan, 1, 256, 256, 256, 4, 32, 256, 256, 8, 256, 0, 256, None) == q.QTIP_ERR_INVALID_CONFIG
    assert lib.qtip_expert_matmul(plan, 5, 256, 256, 256, 4, 32, 256, 256, 8, 256, 1, 256, None) == q.QTIP_ERR_INVALID_ARG
    assert lib.qtip_expert_matmul(plan, 1, 256, 256, 256, 4, 30, 256, 256, 8, 256, 1, 256, None) == q.QTIP_ERR_INVALID_ARG
    assert lib.qtip_moe_route(plan, 256, 0, 256, 256, 256, 256, 256, 256, 256, None) == q.QTIP_ERR_INVALID_CONFIG
    q.qtip_moe_plan_destroy(plan)


def test_status_strings():
    assert q.status_name(0) == "QTIP_OK"
    assert q.status_name(5) == "QTIP_ERR_CAPTURING"


def test_schedule_reports_what_a_forward_launches():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    s4 = q.qtip_moe_plan_schedule(plan, 4)
    s32 = q.qtip_moe_plan_schedule(plan, 32)
    s1024 = q.qtip_moe_plan_schedule(plan, 1024)
    assert s4["arm"] == q.QTIP_ARM_GEMV and s32["arm"] == q.QTIP_ARM_GROUPED and s1024["arm"] == q.QTIP_ARM_GROUPED
    for s in (s32, s1024):
        assert s["tile_m"] == 16
        for st in (s["gate_up"], s["down"]):
            assert 1 <= st["variant"] <= 10
            assert st["rows_per_task"] in (16, 32, 64) and st["waves_per_workgroup"] in (8, 12, 16)
            assert st["pairs_per_decode"] >= 1
    q.qtip_moe_plan_destroy(plan)
    for v in range(1, 9):
        plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, variant=v, arm_override=q.QTIP_ARM_GROUPED), "gfx950")
        sch = q.qtip_moe_plan_schedule(plan, 64)
        assert sch["gate_up"]["variant"] == v and sch["down"]["variant"] == v
        q.qtip_moe_plan_destroy(plan)


def test_default_kernel_shapes_follow_the_measured_rules():
    # V4 layer (E=256, k=6; 6, 11.9 and 23.2 woken experts at n = 1, 2, 4; grouped from 8).  GEMV fused
    # pass: 12 waves of 16-row tasks below 14000 32-row tasks (n <= 64), 8 waves of 32-row tasks
    # from there; GEMV down pass: 16 waves up to 6144 32-row tasks.  Grouped
    # picks by pairs per woken expert (1.41 at n=32, 3.15 at 128, 6.0 at 256, 12.0 at 512, 24.0 at
    # 1024).
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    want = {1: (11, 1), 2: (11, 1), 4: (11, 1), 8: (1, 3), 32: (1, 3), 128: (1, 7), 256: (9, 10), 512: (9, 10), 1024: (9, 10)}
    for n, (gu, dn) in want.items():
        s = q.qtip_moe_plan_schedule(plan, n)
        assert (s["gate_up"]["variant"], s["down"]["variant"]) == (gu, dn), n
    q.qtip_moe_plan_destroy(plan)
    # the GEMV arm forced past the floor: 12-wave 16-row tasks through n=64 (199.8 woken experts,
    # 12787 32-row tasks), 8-wave 32-row tasks from n=128 (243.8 woken, 15603)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, arm_override=q.QTIP_ARM_GEMV), "gfx950")
    for n, gu in {16: 11, 64: 11, 128: 4, 1024: 4}.items():
        assert q.qtip_moe_plan_schedule(plan, n)["gate_up"]["variant"] == gu, n
    q.qtip_moe_plan_destroy(plan)


def test_lut_rung_default_kernel_shapes_follow_its_own_sweep():
    # The LUT rung on the same V4 layer (GEMV up to 4 tokens, grouped from 5).  GEMV fused pass: 12
    # waves of 16-row tasks below 5 of them per CU (n=1), 16 waves from there; GEMV down pass: 32-row
    # tasks from 1536 of them (n >= 3).  Grouped fused
    # pass: 6 (12 waves, 32-row tasks) from 1.15 pairs per woken expert, 5 (8 waves, 64-row
    # tasks) from 8; grouped down pass: 7 (12 waves, 64-row tasks) throughout.
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, rung=q.QTIP_RUNG_LUT), "gfx950")
    want = {1: (11, 1), 2: (1, 1), 4: (1, 3), 8: (1, 7), 16: (6, 7), 32: (6, 7), 128: (6, 7), 256: (6, 7),
            512: (5, 7), 1024: (5, 7)}
    for n, (gu, dn) in want.items():
        s = q.qtip_moe_plan_schedule(plan, n)
        assert (s["gate_up"]["variant"], s["down"]["variant"]) == (gu, dn), n
    q.qtip_moe_plan_destroy(plan)


def test_router_argument_errors_return_before_any_launch():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    ws = q.qtip_moe_plan_info(plan)["workspace_bytes"]
    lib = q.lib()
    rl = lambda x, wr, n, lg, wsp, wsb: lib.qtip_moe_router_logits(plan, x, wr, n, lg, wsp, wsb, None)
    assert rl(256, 256, 0, 256, 256, ws) == q.QTIP_ERR_INVALID_CONFIG
    assert rl(256, 256, 1025, 256, 256, ws) == q.QTIP_ERR_INVALID_CONFIG
    assert rl(None, 256, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG
    assert rl(256, None, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG
    assert rl(256, 264, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG              # misaligned router weight
    assert rl(256, 256, 4, 256, 256, ws - 1) == q.QTIP_ERR_INVALID_ARG
    w = q.qtip_moe_weights(256, 256, 256, 256, 256, 256, 256)
    fh = lambda wr, x, n, out, wsp, wsb: lib.qtip_moe_forward_hidden(plan, ctypes.byref(w), wr, x, n, out, wsp, wsb,
                                                                      None)
    assert fh(None, 256, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG
    assert fh(264, 256, 4, 256, 256, ws) == q.QTIP_ERR_INVALID_ARG
    assert fh(256, 256, 0, 256, 256, ws) == q.QTIP_ERR_INVALID_CONFIG
    assert fh(256, 256, 4, 256, 256, ws - 1) == q.QTIP_ERR_INVALID_ARG
    q.qtip_moe_plan_destroy(plan)


def test_router_split_divides_the_input_blocks():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    # 32-expert x 32-token tiles, about 256 workgroups, at most 4 chunks: n=32 -> 8 tiles -> 4
    # chunks; n=1024 -> 256 tiles -> 1
    assert q.qtip_moe_router_split(plan, 32) == 4
    assert q.qtip_moe_router_split(plan, 1024) == 1
    for n in (1, 7, 33, 100, 683):
        S = q.qtip_moe_router_split(plan, n)
        assert S >= 1 and (4096 // 128) % S == 0
    assert q.qtip_moe_router_split(plan, 0) == -1
    q.qtip_moe_plan_destroy(plan)
    tiny = q.qtip_moe_plan_for_arch(q.make_desc(8, 2, 256, 128, 16), "gfx950")
    assert q.qtip_moe_router_split(tiny, 16) == 2
    q.qtip_moe_plan_destroy(tiny)


def test_gather_calibration_argument_errors():
    lib = q.lib()
    out = ctypes.c_double()
    assert lib.qtip_measure_lut_gather(100, None, 0, None, ctypes.byref(out)) == q.QTIP_ERR_INVALID_ARG
    assert lib.qtip_measure_lut_gather(0, 256, 1 << 20, None, ctypes.byref(out)) == q.QTIP_ERR_INVALID_CONFIG
    assert lib.qtip_measure_lut_gather(1 << 21, 256, 1 << 20, None, ctypes.byref(out)) == q.QTIP_ERR_INVALID_CONFIG


def test_offset_width_limits_are_enforced():
    with pytest.raises(q.QtipError) as ei:
        q.qtip_moe_plan_for_arch(q.make_desc(256, 8, 8192, 8192, 40000), "gfx950")
    assert ei.value.status == q.QTIP_ERR_INVALID_ARG


def test_workspace_holds_only_the_layouts_the_plan_can_take():
    ws = lambda mt, **kw: q.qtip_moe_plan_info(q.qtip_moe_plan_for_arch(q.make_desc(256, 6, 4096, 2048, mt, **kw),
                                                                      "gfx950"))["workspace_bytes"]
    # a decode-width plan (1.41 pairs per woken expert at n=32) never reaches the fragment layout
    assert ws(32) == ws(32, act_layout=q.QTIP_ACT_ROWS) < ws(32, act_layout=q.QTIP_ACT_FRAGMENTS)
    # at 1024 tokens (24 pairs) the automatic layout packs x: padded h and x buffers are added
    rows, auto = ws(1024, act_layout=q.QTIP_ACT_ROWS), ws(1024)
    P, PP = 1024 * 6, ((1024 * 6 + 15 * 256 + 15) // 16) * 16
    assert auto - rows >= (PP - P) * 2048 * 2 + PP * 4096 * 2
    # pinning the GEMV arm leaves the grouped layouts out
    assert ws(1024, arm_override=q.QTIP_ARM_GEMV) == rows


# ---- the boundary's closed-form predicate, counters and engagement log -------------------
SHAPES = [(6, 256, 16), (6, 256, 1), (2, 8, 16), (6, 8, 16), (8, 128, 16), (4, 64, 32), (1, 16, 4), (8, 256, 64)]


@pytest.mark.parametrize("k,E,thr", SHAPES)
def test_select_grouped_is_the_oracle_predicate(k, E, thr):
    # the pages' floor (8) set on the plan, so the closed form is the pages' predicate exactly
    plan = q.qtip_moe_plan_for_arch(q.make_desc(E, k, 256, 128, 4096, dispatch_tile_m=thr, decode_floor=8), "gfx950")
    for n in list(range(1, 40)) + [64, 127, 128, 512, 682, 683, 684, 1024, 1572, 2000, 4096]:
        assert q.qtip_moe_select_grouped(plan, n) == int(fill.select_grouped(n, k, E, thr)), (k, E, thr, n)
    n0 = fill.min_tokens_grouped(k, E, thr)
    if n0 <= 4096:
        assert q.qtip_moe_select_grouped(plan, n0) == 1 and q.qtip_moe_select_grouped(plan, n0 - 1) == 0
    assert q.qtip_moe_select_grouped(plan, 0) == -1
    q.qtip_moe_plan_destroy(plan)


def test_select_grouped_ignores_the_arm_pin():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, arm_override=q.QTIP_ARM_GEMV, dispatch_tile_m=16), "gfx950")
    assert q.qtip_moe_select_grouped(plan, 1024) == 1          # the closed form
    assert q.qtip_moe_select_arm(plan, 1024) == q.QTIP_ARM_GEMV  # the arm a forward takes
    q.qtip_moe_plan_destroy(plan)


def test_stats_start_at_zero_with_per_variant_slots():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    st = q.qtip_moe_stats(plan)
    assert st["forward_calls"] == 0 and st["last_arm"] == 0
    assert st["routed_in_gate_up"] == 0 and st["combined_in_down"] == 0
    assert st["gemv_variant_launches"] == [0] * 12 and st["grouped_variant_launches"] == [0] * 12
    q.qtip_moe_stats_reset(plan)
    assert ctypes.sizeof(q.qtip_moe_stats_t) == 7 * 8 + 2 * 4 + 2 * 12 * 8 + 2 * 8
    q.qtip_moe_plan_destroy(plan)


def test_log_engaged_prints_once_per_arm(capfd):
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, dispatch_tile_m=16), "gfx950")
    assert q.qtip_moe_log_engaged(plan, 1572) is True
    assert q.qtip_moe_log_engaged(plan, 2000) is False        # grouped again: already logged
    assert q.qtip_moe_log_engaged(plan, 32) is True           # first GEMV engagement
    err = capfd.readouterr().err.strip().splitlines()
    assert len(err) == 2
    pct = 100 * fill.pairs_per_woken_expert(1572, 6, 256) / 16
    assert "grouped arm for 1572 tokens" in err[0] and f"{pct:.1f}%" in err[0] and "grouped from 683" in err[0]
    assert "GEMV arm for 32 tokens" in err[1]
    with pytest.raises(q.QtipError):
        q.qtip_moe_log_engaged(plan, 0)
    q.qtip_moe_plan_destroy(plan)


def test_engaged_line_names_the_dequantize_arm():
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**{**V4, "max_tokens": 64}, arm_override=q.QTIP_ARM_DEQUANT), "gfx950")
    line = q.qtip_moe_engaged_line(plan, 32)
    assert line.startswith("qtip_moe: dequantize arm for 32 tokens") and "pinned" in line
    q.qtip_moe_plan_destroy(plan)
    # a window between the traffic ratio and a raised grouped threshold, reached by AUTO
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**{**V4, "max_tokens": 2048}, dispatch_tile_m=32), "gfx950")
    lo, hi = q.qtip_moe_dequant_range(plan)
    assert lo < hi and fill.select_arm(lo, 6, 256, 32) == "dequant"
    assert q.qtip_moe_engaged_line(plan, lo).startswith(f"qtip_moe: dequantize arm for {lo} tokens")
    q.qtip_moe_plan_destroy(plan)


def test_build_rejects_packed_fp32_in_device_assembly():
    from trellis_quantized_moe_expert_amd import build
    asm = "\tv_fmac_f32_e32 v1, v5, v7\n\tv_pk_fma_f32 v[0:1], v[4:5], v[6:7], s[0:1]\n; v_pk_add_f32 in a comment\n"
    assert build.packed_fp32_lines(asm) == ["v_pk_fma_f32 v[0:1], v[4:5], v[6:7], s[0:1]"]
    assert build.packed_fp32_lines("\tv_pk_mul_f16 v0, v1, v2\n\tv_add_f32 v0, v1, v2\n") == []
    cmd = build.compile_command("csrc/expert.hip", "/tmp/x.o")
    i = cmd.index("-target-feature")
    assert cmd[i - 1:i + 3] == ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    # the build kept the device assembly of the library it produced: none of it is packed FP32
    asm_dir = os.path.join(ROOT, "_build", "expert")
    if os.path.isdir(asm_dir):
        files = build.device_asm_files(asm_dir)
        assert files
        for f in files:
            assert build.packed_fp32_lines(open(f).read()) == [], f


def test_noalloc_refuses_layers_beyond_its_scratch_on_the_host():
    w = q.make_weights(*[256] * 7)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    with pytest.raises(q.QtipError) as ei:
        q.qtip_moe_forward_noalloc(plan, w, 256, 256, 406, 256)     # first V4 size past 64 MiB
    assert ei.value.status == q.QTIP_ERR_INVALID_CONFIG and "scratch" in str(ei.value)
    for n in (0, 1025):
        with pytest.raises(q.QtipError) as ei:
            q.qtip_moe_forward_noalloc(plan, w, 256, 256, n, 256)
        assert ei.value.status == q.QTIP_ERR_INVALID_CONFIG
    q.qtip_moe_plan_destroy(plan)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, arm_override=q.QTIP_ARM_DEQUANT), "gfx950")
    with pytest.raises(q.QtipError) as ei:
        q.qtip_moe_forward_noalloc(plan, w, 256, 256, 1, 256)       # dense weights never fit
    assert "scratch" in str(ei.value)
    q.qtip_moe_plan_destroy(plan)
    assert q.QTIP_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_dequantize_workspace_holds_only_the_woken_experts():
    # at most min(E, max_tokens * k) experts are woken, one dense slot each (3 matrices of H x I bf16)
    per_expert = 3 * 4096 * 2048 * 2
    for max_tokens, woken in ((1, 6), (32, 192), (43, 256), (1024, 256)):
        plan = q.qtip_moe_plan_for_arch(q.make_desc(**{**V4, "max_tokens": max_tokens},
                                                    arm_override=q.QTIP_ARM_DEQUANT), "gfx950")
        base = q.qtip_moe_plan_for_arch(q.make_desc(**{**V4, "max_tokens": max_tokens},
                                                    arm_override=q.QTIP_ARM_GEMV), "gfx950")
        extra = q.qtip_moe_plan_info(plan)["workspace_bytes"] - q.qtip_moe_plan_info(base)["workspace_bytes"]
        assert woken * per_expert <= extra < woken * per_expert + 4096, (max_tokens, extra)
        q.qtip_moe_plan_destroy(plan)
        q.qtip_moe_plan_destroy(base)


def test_small_gemv_batches_run_in_fewer_launches():
    # V4 (k = 6): the GEMV arm serves n <= 7 by default; a batch of at most 16 tokens and 64 pairs on
    # that arm is routed inside the gate+up launch, and a single token (256 token tasks of 16 rows:
    # one round on the CUs) is also combined inside the down launch (6 pairs x 2 input halves = 12
    # waves of the 16-wave down configuration), unless the plan asks for the separate kernels.
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4), "gfx950")
    s = q.qtip_moe_plan_schedule(plan, 1)
    assert (s["route_in_gate_up"], s["combine_in_down"]) == (1, 1)
    assert s["down"]["waves_per_workgroup"] == 16 and s["down"]["rows_per_task"] == 16
    for n in range(2, 8):
        s = q.qtip_moe_plan_schedule(plan, n)
        assert (s["route_in_gate_up"], s["combine_in_down"]) == (1, 0), n
    for n in (8, 16, 1024):
        s = q.qtip_moe_plan_schedule(plan, n)
        assert (s["route_in_gate_up"], s["combine_in_down"]) == (0, 0), n
    q.qtip_moe_plan_destroy(plan)
    # smaller rows: more tokens fit one round (H = 512: 32 tasks per token, 8 tokens)
    small = dict(num_experts=16, top_k=4, hidden=512, inter=256, max_tokens=32, arm_override=q.QTIP_ARM_GEMV)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**small), "gfx950")
    assert [q.qtip_moe_plan_schedule(plan, n)["combine_in_down"] for n in (1, 8, 9)] == [1, 1, 0]
    q.qtip_moe_plan_destroy(plan)
    # the LUT rung's default GEMV down configuration at n >= 3 (32-row tasks) cannot split its
    # inputs; at one token (16-row configuration) it can
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, rung=q.QTIP_RUNG_LUT), "gfx950")
    s = q.qtip_moe_plan_schedule(plan, 1)
    assert (s["route_in_gate_up"], s["combine_in_down"], s["down"]["variant"]) == (1, 1, 1)
    s = q.qtip_moe_plan_schedule(plan, 3)
    assert (s["route_in_gate_up"], s["combine_in_down"], s["down"]["variant"]) == (1, 0, 3)
    q.qtip_moe_plan_destroy(plan)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, arm_override=q.QTIP_ARM_GEMV), "gfx950")
    assert [q.qtip_moe_plan_schedule(plan, n)["route_in_gate_up"] for n in (10, 11, 16, 17)] == [1, 0, 0, 0]
    q.qtip_moe_plan_destroy(plan)
    small = dict(num_experts=16, top_k=4, hidden=256, inter=128, max_tokens=32, arm_override=q.QTIP_ARM_GEMV)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**small), "gfx950")
    assert [q.qtip_moe_plan_schedule(plan, n)["route_in_gate_up"] for n in (1, 16, 17)] == [1, 1, 0]
    q.qtip_moe_plan_destroy(plan)
    # a forced kernel configuration that cannot split its inputs keeps the combine kernel
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, variant=4), "gfx950")
    s = q.qtip_moe_plan_schedule(plan, 1)
    assert (s["route_in_gate_up"], s["combine_in_down"], s["down"]["variant"]) == (1, 0, 4)
    q.qtip_moe_plan_destroy(plan)
    # top-k above the down configuration's waves keeps the combine kernel
    wide = dict(num_experts=64, top_k=20, hidden=256, inter=256, max_tokens=8)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**wide, arm_override=q.QTIP_ARM_GEMV), "gfx950")
    s = q.qtip_moe_plan_schedule(plan, 2)
    assert (s["route_in_gate_up"], s["combine_in_down"]) == (1, 0)
    q.qtip_moe_plan_destroy(plan)
    plan = q.qtip_moe_plan_for_arch(q.make_desc(**V4, small_batch=q.QTIP_SMALL_BATCH_SEPARATE), "gfx950")
    s = q.qtip_moe_plan_schedule(plan, 1)
    assert (s["route_in_gate_up"], s["combine_in_down"]) == (0, 0)
    q.qtip_moe_plan_destroy(plan)
    with pytest.raises(q.QtipError) as ei:
        q.qtip_moe_plan_for_arch(q.make_desc(**V4, small_batch=2), "gfx950")
    assert ei.value.status == q.QTIP_ERR_INVALID_ARG
