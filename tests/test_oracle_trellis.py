"""Pins for the oracle's trellis decode (bit layout, window state, run decode, LUT narrowing).

Pinned against: hand-derived states of hand-built streams (tests/golden/trellis_streams.txt),
the run-decode identity (seed once then step == per-symbol window, the contiguous-run decode
of the arch-specialise page, PR #99, "The two levers" item 2), and planted mutations
(off-by-one symbol, wrong state mask, off-by-one seed, shift-by-one), which the pages list as
the mistake classes a decode test must catch ("Verification status").
"""
import numpy as np
import pytest

from golden_io import records
from oracle import numerics, trellis


def _fixture_streams():
    syms, states = [], []
    for rec in records("trellis_streams.txt"):
        kind, hexbytes, colon, *vals = rec
        assert colon == ":"
        b = bytes.fromhex(hexbytes)
        (syms if kind == "symbols" else states).append((b, [int(v) for v in vals]))
    return syms, states


SYMS, STATES = _fixture_streams()


@pytest.mark.parametrize("b,expect", SYMS)
def test_symbols_bruteforce_fixture(b, expect):
    assert trellis.symbols_bruteforce(b) == expect


@pytest.mark.parametrize("b,expect", SYMS)
def test_unpack_symbols_fixture(b, expect):
    got = trellis.unpack_symbols(np.frombuffer(b, np.uint8)[None, :])[0]
    assert got.tolist() == expect


@pytest.mark.parametrize("b,expect", STATES)
def test_window_state_fixture(b, expect):
    syms = trellis.symbols_bruteforce(b)
    assert [trellis.window_state_bruteforce(syms, c) for c in range(len(syms))] == expect
    assert trellis.window_states(np.frombuffer(b, np.uint8)[None, :])[0].tolist() == expect


@pytest.mark.parametrize("b,expect", STATES)
def test_run_states_fixture_every_start(b, expect):
    syms = trellis.symbols_bruteforce(b)
    cols = len(syms)
    for c0 in range(cols):
        got = trellis.run_states(syms, c0, cols)
        assert got == [expect[(c0 + i) % cols] for i in range(cols)]


def test_vectorised_matches_bruteforce_random_rows():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(5, 24), dtype=np.uint8)   # cols = 96
    vec = trellis.window_states(codes)
    for r in range(codes.shape[0]):
        syms = trellis.symbols_bruteforce(codes[r])
        assert vec[r].tolist() == [trellis.window_state_bruteforce(syms, c) for c in range(96)]


def test_run_decode_identity_runs_of_32_including_wrap():
    rng = np.random.default_rng(11)
    row = rng.integers(0, 256, size=64, dtype=np.uint8)         # cols = 256
    syms = trellis.symbols_bruteforce(row)
    full = trellis.window_states(row[None, :])[0].tolist()
    for c0 in range(0, 256, 32):                                 # every 32-symbol run, last wraps
        assert trellis.run_states(syms, c0, 32) == full[c0:c0 + 32]
    for c0 in (249, 250, 255):                                   # runs starting in the wrap region
        run = trellis.run_states(syms, c0, 20)
        assert run == [full[(c0 + i) % 256] for i in range(20)]


def test_states_are_16_bit_and_cover_all_values():
    rng = np.random.default_rng(3)
    st = trellis.window_states(rng.integers(0, 256, size=(64, 1024), dtype=np.uint8))
    assert st.min() >= 0 and st.max() <= 0xFFFF
    # uniform random bits: every state value appears (262144 draws over 65536 values)
    assert np.unique(st).size > 65536 * 0.97


def test_lut_bf16_matches_torch_rounding():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    lut = rng.standard_normal(65536).astype(np.float16)
    ours = trellis.lut_bf16(lut)
    ref = torch.from_numpy(lut.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_round_ties_to_even_cases():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1 + 2^-7: ties go to even (1.0)
    assert numerics.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even): goes up
    assert numerics.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert numerics.bf16_round(-2.5) == -2.5
    assert numerics.bf16_round(1.0 + 2.0 ** -9) == 1.0


def test_decode_exact_applies_row_scale():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, size=(3, 8), dtype=np.uint8)
    lut = rng.standard_normal(65536).astype(np.float16)
    scales = np.array([0.5, 0.25, 2.0], np.float16)
    w = trellis.decode_exact(codes, lut, scales)
    for r in range(3):
        syms = trellis.symbols_bruteforce(codes[r])
        for c in (0, 7, 31):
            s = trellis.window_state_bruteforce(syms, c)
            assert w[r, c] == float(lut[s]) * float(scales[r])


# ------------------------------- planted mutations -------------------------------------
def _check_all_fixture_pins():
    for b, expect in SYMS:
        assert trellis.symbols_bruteforce(b) == expect
    for b, expect in STATES:
        syms = trellis.symbols_bruteforce(b)
        assert [trellis.window_state_bruteforce(syms, c) for c in range(len(syms))] == expect
        for c0 in range(len(syms)):
            got = trellis.run_states(syms, c0, len(syms))
            assert got == [expect[(c0 + i) % len(syms)] for i in range(len(syms))]


def _mut_run_off_by_one_symbol(syms, c0, length):
    cols = len(syms)
    state = trellis.window_state_bruteforce(syms, c0)
    out = [state]
    for i in range(1, length):
        state = (state >> 2) | (syms[(c0 + i + 8) % cols] << 14)     # one symbol too far ahead
        out.append(state)
    return out


def _mut_run_wrong_mask(syms, c0, length):
    cols = len(syms)
    state = trellis.window_state_bruteforce(syms, c0)
    out = [state]
    for i in range(1, length):
        state = ((state << 0) >> 2) | (syms[(c0 + i + 7) % cols] << 14)
        state &= 0x7FFF                                                # drops the top bit
        out.append(state)
    return out


def _mut_run_off_by_one_seed(syms, c0, length):
    cols = len(syms)
    state = trellis.window_state_bruteforce(syms, (c0 + 1) % cols)    # seeded one symbol late
    out = [state]
    for i in range(1, length):
        state = (state >> 2) | (syms[(c0 + i + 7) % cols] << 14)
        out.append(state)
    return out


def _mut_run_shift_by_one(syms, c0, length):
    cols = len(syms)
    state = trellis.window_state_bruteforce(syms, c0)
    out = [state]
    for i in range(1, length):
        state = ((state >> 1) | (syms[(c0 + i + 7) % cols] << 14)) & 0xFFFF   # shifts one bit
        out.append(state)
    return out


def _mut_window_lsb_misordered(syms, c):
    cols = len(syms)
    return sum(syms[(c + j) % cols] * 4 ** (7 - j) for j in range(8))      # window read backwards


def _mut_symbols_msb_first(row_bytes):
    out = []
    for b in row_bytes:
        for q in range(4):
            out.append((int(b) >> (6 - 2 * q)) & 3)
    return out


@pytest.mark.parametrize("name,fn", [
    ("run_states", _mut_run_off_by_one_symbol),
    ("run_states", _mut_run_wrong_mask),
    ("run_states", _mut_run_off_by_one_seed),
    ("run_states", _mut_run_shift_by_one),
    ("window_state_bruteforce", _mut_window_lsb_misordered),
    ("symbols_bruteforce", _mut_symbols_msb_first),
])
def test_planted_mutation_is_caught(monkeypatch, name, fn):
    _check_all_fixture_pins()                       # the unmutated oracle passes
    monkeypatch.setattr(trellis, name, fn)
    with pytest.raises(AssertionError):
        _check_all_fixture_pins()
