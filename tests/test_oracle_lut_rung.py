"""Pins of the LUT rung's decode (oracle/lut_rung.py) and of the layer over LUT-rung experts.

The LUT rung's format is a reading (the pages name the rung, not its bits), so its pins are:
hand-derived states of hand-built streams (tests/golden/lut_rung_streams.txt), an exact integer
codebook decoded by hand, brute force against the vectorised decode, the identity with the
bitshift rung's already-pinned 16-bit window (the pair state is its low 9 bits at weight 2i), a
closed form for all-zero codes, and a separately written dense reference of the layer.  Planted
mutations (an off-by-one start bit, 8 index bits, MSB-first bits, swapped halves, no wrap, a
2-bit step) must each fail a pin."""
import numpy as np
import pytest

import golden_io
import moe_inputs
from oracle import lut_rung, moe, numerics, trellis


def _bytes(hexs):
    return np.frombuffer(bytes.fromhex(hexs), np.uint8)


def int_codebook():
    s = np.arange(512)
    return np.stack([s % 13 - 6, 7 - s % 11], axis=1).astype(np.float16)


def _pins_hold(pair_states, decode) -> bool:
    for rec in golden_io.records("lut_rung_streams.txt"):
        kind, hexs, _, *vals = rec
        row = _bytes(hexs)
        if kind == "pairs":
            if [int(v) for v in pair_states(row[None, :])[0]] != [int(v) for v in vals]:
                return False
        elif kind == "weights":
            got = decode(row[None, :], int_codebook())[0]
            if not np.array_equal(got, np.array([float(v) for v in vals])):
                return False
    rng = np.random.Generator(np.random.PCG64(5))
    codes = rng.integers(0, 256, (6, 32), dtype=np.uint8)
    win = trellis.window_states(codes)[:, ::2] & 0x1FF
    return bool(np.array_equal(pair_states(codes), win))


def test_golden_streams_and_integer_codebook():
    assert _pins_hold(lut_rung.pair_states, lut_rung.decode_declared)


def test_bruteforce_matches_vectorised_with_wrap():
    rng = np.random.Generator(np.random.PCG64(6))
    for nbytes in (2, 4, 32):
        codes = rng.integers(0, 256, (5, nbytes), dtype=np.uint8)
        st = lut_rung.pair_states(codes)
        for r in range(5):
            assert [lut_rung.pair_state_bruteforce(codes[r], i) for i in range(2 * nbytes)] == list(st[r])
    cb = rng.standard_normal((512, 2)).astype(np.float16)
    sc = rng.uniform(0.01, 0.05, 4).astype(np.float16)
    codes = rng.integers(0, 256, (4, 32), dtype=np.uint8)
    assert np.array_equal(lut_rung.dense_weights_bruteforce(codes, cb), lut_rung.decode_declared(codes, cb))
    assert np.allclose(lut_rung.dense_weights_bruteforce(codes, cb, sc, declared=False),
                       lut_rung.decode_exact(codes, cb, sc), rtol=0, atol=0)


def test_state_is_the_low_bits_of_the_bitshift_window():
    rng = np.random.Generator(np.random.PCG64(7))
    codes = rng.integers(0, 256, (3, 8, 64), dtype=np.uint8)
    assert np.array_equal(lut_rung.pair_states(codes), trellis.window_states(codes)[..., ::2] & 0x1FF)


def test_declared_values_are_the_bf16_codebook():
    rng = np.random.Generator(np.random.PCG64(8))
    cb = rng.standard_normal((512, 2)).astype(np.float16)
    codes = rng.integers(0, 256, (16, 32), dtype=np.uint8)
    w = lut_rung.decode_declared(codes, cb)
    st = lut_rung.pair_states(codes)
    assert np.array_equal(w[:, 0::2], numerics.bf16_round(cb[st, 0].astype(np.float32)))
    assert np.array_equal(w[:, 1::2], numerics.bf16_round(cb[st, 1].astype(np.float32)))


def _shape(**kw):
    base = dict(num_experts=4, top_k=2, hidden=128, inter=128, n_tokens=6, rung="lut")
    base.update(kw)
    return moe_inputs.MoEShape(**base)


def test_all_zero_codes_closed_form():
    inp = moe_inputs.make_inputs(_shape(), seed=9)
    import dataclasses
    z = dataclasses.replace(inp, codes_gate=np.zeros_like(inp.codes_gate))
    b0, b1 = lut_rung.codebook_bf16(inp.lut)[0]
    xr = numerics.bf16_bits_to_f64(z.x_bf16)
    for e in range(4):
        wg = moe.decode_expert(z, e)[0]
        assert np.all(wg[:, 0::2] == b0) and np.all(wg[:, 1::2] == b1)
        g = xr @ wg.T
        closed = b0 * xr[:, 0::2].sum(axis=1) + b1 * xr[:, 1::2].sum(axis=1)
        assert np.allclose(g, closed[:, None], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["declared", "exact"])
def test_layer_equals_dense_reference(mode):
    inp = moe_inputs.make_inputs(_shape(n_tokens=5), seed=10)
    a = moe.moe_forward(inp, mode=mode)["out_f64"]
    b = moe.dense_reference(inp, mode=mode).astype(np.float64)
    assert np.allclose(a, b, rtol=1e-5, atol=1e-6)


def test_workload_draws_a_codebook_and_the_same_codes():
    a = moe_inputs.make_inputs(_shape(), seed=11)
    b = moe_inputs.make_inputs(_shape(rung="bitshift"), seed=11)
    assert a.lut.shape == (512, 2) and a.lut.dtype == np.float16 and b.lut.shape == (65536,)
    assert a.codes_gate.shape == b.codes_gate.shape


def _mut_states(start_shift=0, q=9, order="little", swap=False, wrap=True, step=4):
    def pair_states(codes):
        c = np.asarray(codes, np.uint8)
        bits = np.unpackbits(c, axis=-1, bitorder=order).astype(np.int64)
        nb = bits.shape[-1]
        starts = np.arange(0, nb, step)[: nb // 4]
        st = np.zeros(bits.shape[:-1] + (starts.size,), np.int64)
        for b in range(q):
            pos = starts + b + start_shift
            if wrap:
                st += bits[..., pos % nb] << b
            else:
                ok = pos < nb
                st += np.where(ok, bits[..., np.minimum(pos, nb - 1)], 0) << b
        return st

    def decode(codes, cb):
        w = lut_rung.codebook_bf16(cb)[pair_states(codes)]
        if swap:
            w = w[..., ::-1]
        return w.reshape(*w.shape[:-2], w.shape[-2] * 2)
    return pair_states, decode


MUTANTS = {
    "start bit off by one": dict(start_shift=1),
    "8 index bits": dict(q=8),
    "MSB-first bits": dict(order="big"),
    "pair halves swapped": dict(swap=True),
    "no wrap at the row end": dict(wrap=False),
    "2-bit step": dict(step=2),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mutations_are_caught(name):
    assert not _pins_hold(*_mut_states(**MUTANTS[name])), name


def test_unmutated_model_passes_the_mutation_harness():
    assert _pins_hold(*_mut_states())


def test_stored_rows_undoes_the_block_interleaved_storage():
    """Brute force on small matrices: each row byte is placed by the stated formula, one at a time,
    and stored_rows must give the rows back (a transposed axis or a wrong block size fails).  Both
    rungs store their matrices this way."""
    assert lut_rung.stored_rows is trellis.stored_rows
    rng = np.random.default_rng(5)
    for rows, cols in ((16, 128), (32, 256), (48, 384)):
        nb = cols // 4
        r_bytes = rng.integers(0, 256, size=(rows, nb), dtype=np.uint8)
        flat = np.zeros(rows * nb, np.uint8)
        for r in range(rows):
            for c in range(nb):
                k, cc = divmod(c, 32)
                flat[((r // 16) * (cols // 128) + k) * 512 + (r % 16) * 32 + cc] = r_bytes[r, c]
        assert np.array_equal(lut_rung.stored_rows(flat.reshape(rows, nb)), r_bytes), (rows, cols)
    experts = rng.integers(0, 256, size=(3, 32, 64), dtype=np.uint8)
    assert np.array_equal(lut_rung.stored_rows(experts)[1], lut_rung.stored_rows(experts[1]))
    odd = rng.integers(0, 256, size=(8, 32), dtype=np.uint8)  # not whole blocks: taken row by row
    assert np.array_equal(lut_rung.stored_rows(odd), odd)
