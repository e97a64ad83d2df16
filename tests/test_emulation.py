"""Pins of the precision-emulating model (oracle/emulate.c) -- CPU only.

The model is checked against things that fix it independently: its rounding
against IEEE conversions numpy performs (fp32, fp16) and the bf16 routine of the
input generator; with every format set to fp64 it must reproduce the oracle's
plain definition; the two loop nests must agree bit for bit whenever the stored
state is not rounded below the arithmetic format; and deviation must shrink as
the significand widens.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import emulate as E


def test_rounding_matches_ieee_conversions():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-6, 6, 300),
                        [1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 65504.0, 65520.0, 6e-8, 3e-5, -0.0]])
    assert np.array_equal(E.round_fmt(x, "f32"), x.astype(np.float32).astype(np.float64))
    with np.errstate(over="ignore"):
        assert np.array_equal(E.round_fmt(x, "f16"), x.astype(np.float16).astype(np.float64))
    x32 = x.astype(np.float32)
    bf = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(x32))
    assert np.array_equal(E.round_fmt(x32.astype(np.float64), "bf16"), bf)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kv_outer", [False, True])
@pytest.mark.parametrize("bc,order", [(1, 0), (7, 1), (32, 0), (500, 1)])
def test_fp64_model_reproduces_the_definition(causal, kv_outer, bc, order):
    p = synth.make_qkv(1, 2, 257, 16, "f32", 21)
    rows = np.arange(0, 2 * 257, 5)
    ro, _ = oracle.attn_rows(p.q64, p.k64, p.v64, 0.3, rows, causal)
    e = E.flash_rows(p.q64, p.k64, p.v64, 0.3, rows, causal, acc="f64", p="f64", state="f64", out="f64",
                     bc=bc, order=order, kv_outer=kv_outer)
    assert np.abs(e - ro).max() < 1e-12
    b = E.baseline_rows(p.q64, p.k64, p.v64, 0.3, rows, causal, acc="f64", store="f64", out="f64")
    assert np.abs(b - ro).max() < 1e-12


def test_loop_nests_agree_without_stored_state_rounding():
    p = synth.make_qkv(1, 1, 200, 32, "bf16", 22)
    rows = np.arange(200)
    for order in (0, 1):
        a = E.flash_rows(p.q64, p.k64, p.v64, 0.2, rows, True, acc="f32", p="bf16", state="f32", bc=16,
                         order=order)
        b = E.flash_rows(p.q64, p.k64, p.v64, 0.2, rows, True, acc="f32", p="bf16", state="f32", bc=16,
                         order=order, kv_outer=True)
        assert np.array_equal(a, b)
    # rounding the stored state to bf16 changes the result
    c = E.flash_rows(p.q64, p.k64, p.v64, 0.2, rows, True, acc="f32", p="bf16", state="bf16", bc=16,
                     kv_outer=True)
    assert not np.array_equal(a, c)


def test_deviation_shrinks_with_the_significand():
    p = synth.make_qkv(1, 1, 256, 32, "f32", 23)
    rows = np.arange(0, 256, 3)
    ro, _ = oracle.attn_rows(p.q64, p.k64, p.v64, 0.18, rows, False)
    dev = []
    for bits in (6, 9, 12, 16, 20, 24):
        f = E.fmt_bits(bits)
        e = E.flash_rows(p.q64, p.k64, p.v64, 0.18, rows, False, acc=f, p=f, state=f, out=f, bc=32)
        dev.append(np.abs(e - ro).mean())
    assert all(a > b for a, b in zip(dev, dev[1:])), dev


def test_bad_arguments_are_rejected():
    p = synth.make_qkv(1, 1, 8, 4, "f32", 24)
    with pytest.raises(ValueError):
        E.flash_rows(p.q64, p.k64, p.v64, 1.0, [8], bc=4)
    with pytest.raises(ValueError):
        E.flash_rows(p.q64, p.k64, p.v64, 1.0, [0], bc=0)
    with pytest.raises(ValueError):
        E.baseline_rows(p.q64, p.k64, p.v64, 1.0, [-1])
