"""The seeded input generator: determinism and round-to-nearest-even storage."""
import numpy as np
import torch

import synth


def test_bf16_rounding_ties_and_torch_agreement():
    # hand-picked float32 bit patterns: exact, below/above/at half, ties to even
    cases = {0x3F800000: 0x3F80, 0x3F807FFF: 0x3F80, 0x3F808000: 0x3F80, 0x3F808001: 0x3F81,
             0x3F818000: 0x3F82, 0xBF818000: 0xBF82, 0x00000000: 0x0000, 0x80000000: 0x8000}
    x = np.array(list(cases), np.uint32).view(np.float32)
    assert synth.f32_to_bf16_bits(x).tolist() == list(cases.values())
    r = np.random.default_rng([1, 2]).standard_normal(100000).astype(np.float32) * 37
    ours = synth.f32_to_bf16_bits(r)
    theirs = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(synth.bf16_bits_to_f64(ours),
                          torch.from_numpy(r).to(torch.bfloat16).to(torch.float64).numpy())


def test_generator_is_seeded_and_widening_is_exact():
    a = synth.make_qkv(1, 2, 33, 8, "bf16", 3)
    b = synth.make_qkv(1, 2, 33, 8, "bf16", 3)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    c = synth.make_qkv(1, 2, 33, 8, "bf16", 3, variant=1)
    assert not np.array_equal(a.q, c.q)
    for dt in synth.DTYPES:
        p = synth.make_qkv(2, 1, 9, 4, dt, 1, qk_factor=4.0)
        stored = p.k.astype(np.float64) if dt != "bf16" else synth.bf16_bits_to_f64(p.k)
        assert np.array_equal(stored, p.k64)
        assert p.q.shape == (2, 1, 9, 4)


def test_c2_mask_shape():
    m = synth.c2_mask(4, 1024)
    assert m.shape == (4, 1024) and m.dtype == np.uint8
    assert m[1].all() and not m[2].any() and not m[3].any()
    L = int((m[0] == 0).sum())
    assert 1 <= L <= 1024 and not m[0, :L].any() and m[0, L:].all()
