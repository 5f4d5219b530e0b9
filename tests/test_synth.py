"""The input generators' own pins (CPU): values any consumer relies on."""
import numpy as np

import synth


def test_bf16_input_rounding():
    """The BF16 scorer's inputs: float32 rounded to the nearest bfloat16, ties
    to even (hand-worked bit patterns), and read back exactly."""
    x = np.array([1.0, -2.5, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, 0.0, -0.0],
                 np.float32)
    # 1.0 = 0x3F80; -2.5 = 0xC020; 1 + 2^-8 is halfway between 0x3F80 and 0x3F81:
    # ties to even -> 0x3F80; 1 + 3*2^-8 is halfway between 0x3F81 and 0x3F82 -> 0x3F82;
    # just above the first halfway point -> 0x3F81.
    assert synth.bf16_bits(x).tolist() == [0x3F80, 0xC020, 0x3F80, 0x3F82, 0x3F81, 0x0000, 0x8000]
    back = synth.bf16_values(np.array([0x3F80, 0x3F81, 0xC020], np.uint16))
    assert back.tolist() == [1.0, 1.0 + 2.0 ** -7, -2.5]


def test_bf16_rounding_error_bound():
    """Round to nearest: every value moves by at most half a bfloat16 ulp
    (2^-8 of its binade), and values already in bfloat16 do not move."""
    x = synth.normal("pin/bf16/x", (100000,)) * 3.0
    y = synth.bf16_values(synth.bf16_bits(x)).astype(np.float64)
    e = np.abs(y - x.astype(np.float64))
    ulp_half = 2.0 ** (np.floor(np.log2(np.abs(x.astype(np.float64)))) - 8)
    assert (e <= ulp_half).all()
    assert (synth.bf16_bits(y.astype(np.float32)) == synth.bf16_bits(x)).all()
