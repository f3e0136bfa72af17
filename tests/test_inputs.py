"""The seeded input recipe: 16-bit and fp8 operands are round-to-nearest-
even roundings of the float32 N(0, 1) draws (torch's conversions), pinned
here on values whose correct rounding is worked out by hand."""
import torch


def test_fp8_e4m3_conversion_is_round_to_nearest_even():
    # E4M3 near 1: steps of 1/8. 1.0625 lies halfway between 1.0 (mantissa
    # 000) and 1.125 (001): the even neighbour is 1.0. 1.1875 lies halfway
    # between 1.125 (001) and 1.25 (010): 1.25. 1.07 rounds to the nearer 1.125.
    # Subnormal range: the smallest step is 2^-9; 3 * 2^-10 lies halfway
    # between 2^-9 (001) and 2^-8 (010): 2^-8.
    x = torch.tensor([1.0625, 1.1875, 1.07, -1.0625, 3 * 2.0 ** -10, 448.0])
    got = x.to(torch.float8_e4m3fn).to(torch.float64).tolist()
    assert got == [1.0, 1.25, 1.125, -1.0, 2.0 ** -8, 448.0]


def test_bf16_conversion_is_round_to_nearest_even():
    # bf16 near 1: steps of 2^-7; 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    # (even: 1); 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 (even: 1 + 2^-6)
    x = torch.tensor([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])
    assert x.to(torch.bfloat16).to(torch.float64).tolist() == [1.0, 1 + 2.0 ** -6]
