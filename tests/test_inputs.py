"""The seeded fp16 inputs stay inside the range the fp16 output tolerance of
the GPU parity tests is derived for (|v| <= 5.7: the bound 3 * 2^-11 * Vmax
on the rounding of P and of the output)."""
import synth_inputs as si


def test_fp16_value_range_behind_the_tolerance():
    for kw in ({}, dict(L=1000, H=4, D=128, seed=401), dict(L=1000, H=4, D=128, seed=402)):
        _, _, v = si.rolling_inputs(**kw)
        assert float(v.float().abs().max()) <= 5.7, kw
