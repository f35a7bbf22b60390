"""The comparison rule the GPU parity tests use (CPU only): the bf16
rounding helper agrees with torch's conversion, and the bar admits a bf16
output only when it is the rounding of a value within the bar."""
import numpy as np

from helpers import MAX_ABS, bf16_round, parity_stats


def test_bf16_round_matches_torch_conversion():
    import torch

    rng = np.random.Generator(np.random.PCG64(3))
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 7.0, 300.0)]).astype(np.float32)
    # halfway cases: a bf16 value plus half its unit, both signs
    b = torch.from_numpy(x[:2000]).to(torch.bfloat16).float().numpy()
    _, e = np.frexp(b.astype(np.float64))
    half = np.ldexp(1.0, e - 9)
    x = np.concatenate([x, (b + half).astype(np.float32), (-(b + half)).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bar_before_output_rounding():
    # ref 5.0: bf16 neighbours are 5 - 1/32 and 5 + 1/32 (unit 2^-5 in [4, 8))
    ref = np.array([5.0, 5.0, 5.0, 5.0, 0.5, 0.5])
    got = np.array([5.03125, 4.96875, 5.0625, 5.0, 0.5 + 6 / 256, 0.5 + 5 / 256])
    ok, mx, mn, only = parity_stats(got, ref, MAX_ABS, out_bf16=True)
    # 5 + 1/32 is bf16(5.0199...), a value within 2e-2 of 5: passes by the
    # second clause; 5 + 1/16 is two units away: fails; near 0.5 the unit is
    # 2^-8, so 0.5 + 6/256 (0.0234 away, not the rounding of anything within
    # 2e-2 of 0.5) fails and 0.5 + 5/256 (0.0195 away) passes by the first
    assert ok.tolist() == [True, True, False, True, False, True]
    assert only == 2
    ok32, _, _, _ = parity_stats(got, ref, MAX_ABS, out_bf16=False)
    assert ok32.tolist() == [False, False, False, True, False, True]
