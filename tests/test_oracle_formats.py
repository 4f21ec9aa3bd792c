"""The oracle's bf16 decode and round-to-nearest-even, pinned to torch and to hand-derived cases."""
import numpy as np
import torch

from oracle import brute as BR
from oracle.formats import bf16_bits_to_f64, f64_to_bf16_bits


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_bits_to_f64(bits)[finite], ref[finite])


def test_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(300_000) * np.exp(rng.uniform(-60, 60, 300_000))).astype(np.float32)
    u = x.view(np.uint32).copy()
    u[:5000] = (u[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)  # exact ties
    u[5000:6000] = rng.integers(1, 1 << 23, 1000).astype(np.uint32)  # float32 subnormals
    x = u.view(np.float32)
    assert np.array_equal(f64_to_bf16_bits(x.astype(np.float64)), _torch_bf16_bits(x))


def test_hand_derived_cases():
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,  # halfway between 1 and 1+2^-7: even significand (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,  # halfway between 1+2^-7 (odd) and 1+2^-6 (even)
        -(1.0 + 2.0 ** -8): 0xBF80,
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above the tie; a float32 step would lose this
        2.0 ** -134: 0x0000,  # half the smallest subnormal: ties to zero (even)
        3 * 2.0 ** -134: 0x0002,  # 1.5 spacings: ties to the even count 2
        0.0: 0x0000,
    }
    xs = np.array(list(cases), dtype=np.float64)
    want = np.array(list(cases.values()), dtype=np.uint16)
    assert np.array_equal(f64_to_bf16_bits(xs), want)
    assert [BR._round_bf16(float(v)) for v in xs] == [int(w) for w in want]


def test_rounding_agrees_with_brute_force_on_float64_values():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * 10.0 ** rng.uniform(-5, 5, 3000)
    assert [int(v) for v in f64_to_bf16_bits(x)] == [BR._round_bf16(float(v)) for v in x]
