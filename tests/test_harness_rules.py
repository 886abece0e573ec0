"""CPU checks of the parity harness's own arithmetic (tests/decode_harness.py):
its float64 -> bf16 rounding agrees with torch's conversion, and its ulp
distance with the bf16 ordering."""
import numpy as np
import torch

from decode_harness import bf16_to_f64, rne_bf16, ulp_diff_bf16


def test_rne_bf16_matches_torch_on_float32_values():
    g = torch.Generator().manual_seed(5)
    x = torch.cat([torch.randn(200000, generator=g) * s for s in (1e-3, 1.0, 37.0)])
    # exact ties between two bf16 values, both parities of the even neighbour
    b = torch.randint(0, 0x7F00, (20000,), generator=g, dtype=torch.int32)
    ties = ((b << 16) | 0x8000).view(torch.float32)
    x = torch.cat([x, ties, -ties])
    want = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = rne_bf16(x.to(torch.float64).numpy())
    assert np.array_equal(got, want)


def test_ulp_distance_counts_representable_steps():
    a = np.array([0x3F80, 0x3F80, 0xBF80, 0x0001, 0x8001], dtype=np.uint16)
    b = np.array([0x3F81, 0x3F7F, 0xBF81, 0x8001, 0x0002], dtype=np.uint16)
    assert ulp_diff_bf16(a, b).tolist() == [1, 1, 1, 2, 3]
    assert bf16_to_f64(np.array([0x3F80], dtype=np.uint16))[0] == 1.0
