"""Pins of the oracle's pieces against closed forms, invariants and library
routines (CPU only).  Each test names the plausible mistake it would catch."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc

pytestmark = pytest.mark.filterwarnings("ignore")


def _bits_of_f32(vals):
    return torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- bf16

def test_bf16_widen_all_patterns_match_torch():
    # every bf16 bit pattern widens exactly as torch's bf16 -> float64
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_to_f64(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_round_matches_torch_on_fp32_values():
    # for fp32-representable inputs, one-step RNE to bf16 equals torch's conversion
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    got = orc.f64_to_bf16(v.astype(np.float64))
    assert np.array_equal(got, _bits_of_f32(v))


def test_bf16_round_half_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert orc.f64_to_bf16(1.0 + 2.0 ** -8)[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> rounds up
    assert orc.f64_to_bf16(1.0 + 3 * 2.0 ** -8)[0] == 0x3F82
    # just above the half rounds up
    assert orc.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30)[0] == 0x3F81
    assert orc.f64_to_bf16(-2.5)[0] == 0xC020
    assert orc.f64_to_bf16(0.0)[0] == 0 and orc.f64_to_bf16(-0.0)[0] == 0x8000


# ---------------------------------------------------------------- matvec

def test_matvec_matches_numpy_nonsquare():
    # catches a transposed operand or a dropped term
    rng = np.random.default_rng(2)
    W = rng.standard_normal((37, 53)).astype(np.float32)
    Wb = _bits_of_f32(W).reshape(37, 53)
    x = rng.standard_normal(53)
    Wd = orc.bf16_to_f64(Wb.ravel()).reshape(37, 53)
    ref = Wd @ x
    got = orc.matvec(Wb, x)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("eps", [1e-5, 1e-2, 0.5])
def test_rmsnorm_output_rms_closed_form(eps):
    # before the gain the output's RMS is sqrt(ms / (ms + eps)): pins eps inside the sqrt
    rng = np.random.default_rng(3)
    x = rng.standard_normal(256) * 0.3
    y = orc.rmsnorm(x, None, eps)
    ms = np.mean(x * x)
    assert math.isclose(np.sqrt(np.mean(y * y)), math.sqrt(ms / (ms + eps)), rel_tol=1e-12)
    # direction is preserved
    assert np.allclose(y / np.linalg.norm(y), x / np.linalg.norm(x), rtol=1e-12, atol=1e-15)


def test_rmsnorm_gain_is_elementwise_and_scale_invariant():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(64)
    g = (1.0 + 0.5 * rng.standard_normal(64)).astype(np.float32)
    gb = _bits_of_f32(g)
    gd = orc.bf16_to_f64(gb)
    y0 = orc.rmsnorm(x, None, 1e-5)
    y = orc.rmsnorm(x, gb, 1e-5)
    assert np.allclose(y, y0 * gd, rtol=1e-14, atol=0)
    # scaling: rmsnorm(a x) = x / sqrt(ms + eps / a^2), so it tends to x / rms(x)
    ms = np.mean(x * x)
    assert np.allclose(orc.rmsnorm(1000.0 * x, None, 1e-5), x / np.sqrt(ms + 1e-5 / 1e6), rtol=1e-12)
    assert np.allclose(orc.rmsnorm(1000.0 * x, None, 1e-5), x / np.sqrt(ms), rtol=1e-10)


# ---------------------------------------------------------------- RoPE

def _rope_complex(u, pos, theta):
    # textbook complex form: z_i = u_i + j u_{i+d/2} multiplied by exp(j pos theta^(-2i/d))
    d = u.size
    h = d // 2
    z = u[:h] + 1j * u[h:]
    ang = pos * theta ** (-2.0 * np.arange(h) / d)
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag])


@pytest.mark.parametrize("d,pos,theta", [(8, 5, 1e4), (64, 1023, 1e4), (128, 8255, 1e4), (64, 3, 5e5)])
def test_rope_matches_complex_rotation(d, pos, theta):
    rng = np.random.default_rng(5)
    u = rng.standard_normal(d)
    assert np.allclose(orc.rope(u, pos, theta), _rope_complex(u, pos, theta), rtol=1e-12, atol=1e-12)


def test_rope_identity_at_zero_and_norm_preserved():
    rng = np.random.default_rng(6)
    u = rng.standard_normal(64)
    assert np.array_equal(orc.rope(u, 0, 1e4), u)
    r = orc.rope(u, 777, 1e4)
    pairs0 = u[:32] ** 2 + u[32:] ** 2
    pairs1 = r[:32] ** 2 + r[32:] ** 2
    assert np.allclose(pairs0, pairs1, rtol=1e-12)


def test_rope_relative_position_invariance():
    # <R_m q, R_n k> = <R_{m-n} q, k>
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(10, 3), (1030, 1000), (5, 5)]:
        lhs = orc.rope(q, m, 1e4) @ orc.rope(k, n, 1e4)
        rhs = orc.rope(q, m - n, 1e4) @ k
        assert math.isclose(lhs, rhs, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_unit_vector_convention():
    # e_i goes to cos in slot i and sin in slot i + d/2 (rotate-half pairing, positive angle)
    d, pos, theta = 16, 7, 1e4
    for i in range(d // 2):
        e = np.zeros(d)
        e[i] = 1.0
        r = orc.rope(e, pos, theta)
        ang = pos * theta ** (-2 * i / d)
        want = np.zeros(d)
        want[i], want[i + d // 2] = math.cos(ang), math.sin(ang)
        assert np.allclose(r, want, atol=1e-15)


# ---------------------------------------------------------------- SiLU

def test_silu_closed_forms():
    assert orc.silu(0.0) == 0.0
    assert math.isclose(orc.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(orc.silu(1.0), 0.7310585786300049, rel_tol=1e-15)
    assert math.isclose(orc.silu(-1.0), -1.0 / (1.0 + math.e), rel_tol=1e-15)
    assert math.isclose(orc.silu(40.0), 40.0, rel_tol=1e-15)
    assert abs(orc.silu(-40.0)) < 1e-15
    # agrees with torch's SiLU in double
    z = np.linspace(-8, 8, 33)
    ref = torch.nn.functional.silu(torch.tensor(z, dtype=torch.float64)).numpy()
    assert np.allclose([orc.silu(v) for v in z], ref, rtol=1e-15, atol=1e-16)


# ---------------------------------------------------------------- attention

def test_attention_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(8)
    n, d = 37, 64
    k = rng.standard_normal(d)
    K = np.tile(k, (n, 1))
    V = rng.standard_normal((n, d))
    q = rng.standard_normal(d) * 3
    out, w = orc.attend(q, K, V, 1 / 8)
    assert np.allclose(w, 1.0 / n, rtol=1e-13)
    assert np.allclose(out, V.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_attention_dominant_key_and_single_position():
    rng = np.random.default_rng(9)
    n, d = 20, 8
    K = rng.standard_normal((n, d)) * 0.01
    V = rng.standard_normal((n, d))
    q = np.zeros(d)
    q[0] = 1.0
    K[13, 0] = 400.0  # score 400 * scale apart from the rest
    out, _ = orc.attend(q, K, V, 1 / math.sqrt(d))
    assert np.allclose(out, V[13], rtol=1e-12, atol=1e-12)
    out1, w1 = orc.attend(q, K[:1], V[:1], 1 / math.sqrt(d))
    assert np.array_equal(out1, V[0]) and w1[0] == 1.0


def test_attention_weight_ratio_closed_form_and_normalised():
    # two keys whose dot products with q differ by delta: weight ratio exp(delta * scale)
    d = 64
    q = np.zeros(d)
    q[3] = 2.0
    K = np.zeros((2, d))
    K[0, 3], K[1, 3] = 1.0, 2.5   # dots 2 and 5
    V = np.eye(2, d)
    scale = 1 / math.sqrt(d)
    out, w = orc.attend(q, K, V, scale)
    assert math.isclose(w[1] / w[0], math.exp(3.0 * scale), rel_tol=1e-13)
    assert math.isclose(w.sum(), 1.0, rel_tol=1e-15)
    rng = np.random.default_rng(10)
    for n in (1, 7, 300):
        _, w = orc.attend(rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d)), scale)
        assert math.isclose(w.sum(), 1.0, rel_tol=1e-13)


def test_attention_bf16_cache_reads_widened_values():
    # bf16 cache gives the same result as a float64 cache holding the widened values
    rng = np.random.default_rng(11)
    K = _bits_of_f32(rng.standard_normal((9, 16))).reshape(9, 16)
    V = _bits_of_f32(rng.standard_normal((9, 16))).reshape(9, 16)
    q = rng.standard_normal(16)
    a, _ = orc.attend(q, K, V, 0.25)
    b, _ = orc.attend(q, orc.bf16_to_f64(K.ravel()).reshape(9, 16), orc.bf16_to_f64(V.ravel()).reshape(9, 16), 0.25)
    assert np.array_equal(a, b)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(12)
    n, d = 50, 64
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    out, _ = orc.attend(q, K, V, 1 / 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None]).numpy().ravel()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- argmax

def test_argmax_lowest_index_tie_break_in_fp32():
    v = np.array([0.5, 2.0, -1.0, 2.0, 1.9])
    assert orc.argmax_f32(v) == 1
    # two doubles that round to the same fp32 value tie; the lower index wins
    a = 1.0 + 2.0 ** -30
    assert orc.argmax_f32(np.array([1.0, a])) == 0
    assert orc.argmax_f32(np.array([-5.0])) == 0
