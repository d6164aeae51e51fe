"""The seeded input generators (kda_inputs), on the CPU."""
import numpy as np
import pytest

import kda_inputs

torch = pytest.importorskip("torch")


def test_make_inputs_is_deterministic_and_shaped():
    w = kda_inputs.custom(seqlens=[5, 0, 40], H=3, state_dtype="bf16", seed=9)
    a, b = kda_inputs.make_inputs(w), kda_inputs.make_inputs(w)
    for n in ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "initial_state", "cu_seqlens"):
        assert np.array_equal(a[n], b[n]), n
    assert a["q"].shape == (1, 45, 3, 128) and a["q"].dtype == np.uint16
    assert a["beta"].shape == (1, 45, 3)
    assert a["initial_state"].shape == (3, 3, 128, 128) and a["initial_state"].dtype == np.uint16
    assert a["cu_seqlens"].tolist() == [0, 5, 5, 45] and a["cu_seqlens"].dtype == np.int32


def test_bf16_rounding_is_nearest_even():
    # bf16 keeps 7 fraction bits: at 1 the spacing is 2^-7, so 1 + 2^-8 and
    # 1 + 3 * 2^-8 are ties, which go to the even neighbour (1 and 1 + 2^-6)
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5],
                 dtype=np.float32)
    bits = kda_inputs.f32_to_bf16_bits(x)
    assert kda_inputs.bf16_bits_to_f32(bits).tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, 1.0 + 2.0 ** -7, -2.5]
    # and the same bits as torch's conversion, which the device generator uses
    y = np.random.Generator(np.random.PCG64(3)).standard_normal(4096, dtype=np.float32)
    assert np.array_equal(kda_inputs.f32_to_bf16_bits(y),
                          torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_device_inputs_deterministic_and_rounded_like_the_host_path():
    w = kda_inputs.custom(B=5, T=33, H=2, init_std=0.05, state_dtype="fp32", seed=7)
    a = kda_inputs.make_device_inputs(w, "cpu", rows_per_draw=2)
    b = kda_inputs.make_device_inputs(w, "cpu", rows_per_draw=2)
    for n in ("q", "k", "v", "g", "beta", "initial_state"):
        assert torch.equal(a[n], b[n]), n
    assert tuple(a["q"].shape) == (5, 33, 2, 128) and a["q"].dtype == torch.bfloat16
    assert tuple(a["beta"].shape) == (5, 33, 2) and a["beta"].dtype == torch.bfloat16
    assert tuple(a["initial_state"].shape) == (5, 2, 128, 128) and a["initial_state"].dtype == torch.float32
    # A_log and dt_bias follow the numpy draw of make_inputs (first two small draws of PCG64(seed))
    rng = np.random.Generator(np.random.PCG64(w.seed))
    assert np.array_equal(a["A_log"], rng.standard_normal(2, dtype=np.float32))
    assert np.array_equal(a["dt_bias"], rng.standard_normal((2, 128), dtype=np.float32) * np.float32(0.1))
    # the bf16 tensors are the generator's fp32 normals rounded to nearest even
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    first = torch.randn((2, 33, 2, 128), generator=gen, dtype=torch.float32)
    want = kda_inputs.f32_to_bf16_bits(first.numpy())
    assert np.array_equal(a["q"][:2].view(torch.int16).numpy().view(np.uint16), want)
    q = a["q"].float()
    assert abs(float(q.mean())) < 0.05 and abs(float(q.std()) - 1.0) < 0.05
    assert abs(float(a["initial_state"].std()) - 0.05) < 0.005


def test_device_inputs_reject_varlen_workloads():
    with pytest.raises(ValueError):
        kda_inputs.make_device_inputs(kda_inputs.custom(seqlens=[3, 4], H=1), "cpu")
