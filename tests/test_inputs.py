"""The seeded input generator: reproducible bytes and the stated recipe."""

import numpy as np

from fp8_block_scaled_quantize_amd import inputs


def test_reproducible_and_independent_streams():
    lin = inputs.WORKLOADS["tiny_fwd_128x256x256"]["linears"][0]
    a = inputs.linear_tensors(lin, seed=0)
    b = inputs.linear_tensors(lin, seed=0, which=("w",))
    assert np.array_equal(a["w"], b["w"])                 # a tensor does not depend on the others
    c = inputs.linear_tensors(lin, seed=1)
    assert not np.array_equal(a["x"], c["x"])


def test_outlier_columns_and_std():
    (g,) = inputs.tensor_streams(0, 1)
    x = inputs.bf16_normal(g, (2048, 4096), 1.0, 0.01)
    v = (x.astype(np.uint32) << 16).view(np.float32)
    col_std = v.std(axis=0)
    outliers = col_std > 5.0
    assert outliers.sum() == round(0.01 * 4096)
    assert abs(np.median(col_std) - 1.0) < 0.05
    assert abs(np.median(col_std[outliers]) - 20.0) < 1.5


def test_bf16_rounding_of_generator_is_nearest_even():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8 - 2.0 ** -20], dtype=np.float32)
    bits = inputs.f32_to_bf16_bits(v)
    assert list(bits) == [0x3F80, 0x3F82, 0xBF81]


def test_workload_shapes_are_group_aligned():
    for name, wl in inputs.WORKLOADS.items():
        for lin in wl["linears"]:
            assert lin["N"] % 128 == 0 and lin["K"] % 128 == 0, name
            if "wgrad" in wl["passes"]:
                assert lin["M"] % 128 == 0, name
