"""The shared input generator: numpy and torch draws agree bit for bit."""
import numpy as np
import pytest
import torch

from workloads import values


@pytest.mark.parametrize("dtype", values.DTYPES)
def test_numpy_and_torch_draws_identical(dtype):
    ids = np.array([0, 1, 7, 123456, 2**33 + 5, 10**10], dtype=np.int64)
    a = values.draw_np(5, values.STREAM_K, ids, 3, 16, dtype)
    b = values.draw_torch(5, values.STREAM_K, ids, 3, 16, dtype, "cpu")
    if dtype == "f32":
        assert np.array_equal(a, b.numpy())
    else:
        assert np.array_equal(a, b.view(torch.int16).numpy().view(np.uint16))


def test_streams_and_seeds_differ():
    a = values.draw_np(1, values.STREAM_K, np.arange(64), 2, 16, "f32")
    assert not np.array_equal(a, values.draw_np(1, values.STREAM_V, np.arange(64), 2, 16, "f32"))
    assert not np.array_equal(a, values.draw_np(2, values.STREAM_K, np.arange(64), 2, 16, "f32"))
    assert np.array_equal(a, values.draw_np(1, values.STREAM_K, np.arange(64), 2, 16, "f32"))


def test_standard_normal_moments():
    x = values.draw_np(9, values.STREAM_Q, np.arange(4096), 4, 64, "f32").astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert np.abs(x).max() < 4.4


def test_head_subset_matches_full_draw():
    full = values.draw_np(3, values.STREAM_V, np.arange(50), 5, 16, "bf16")
    sub = values.draw_np(3, values.STREAM_V, np.arange(50), 5, 16, "bf16", heads=[4, 1])
    assert np.array_equal(sub, full[:, [4, 1]])
