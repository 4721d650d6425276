"""CPU checks of the input recipes (workloads/): the stress distribution
carries the rows the 1e-6 guard of "9-2 flash_attn_single_q_q8_neon" §2
segment 1 separates (max-abs exactly 1e-6, and the float just below), on
the numpy path and on the torch path the bench and the full-size GPU tests
draw from; and the draws are reproducible."""
import numpy as np

import workloads

G1 = np.float32(1e-6)
G0 = np.nextafter(np.float32(1e-6), np.float32(0))


def _maxabs_rows(x):
    return np.abs(np.asarray(x, np.float32).reshape(-1, x.shape[-1])).max(1)


def test_numpy_stress_rows_hit_both_sides_of_the_guard():
    w = workloads.WORKLOADS["qwen8b_b128_stress"]
    lens = np.array([40, 7, 100], np.int32)
    k, v = workloads.kv_host(w, lens)
    for x in (k, v):
        m = _maxabs_rows(x)
        assert np.any(m == G1) and np.any(m == G0)
        assert np.any(m == 0) and np.any((m > 0) & (m < 1e-5))


def test_torch_stress_rows_hit_both_sides_of_the_guard():
    import torch
    w = workloads.WORKLOADS["qwen8b_b128_stress"]
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    x = workloads.kv_pool_torch(w, 3000, g, "cpu").numpy()
    m = _maxabs_rows(x)
    assert (m == G1).sum() >= 1 and (m == G0).sum() >= 1
    assert np.any(m == 0) and np.any((m > 0) & (m < 1e-5))
    c = workloads.kv_chunk_torch(w, 0, 3, 1, 0, "cpu").numpy()
    m = _maxabs_rows(c)
    assert np.any(m == G1) and np.any(m == G0)
    # the same key gives the same chunk
    np.testing.assert_array_equal(c, workloads.kv_chunk_torch(w, 0, 3, 1, 0, "cpu").numpy())


def test_normal_draws_have_no_injected_rows():
    import torch
    w = workloads.WORKLOADS["qwen2b_b64_ragged"]
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    m = _maxabs_rows(workloads.kv_pool_torch(w, 500, g, "cpu").numpy())
    assert m.min() > 0.5
