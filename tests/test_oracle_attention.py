"""Pins for the oracle's sparse attention."""
import numpy as np
import torch

from oracle.attention import attend, dense_reference


def _kv(H, T, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((H, T, d)), rng.standard_normal((H, T, d))


def test_attend_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((32, 128))
    k, v = _kv(4, 300, 128, 1)
    got = attend(q, k, v)
    qt = torch.from_numpy(q).reshape(4, 8, 1, 128)          # [Hkv][G][1][d]
    kt = torch.from_numpy(k).reshape(4, 1, 300, 128).expand(4, 8, 300, 128)
    vt = torch.from_numpy(v).reshape(4, 1, 300, 128).expand(4, 8, 300, 128)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(32, 128).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attend_equals_dense_reference():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((8, 128))
    k, v = _kv(1, 77, 128, 3)
    assert np.allclose(attend(q, k, v), dense_reference(q, k, v), rtol=1e-12, atol=1e-12)


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((8, 128))
    k = np.tile(rng.standard_normal((1, 1, 128)), (1, 50, 1))
    v = rng.standard_normal((1, 50, 128))
    out = attend(q, k, v)
    assert np.allclose(out, np.tile(v[0].mean(axis=0), (8, 1)), atol=1e-12)


def test_single_token_and_empty():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((8, 128))
    k, v = _kv(1, 1, 128, 6)
    assert np.allclose(attend(q, k, v), np.tile(v[0, 0], (8, 1)))
    e = np.zeros((1, 0, 128))
    assert not np.any(attend(q, e, e))
