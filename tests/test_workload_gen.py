"""Pins for the seeded input generator (not the method): Philox4x64-10 from
its published definition, the grid tables, and the workload shapes."""
import numpy as np

from workload import gen, get_workload

M64 = (1 << 64) - 1


def _philox4x64_10(ctr, key):
    """Salmon et al. (SC 2011), Philox4x64 with 10 rounds."""
    c, k = list(ctr), list(key)
    for _ in range(10):
        p0 = 0xD2E7470EE14C6C93 * c[0]
        p1 = 0xCA5A826395121157 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & M64, (p0 >> 64) ^ c[3] ^ k[1], p0 & M64]
        k = [(k[0] + 0x9E3779B97F4A7C15) & M64, (k[1] + 0xBB67AE8584CAA73B) & M64]
    return c


def test_block_stream_is_philox_with_counter_from_one():
    key = gen.philox_key(gen.KIND_V, 1003, 7, 2, 123)
    raw = np.random.Philox(key=key).random_raw(12)
    exp = []
    for i in range(3):
        exp += _philox4x64_10([i + 1, 0, 0, 0], [int(key[0]), int(key[1])])
    assert [int(x) for x in raw] == exp


def test_block_ints_use_low_half_first():
    key = gen.philox_key(gen.KIND_K, 1001, 0, 0, 5)
    raw = _philox4x64_10([1, 0, 0, 0], [int(key[0]), int(key[1])])[0]
    u = [(raw >> (16 * i)) & 0xFFFF for i in range(4)]
    m = gen.block_ints(gen.KIND_K, 1001, 0, 0, 5, 16, 1, 128).reshape(-1)
    assert m[:4].tolist() == [int(gen.kv_table()[x]) for x in u]


def test_tables_are_symmetric_grid_normals():
    for tab, lim, sc in ((gen.kv_table(), 64, 16), (gen.q_table(), 128, 32)):
        assert tab.min() == -lim and tab.max() == lim
        assert np.array_equal(tab, -tab[::-1])
        assert abs(tab.astype(np.float64).std() / sc - 1.0) < 0.01


def test_queries_shapes_and_grid():
    wl = get_workload("c4s")
    q = gen.decode_queries(wl)
    assert q.shape == (wl.steps, wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim)
    assert np.all(np.mod(q * 32, 1) == 0) and np.abs(q).max() <= 4
    gen.to_bf16_bits(q)


def test_ar_queries_are_stationary_and_correlated():
    wl = get_workload("c2")
    q = gen.decode_queries(wl).astype(np.float64)
    assert abs(q.std() - 1.0) < 0.05
    a, b = q[:-1].reshape(-1), q[1:].reshape(-1)
    corr = np.corrcoef(a, b)[0, 1]
    assert abs(corr - 0.9 / np.sqrt(0.82)) < 0.02


def test_block_tables_partition_logical_space():
    wl = get_workload("c4")
    bt, npg = gen.block_tables(wl)
    ids = np.concatenate([bt[b, :npg[b]] for b in range(wl.batch)])
    assert np.array_equal(np.sort(ids), np.arange(wl.num_logical_pages))
    assert npg.tolist() == [512, 1536, 3072, 4096] and wl.num_logical_pages == 9216


def test_zipf_bias():
    wl = get_workload("c3")
    bias = gen.page_bias(wl)
    assert bias.shape == (3072,) and bias.max() == 0.0
    assert np.isclose(np.sort(bias)[0], np.float32(-1.1 * np.log(3072)))


def test_bf16_table_is_nearest_bf16_of_the_normal_quantiles():
    """Off-grid mode: each entry is the bf16 value nearest Phi^-1((u+.5)/65536)
    (ties to even), checked against a brute-force neighbour search."""
    from statistics import NormalDist
    tab = gen.bf16_table()
    nd = NormalDist()
    for u in (0, 1, 777, 32767, 32768, 40000, 65535):
        x = nd.inv_cdf((u + 0.5) / 65536.0)
        got = float((np.uint32(tab[u]) << 16).view(np.float32))
        f32 = np.float32(x)
        bits = int(f32.view(np.uint32)) >> 16
        cands = [float((np.uint32(b) << 16).view(np.float32)) for b in (bits - 1, bits, bits + 1)]
        best = min(cands, key=lambda c: abs(c - float(f32)))
        assert got == best
    v = (tab.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(v.std() - 1.0) < 0.01 and np.array_equal(v, -v[::-1])


def test_offgrid_workload_values_are_bf16_not_on_the_grid():
    wl = get_workload("c2s_bf16")
    k = gen.kv_page(wl, gen.KIND_K, 0, 0, 3)
    gen.to_bf16_bits(k)
    assert np.any(np.mod(k * 16, 1) != 0)
    q = gen.decode_queries(wl)
    gen.to_bf16_bits(q)
    assert np.any(np.mod(q * 32, 1) != 0)
