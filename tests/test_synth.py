"""The seeded input generator: determinism, distribution and structure (CPU)."""

import numpy as np

import synth


def test_fmix32_known_values():
    # MurmurHash3 fmix32 is a bijection with fmix32(0) == 0; spot-check a few
    # values against a straightforward Python-int evaluation.
    def ref(h):
        h ^= h >> 16
        h = (h * 0x85EBCA6B) & 0xFFFFFFFF
        h ^= h >> 13
        h = (h * 0xC2B2AE35) & 0xFFFFFFFF
        h ^= h >> 16
        return h
    xs = np.array([0, 1, 2, 12345, 0xFFFFFFFF, 0x80000000, 0xDEADBEEF], dtype=np.uint32)
    assert synth.fmix32(xs).tolist() == [ref(int(x)) for x in xs]


def test_table_is_a_bf16_normal():
    t = synth.normal_table(1.0)
    v = (t.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.diff(v) >= 0)
    assert np.array_equal(v, -v[::-1])
    assert abs(v.mean()) < 1e-6 and abs(v.std() - 1.0) < 2e-3
    h = (synth.normal_table(0.5).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(h.astype(np.float64), v * 0.5)


def test_values_are_deterministic_and_regenerable_per_request():
    a = synth.mixed_8req()
    b = synth.mixed_8req()
    assert np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.pool_tags, b.pool_tags)
    x = a.kv_bits(0, "k", 3, 0, 40)
    assert np.array_equal(x, b.kv_bits(0, "k", 3, 0, 40))
    assert np.array_equal(x[10:20], a.kv_bits(0, "k", 3, 10, 20))
    assert not np.array_equal(x, a.kv_bits(0, "v", 3, 0, 40))
    assert not np.array_equal(x, a.kv_bits(0, "k", 4, 0, 40))
    assert np.array_equal(a.new_token_bits(0, "k", 0)[3], a.kv_bits(0, "k", 3, int(a.seq_lens0[3]),
                                                                   int(a.seq_lens0[3]) + 1)[0])


def test_value_statistics():
    wl = synth.mixed_8req()
    k = (wl.kv_bits(0, "k", 0, 0, 512).astype(np.uint32) << 16).view(np.float32)
    v = (wl.kv_bits(0, "v", 0, 0, 512).astype(np.uint32) << 16).view(np.float32)
    assert abs(k.std() - 1.0) < 0.01 and abs(v.std() - 0.5) < 0.005
    assert abs(k.mean()) < 0.01


def test_config_shapes():
    tiny = synth.tiny_1req()
    assert tiny.num_pages == 64 and tiny.block_table.shape == (1, 16)
    assert int(tiny.seq_lens_at(0)[0]) == 256
    assert len(set(tiny.block_table[0].tolist())) == 16
    mixed = synth.mixed_8req()
    L = mixed.seq_lens_at(0)
    assert L.min() >= 1024 and L.max() <= 8192
    assert mixed.num_pages == 2 * int(mixed.pages_allocated.sum())
    batch64 = synth.batch64_ctx8k()
    L = batch64.seq_lens_at(0)
    assert L.min() >= 8192 and L.max() <= 9192 and batch64.batch == 64 and batch64.num_layers == 8
    skewed = synth.skewed_16req()
    L = skewed.seq_lens_at(0)
    assert (L == 131072).sum() >= 2 and L.min() >= 512
    assert skewed.partition_tokens == 512
    # no physical page is owned twice
    for wl in (tiny, mixed, batch64, skewed):
        ids = np.concatenate([wl.block_table[b, :wl.pages_allocated[b]] for b in range(wl.batch)])
        assert len(np.unique(ids)) == len(ids)
        assert ids.min() >= 0 and ids.max() < wl.num_pages


def test_initial_scales_are_amax_over_448():
    wl = synth.tiny_1req()
    ks, vs = wl.initial_scales(0)
    k = (wl.kv_bits(0, "k", 0, 0, 255).astype(np.uint32) << 16).view(np.float32)
    assert ks.dtype == np.float32
    assert ks[0] == np.float32(np.abs(k).max()) / np.float32(448)
