"""The seeded input generator (CPU only): bf16 rounding, page tables, pool
layout and determinism."""

import json
import os

import numpy as np
import torch

from paged_kv_cache_10_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_golden():
    with open(os.path.join(GOLDEN, "bf16_patterns.json")) as f:
        g = json.load(f)
    for src, dst in g["round"]:
        x = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)
        assert int(I.bf16_bits(x)[0]) == int(dst, 16), src


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(200000).astype(np.float32)
    x = np.concatenate([x, x * 1e-30, x * 1e30])
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.bf16_bits(x), t)


def test_draws_are_deterministic_and_distinct():
    w = I.workload("tiny", ctx_lens=[300])
    k1, v1 = I.draw_kv(w, 0, 0)
    k2, v2 = I.draw_kv(w, 0, 0)
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
    assert not np.array_equal(k1, v1)
    w2 = I.workload("tiny", ctx_lens=[300], num_layers=2)
    k3, _ = I.draw_kv(w2, 1, 0)
    assert not np.array_equal(k1, k3)


def test_boost_count_and_factor():
    w = I.workload("long262k", ctx_lens=[6400], num_layers=1)
    idx = I.boost_positions(w, 0, 0, 2, 6400)
    assert len(idx) == 64 and len(set(idx.tolist())) == 64
    k, _ = I.draw_kv(w, 0, 0)
    w0 = I.workload("long262k", ctx_lens=[6400], num_layers=1, boost_frac=0.0)
    k0, _ = I.draw_kv(w0, 0, 0)
    from oracle import widen_bf16
    a, b = widen_bf16(k[2, idx]), widen_bf16(k0[2, idx])
    np.testing.assert_array_equal(a, 4 * b)
    rest = np.setdiff1d(np.arange(6400), idx)
    np.testing.assert_array_equal(k[2, rest], k0[2, rest])


def test_page_tables_are_a_permutation_with_sinks():
    w = I.workload("mixed", num_layers=1)
    t = I.draw_page_tables(w)
    assert t.shape == (16, w.pt_stride) and t.dtype == np.int32
    used = []
    for b, n in enumerate(w.pages_per_req):
        assert np.all(t[b, :n] >= 0) and np.all(t[b, n:] == -1)
        assert t[b, 0] >= 0                               # sink page present
        used += t[b, :n].tolist()
    assert sorted(used) == list(range(w.num_pages))
    w2 = I.workload("conc", num_layers=1)
    t2 = I.draw_page_tables(w2)
    u2 = t2[t2 >= 0]
    assert len(u2) == 1984 and len(set(u2.tolist())) == 1984 and u2.max() < 2048


def test_mixed_lengths_in_range():
    w = I.workload("mixed")
    assert len(w.ctx_lens) == 16
    assert all(1024 <= c <= 131072 for c in w.ctx_lens)


def k_position(j, ch):
    """Storage position (in 16-byte pieces) of K's token j, channels
    8*(ch//8)..+7, inside a block, plus the element within the piece: the
    operand order of the decode kernel (32-token halves, two 16-row tiles,
    8 k-steps of 32 channels, 4 lane groups of 8 channels, 16 rows)."""
    half, jj = divmod(j, 32)
    tile = (jj % 8) // 4
    row = 4 * (jj // 8) + jj % 4
    kstep, rem = divmod(ch, 32)
    group, elem = divmod(rem, 8)
    return (((half * 2 + tile) * 8 + kstep) * 4 + group) * 16 + row, elem


def v_position(j, ch):
    """Storage position of V's channel ch, token j: pieces hold 8 tokens of
    one channel; 32-token halves, 16 channel blocks of 16, 4 lane groups."""
    half, jj = divmod(j, 32)
    group, elem = divmod(jj, 8)
    cblock, row = divmod(ch, 16)
    return ((half * 16 + cblock) * 4 + group) * 16 + row, elem


def test_pool_layout():
    """Layer-major arena; block at [layer][page][K|V][kv head]; pieces in
    the kernel's operand order."""
    w = I.Workload("t", seed=3, ctx_lens=[100, 70], num_layers=2, tile_tokens=64,
                   num_q_heads=8, num_kv_heads=2, head_dim=256)
    t = I.draw_page_tables(w)
    pool, kv = I.host_pool(w, t, fill=I.BF16_QNAN)
    assert pool.shape == (2, w.num_pages, 2, 2, 64 * 256)
    g = np.random.default_rng(0)
    for (layer, b), (k, v) in kv.items():
        for kvh in range(2):
            for j in [0, 1, 5, 31, 32, 63, 64, w.ctx_lens[b] - 1] + g.integers(0, 64, 6).tolist():
                if j >= w.ctx_lens[b]:
                    continue
                p = t[b, j // 64]
                for ch in [0, 7, 8, 100, 255] + g.integers(0, 256, 6).tolist():
                    pos, e = k_position(j % 64, ch)
                    assert pool[layer, p, 0, kvh, pos * 8 + e] == k[kvh, j, ch]
                    pos, e = v_position(j % 64, ch)
                    assert pool[layer, p, 1, kvh, pos * 8 + e] == v[kvh, j, ch]
    # padding past ctx in the last page keeps the poison pattern
    p = t[0, 1]
    pos, e = k_position(100 - 64, 3)
    assert pool[0, p, 0, 0, pos * 8 + e] == I.BF16_QNAN


def test_device_scatter_matches_host_layout():
    """The torch scatter used for full-size workloads writes the same layout."""
    w = I.Workload("t", seed=4, ctx_lens=[130, 64], num_layers=2, tile_tokens=64,
                   num_q_heads=4, num_kv_heads=2, head_dim=256)
    t = I.draw_page_tables(w)
    pool_h, kv = I.host_pool(w, t, fill=0)
    pool_d = torch.zeros(pool_h.shape, dtype=torch.int16)
    for (layer, b), (k, v) in kv.items():
        kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16)
        vt = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16)
        I.device_scatter(pool_d, w, layer, b, t[b], kt, vt)
    np.testing.assert_array_equal(pool_d.numpy().view(np.uint16), pool_h)


def test_stress_draws_forced_rows():
    d = I.stress_draws(batch=2, heads=3, tiles=32, keys=2, dim=4)
    assert d["empty"][0, 0].all()
    assert (~d["empty"][0, 1]).sum() == 1
    assert d["target_lse"].min() >= -40 and d["target_lse"].max() <= 40


def test_shorter_history_is_a_prefix():
    """Per-head streams: the K/V of a shorter history are the first rows of a
    longer one, which is what lets an appended token be checked bit for bit."""
    w = I.Workload("p", seed=8, ctx_lens=[70], num_layers=2, tile_tokens=64)
    w2 = I.Workload("p", seed=8, ctx_lens=[71], num_layers=2, tile_tokens=64)
    for layer in range(2):
        k, v = I.draw_kv(w, layer, 0)
        k2, v2 = I.draw_kv(w2, layer, 0)
        np.testing.assert_array_equal(k, k2[:, :70])
        np.testing.assert_array_equal(v, v2[:, :70])


def test_compact_block_maps_are_bijections_with_the_stated_offsets():
    for m in (I.KC_BYTES, I.VC_BYTES):
        assert sorted(m.ravel().tolist()) == list(range(64 * 256))
    # K: token 0 channels 0 / 32 share piece 0 (bytes 0 and 8); token 1 is
    # row 1 of the same tile (piece 1); token 4 is tile 1 (load 4, piece 256)
    assert I.KC_BYTES[0, 0] == 0 and I.KC_BYTES[0, 32] == 8 and I.KC_BYTES[0, 7] == 7
    assert I.KC_BYTES[1, 0] == 16 and I.KC_BYTES[4, 0] == 256 * 16
    assert I.KC_BYTES[0, 8] == 16 * 16 and I.KC_BYTES[0, 64] == 64 * 16
    # V: channel d is row d%16 of block d/16; tokens 8q.. in bytes 0..7, the
    # second half's tokens in bytes 8..15
    assert I.VC_BYTES[0, 0] == 0 and I.VC_BYTES[32, 0] == 8 and I.VC_BYTES[8, 0] == 16 * 16
    assert I.VC_BYTES[0, 1] == 16 and I.VC_BYTES[0, 16] == 64 * 16
    r = np.random.default_rng(1)
    c = r.integers(0, 256, (64, 256), dtype=np.uint8)
    for kind in "kv":
        np.testing.assert_array_equal(I.compact_block_codes(I.compact_block_image(c, kind), kind), c)
