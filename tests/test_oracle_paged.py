"""Block-table cache model ("10.3 - KV cache implementation details", section 7.2) against the static
cache model: with each sequence owning consecutive blocks the pool is the static buffer re-indexed;
any permutation of physical blocks gives the same logical rows; shared blocks are shared rows."""

import numpy as np

from oracle import attention as att
from oracle.buffer import RefCache
from oracle.paged import RefPagedCache
from static_kv_cache_amd import synthetic


def ops(rng, B, Hkv, S, D, steps):
    """A prefill-sized append then single-row appends, as (k, v, cache_index) in bf16 bits."""
    out = [(synthetic.draw(rng, (B, Hkv, 20, D), "bf16"), synthetic.draw(rng, (B, Hkv, 20, D), "bf16"),
            np.zeros(B, dtype=np.int32))]
    for s in range(steps):
        out.append((synthetic.draw(rng, (B, Hkv, 1, D), "bf16"), synthetic.draw(rng, (B, Hkv, 1, D), "bf16"),
                    np.full(B, 20 + s, dtype=np.int32)))
    return out


def test_identity_table_is_the_static_buffer():
    rng = np.random.default_rng(0)
    B, Hkv, S, D, bs = 3, 2, 32, 8, 8
    W = S // bs
    table = np.arange(B * W, dtype=np.int32).reshape(B, W)
    paged = RefPagedCache(1, B * W, Hkv, bs, D, "bf16", S)
    static = RefCache(1, B, Hkv, S, D, "bf16")
    for k, v, ci in ops(rng, B, Hkv, S, D, 5):
        assert paged.append(0, k, v, ci, table) == static.append(0, k, v, ci) == []
    for b in range(B):
        for i in range(W):
            assert np.array_equal(paged.pool[0, :, b * W + i], static.buf[0, :, b, :, i * bs:(i + 1) * bs])
    kg, vg = paged.gather(0, table, B)
    assert np.array_equal(kg, static.keys(0)) and np.array_equal(vg, static.values(0))


def test_permuted_blocks_give_the_same_rows_and_decode():
    rng = np.random.default_rng(1)
    B, Hkv, H, S, D, bs = 3, 2, 8, 48, 16, 16
    W = S // bs
    ident = np.arange(B * W, dtype=np.int32).reshape(B, W)
    perm = rng.permutation(B * W + 5)[:B * W].astype(np.int32).reshape(B, W)  # spare blocks never used
    a = RefPagedCache(1, B * W, Hkv, bs, D, "bf16", S)
    p = RefPagedCache(1, B * W + 5, Hkv, bs, D, "bf16", S)
    for k, v, ci in ops(rng, B, Hkv, S, D, 7):
        a.append(0, k, v, ci, ident)
        p.append(0, k, v, ci, perm)
    ka, va = a.gather(0, ident, B)
    kp, vp = p.gather(0, perm, B)
    assert np.array_equal(ka, kp) and np.array_equal(va, vp)
    q = synthetic.draw(rng, (B, H, D), "bf16")
    n = [27, 1, 20]
    assert np.array_equal(att.decode_attention(q, ka, va, n, 0.25), att.decode_attention(q, kp, vp, n, 0.25))


def test_shared_prefix_blocks_are_shared_rows():
    rng = np.random.default_rng(2)
    B, Hkv, H, S, D, bs = 2, 1, 4, 32, 8, 8
    table = np.array([[0, 1, 2, 3], [0, 1, 4, 5]], dtype=np.int32)  # rows [0, 16) shared
    c = RefPagedCache(1, 6, Hkv, bs, D, "bf16", S)
    k = synthetic.draw(rng, (B, Hkv, 16, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, 16, D), "bf16")
    c.append(0, k[:1].repeat(2, axis=0), v[:1].repeat(2, axis=0), np.array([0, 0]), table)  # both write the prefix
    k2 = synthetic.draw(rng, (B, Hkv, 4, D), "bf16")
    v2 = synthetic.draw(rng, (B, Hkv, 4, D), "bf16")
    c.append(0, k2, v2, np.array([16, 16]), table)  # private suffixes
    kg, vg = c.gather(0, table, B)
    assert np.array_equal(kg[0, :, :16], kg[1, :, :16]) and not np.array_equal(kg[0, :, 16:20], kg[1, :, 16:20])
    q = synthetic.draw(rng, (1, H, D), "bf16").repeat(2, axis=0)
    o = att.decode_attention(q, kg, vg, [16, 16], 0.3)
    assert np.array_equal(o[0], o[1])  # the same prefix rows attended by both sequences


def test_out_of_range_appends_are_skipped():
    rng = np.random.default_rng(3)
    B, Hkv, S, D, bs = 3, 2, 16, 8, 8
    table = np.array([[0, 1], [2, -1], [3, 9]], dtype=np.int32)
    c = RefPagedCache(1, 4, Hkv, bs, D, "bf16", S)
    k = synthetic.draw(rng, (B, Hkv, 4, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, 4, D), "bf16")
    before = c.pool.copy()
    # b = 0 fits; b = 1 reaches block -1; b = 2 reaches block 9 (outside the pool)
    assert c.append(0, k, v, np.array([6, 6, 6]), table) == [1, 2]
    changed = np.argwhere(np.any(c.pool != before, axis=-1))
    assert {(int(x[2]), int(x[4])) for x in changed} == {(0, 6), (0, 7), (1, 0), (1, 1)}
    assert c.append(0, k, v, np.array([13, 10, 10]), table) == [0, 1, 2]  # 13 + 4 > 16; rows 10..13 reach blocks -1, 9
