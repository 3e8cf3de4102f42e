"""Block-table (paged) cache on the GPU ("10.3 - KV cache implementation details", section 7.2).

* kvc_paged_append writes the oracle's pool bit for bit through random (non-contiguous) block tables,
  for prefill-sized and single-row appends, and skips (and flags) sequences whose rows leave the
  capacity or reach a block outside the pool.
* kvc_paged_decode_attn matches the oracle's decode over the rows the tables map, within the bf16
  bound, on ragged lengths, empty sequences, every head_dim and block sizes 16..256.
* For any tables, its output bits equal those of the static cache's decode over the same logical
  rows with the same grid (the paged piece changes only where rows are loaded from).
* Shared prefix blocks are shared rows; entries outside the pool read as zeros and raise the flag.
"""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, say, to_f64, tol_check
from oracle import attention as oatt
from oracle.paged import RefPagedCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def random_tables(rng, B, W, nb):
    """An injective map of the B * W logical blocks onto a random subset of nb physical blocks."""
    return rng.permutation(nb)[:B * W].reshape(B, W).astype(np.int32)


def make(dev, B, H, Hkv, D, S, bs, nb):
    desc = kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16")
    return kvc.PagedCache(desc, bs, nb), RefPagedCache(1, nb, Hkv, bs, D, "bf16", S)


def pools_equal(cache, ref, layer=0):
    k, v = cache.layer_tensors(layer)
    return (np.array_equal(bits_of(k, "bf16"), ref.pool[layer, 0])
            and np.array_equal(bits_of(v, "bf16"), ref.pool[layer, 1]))


def fill_both(dev, cache, ref, rng, table, lens):
    """Append rows [0, max(lens)) to every sequence (one prefill-sized call), then return."""
    B, Hkv, D = cache.desc.batch, cache.desc.n_kv_heads, cache.desc.head_dim
    t = max(max(lens), 1)
    k = synthetic.draw(rng, (B, Hkv, t, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, t, D), "bf16")
    zero = np.zeros(B, dtype=np.int32)
    cache.paged_append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), kvc.to_device(table, dev),
                       kvc.to_device(zero, dev))
    assert ref.append(0, k, v, zero, table) == []
    return k, v


@pytest.mark.parametrize("bs,D", [(16, 128), (32, 64), (256, 128), (16, 256)])
def test_paged_append_bit_exact(bs, D):
    dev = device()
    rng = np.random.default_rng(bs + D)
    B, Hkv, S = 3, 2, 2 * 256
    W = S // bs
    nb = B * W + 7
    say(f"paged append: bs={bs} D={D}")
    cache, ref = make(dev, B, 4, Hkv, D, S, bs, nb)
    table = random_tables(rng, B, W, nb)
    tab = kvc.to_device(table, dev)
    # a prefill chunk that starts mid-block and crosses blocks, then single-row appends
    k = synthetic.draw(rng, (B, Hkv, 45, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, 45, D), "bf16")
    ci = np.array([3, 17, bs - 1], dtype=np.int32)
    cache.paged_append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), tab, kvc.to_device(ci, dev))
    assert ref.append(0, k, v, ci, table) == []
    for step in range(5):
        k1 = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
        v1 = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
        ci = np.array([48 + step, 62 + step, bs + 44 + step], dtype=np.int32)
        cache.paged_append(0, kvc.to_device(k1, dev), kvc.to_device(v1, dev), tab, kvc.to_device(ci, dev))
        assert ref.append(0, k1, v1, ci, table) == []
    cache.check()
    assert pools_equal(cache, ref)
    cache.free()


DECODE_SHAPES = [  # B, H, Hkv, D, S, bs, valid lengths
    (3, 8, 2, 128, 256, 16, [256, 1, 77]),      # GQA; full, one row, ragged
    (2, 4, 4, 64, 128, 32, [100, 0]),           # MHA; an empty sequence
    (2, 16, 1, 128, 96, 16, [96, 50]),          # MQA (G = 16)
    (1, 32, 1, 128, 64, 64, [64]),              # G = 32: two chunks of 16 heads
    (2, 8, 2, 256, 512, 256, [512, 300]),       # widest rows, largest blocks
    (2, 4, 2, 32, 64, 16, [33, 64]),            # narrowest rows
    (4, 8, 8, 64, 1024, 16, [1024, 1000, 513, 17]),
]


@pytest.mark.parametrize("B,H,Hkv,D,S,bs,lens", DECODE_SHAPES)
def test_paged_decode_matches_oracle(B, H, Hkv, D, S, bs, lens):
    dev = device()
    rng = np.random.default_rng(7 * S + D + bs)
    say(f"paged decode: B={B} H={H} Hkv={Hkv} D={D} S={S} bs={bs} lens={lens}")
    W = S // bs
    nb = B * W + 3
    cache, ref = make(dev, B, H, Hkv, D, S, bs, nb)
    table = random_tables(rng, B, W, nb)
    fill_both(dev, cache, ref, rng, table, lens)
    q = synthetic.draw(rng, (B, H, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    valid = np.array(lens, dtype=np.int32)
    cache.paged_decode_attn(0, kvc.to_device(q, dev), out, kvc.to_device(table, dev),
                            valid_lens=kvc.to_device(valid, dev), sm_scale=scale)
    cache.check()
    kg, vg = ref.gather(0, table, B)
    want = oatt.decode_attention(q, kg, vg, lens, scale)
    err = tol_check(to_f64(out), want, "bf16", "paged decode")
    say(f"  max abs err {err:.3e}")
    cache.free()


@pytest.mark.parametrize("wg", [0, 1, 7, 64])
def test_paged_decode_bits_equal_static_decode(wg):
    """Same logical rows, same grid: the paged and static decode give the same output bits."""
    dev = device()
    rng = np.random.default_rng(11 + wg)
    B, H, Hkv, D, S, bs = 4, 16, 4, 128, 1024, 16
    lens = [1024, 900, 1, 333]
    W = S // bs
    nb = B * W + 11
    say(f"paged vs static bits: workgroups={wg}")
    cache, ref = make(dev, B, H, Hkv, D, S, bs, nb)
    table = random_tables(rng, B, W, nb)
    k, v = fill_both(dev, cache, ref, rng, table, lens)
    static = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"))
    static.prefill_fill(0, kvc.to_device(k, dev), kvc.to_device(v, dev), 0)
    cache.set_workgroups(wg)
    static.set_workgroups(wg)
    q = kvc.to_device(synthetic.draw(rng, (B, H, D), "bf16"), dev)
    valid = kvc.to_device(np.array(lens, dtype=np.int32), dev)
    a = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    cache.paged_decode_attn(0, q, a, kvc.to_device(table, dev), valid_lens=valid, sm_scale=0.088)
    static.decode_attn(0, q, b, valid_lens=valid, sm_scale=0.088)
    cache.check()
    static.check()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    cache.free()
    static.free()


def test_shared_prefix_blocks():
    """Two sequences whose tables share their first blocks attend the same prefix rows; each
    then appends private rows into its own blocks."""
    dev = device()
    rng = np.random.default_rng(5)
    B, H, Hkv, D, S, bs = 2, 8, 2, 128, 128, 16
    table = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [0, 1, 2, 8, 9, 10, 11, 12]], dtype=np.int32)  # 48 rows shared
    cache, ref = make(dev, B, H, Hkv, D, S, bs, 13)
    tab = kvc.to_device(table, dev)
    pk = synthetic.draw(rng, (1, Hkv, 48, D), "bf16")
    pv = synthetic.draw(rng, (1, Hkv, 48, D), "bf16")
    # the prefix is written once, through sequence 0's table (sequence 1 skips: start past capacity)
    ci = np.array([0, S], dtype=np.int32)
    kk, vv = np.concatenate([pk, pk]), np.concatenate([pv, pv])
    cache.paged_append(0, kvc.to_device(kk, dev), kvc.to_device(vv, dev), tab, kvc.to_device(ci, dev))
    assert ref.append(0, kk, vv, ci, table) == [1]
    assert cache.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    sk = synthetic.draw(rng, (B, Hkv, 20, D), "bf16")
    sv = synthetic.draw(rng, (B, Hkv, 20, D), "bf16")
    ci = np.array([48, 48], dtype=np.int32)
    cache.paged_append(0, kvc.to_device(sk, dev), kvc.to_device(sv, dev), tab, kvc.to_device(ci, dev))
    assert ref.append(0, sk, sv, ci, table) == []
    cache.check()
    assert pools_equal(cache, ref)
    q = synthetic.draw(rng, (1, H, D), "bf16").repeat(2, axis=0)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / np.sqrt(D)
    for lens in ([48, 48], [68, 68], [30, 61]):
        cache.paged_decode_attn(0, kvc.to_device(q, dev), out, tab,
                                valid_lens=kvc.to_device(np.array(lens, dtype=np.int32), dev), sm_scale=scale)
        cache.check()
        kg, vg = ref.gather(0, table, B)
        tol_check(to_f64(out), oatt.decode_attention(q, kg, vg, lens, scale), "bf16", f"shared prefix {lens}")
        if lens[0] == lens[1] == 48:  # only the shared rows: the same output for both
            assert torch.equal(out[0].view(torch.int16), out[1].view(torch.int16))
    cache.free()


def test_out_of_pool_entries():
    dev = device()
    rng = np.random.default_rng(6)
    B, H, Hkv, D, S, bs = 3, 4, 2, 64, 64, 16
    nb = 10
    table = np.array([[0, 1, 2, 3], [4, -1, 5, 6], [7, 8, 9, 10]], dtype=np.int32)
    cache, ref = make(dev, B, H, Hkv, D, S, bs, nb)
    tab = kvc.to_device(table, dev)
    k = synthetic.draw(rng, (B, Hkv, 12, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, 12, D), "bf16")
    # b = 0 fits; b = 1 reaches entry -1 (rows 16..27); b = 2 rows 40..51 reach block 10 (outside)
    ci = np.array([10, 10, 40], dtype=np.int32)
    cache.paged_append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), tab, kvc.to_device(ci, dev))
    assert ref.append(0, k, v, ci, table) == [1, 2]
    assert cache.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    assert cache.check_status() == kvc.KVC_OK  # the flag was cleared
    ci = np.array([0, 0, 0], dtype=np.int32)
    cache.paged_append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), tab, kvc.to_device(ci, dev))
    assert ref.append(0, k, v, ci, table) == []
    cache.check()
    assert pools_equal(cache, ref)
    # decode over rows whose entries lie outside the pool: zeros there, and the flag
    q = synthetic.draw(rng, (B, H, D), "bf16")
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    lens = [12, 30, 64]
    cache.paged_decode_attn(0, kvc.to_device(q, dev), out, tab,
                            valid_lens=kvc.to_device(np.array(lens, dtype=np.int32), dev), sm_scale=0.125)
    assert cache.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    kg, vg = ref.gather(0, table, B)
    tol_check(to_f64(out), oatt.decode_attention(q, kg, vg, lens, 0.125), "bf16", "out-of-pool rows")
    # lengths outside [0, S]: zero outputs and the flag
    bad = np.array([12, S + 1, -3], dtype=np.int32)
    cache.paged_decode_attn(0, kvc.to_device(q, dev), out, tab, valid_lens=kvc.to_device(bad, dev),
                            sm_scale=0.125)
    assert cache.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    assert torch.count_nonzero(out[1:].float()) == 0
    cache.free()


def test_paged_and_static_calls_do_not_mix():
    dev = device()
    B, H, Hkv, D, S = 1, 4, 2, 64, 32
    paged = kvc.PagedCache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"), 16, 4)
    static = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"))
    q = torch.zeros((B, H, D), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((B, Hkv, 1, D), dtype=torch.bfloat16, device=dev)
    ci = torch.zeros((B,), dtype=torch.int32, device=dev)
    tab = torch.zeros((B, 2), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    for call in (lambda: paged.append(0, kv, kv, ci), lambda: paged.decode_attn(0, q, out, cache_index=ci,
                                                                                 sm_scale=0.1),
                 lambda: paged.append_decode_attn(0, kv, kv, q, out, ci, 0.1),
                 lambda: kvc._call("kvc_paged_append", static.handle, 0, kv.data_ptr(), kv.data_ptr(),
                                   tab.data_ptr(), ci.data_ptr(), 1, None)):
        with pytest.raises(kvc.KvcError) as e:
            call()
        assert e.value.status == kvc.KVC_ERR_INVALID_ARG
    paged.free()
    static.free()


def test_paged_llama3_full_size():
    """Llama-3-8B-shaped decode (B=16, H=32, H_kv=8, d_h=128, S=4096) through block tables of
    16-row blocks scattered over the pool, lengths ~U[1024, 4096]: every output against the
    oracle, and all of them bit-equal to the static decode."""
    dev = device()
    rng = np.random.default_rng(4096)
    B, H, Hkv, D, S, bs = 16, 32, 8, 128, 4096, 16
    W = S // bs
    nb = B * W
    lens = synthetic.gqa_valid_lens(dict(batch=B, max_context=S, valid_lo=1024, valid_hi=S), rng)
    say(f"paged llama: lens={lens.tolist()}")
    cache = kvc.PagedCache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"), bs, nb)
    table = random_tables(rng, B, W, nb)
    k = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
    zero = kvc.to_device(np.zeros(B, dtype=np.int32), dev)
    cache.paged_append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), kvc.to_device(table, dev), zero)
    q = synthetic.draw(rng, (B, H, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    valid = kvc.to_device(lens.astype(np.int32), dev)
    cache.paged_decode_attn(0, kvc.to_device(q, dev), out, kvc.to_device(table, dev), valid_lens=valid,
                            sm_scale=scale)
    cache.check()
    static = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"))
    static.prefill_fill(0, kvc.to_device(k, dev), kvc.to_device(v, dev), 0)
    ref_out = torch.empty_like(out)
    static.decode_attn(0, kvc.to_device(q, dev), ref_out, valid_lens=valid, sm_scale=scale)
    static.check()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    want = oatt.decode_attention(q, k, v, lens, scale)
    err = tol_check(to_f64(out), want, "bf16", "paged, every sequence")
    say(f"  max abs err {err:.3e}")
    cache.free()
    static.free()


@pytest.mark.parametrize("B,H,Hkv,D,S,bs,wg", [
    (4, 16, 4, 128, 1024, 16, 0),
    (3, 8, 2, 64, 512, 32, 64),
    (2, 32, 8, 128, 2048, 256, 0),
    (5, 4, 1, 256, 256, 16, 7),
])
def test_paged_fused_equals_append_then_decode(B, H, Hkv, D, S, bs, wg):
    """kvc_paged_append_decode_attn gives the output bits and pool bits of
    kvc_paged_append followed by kvc_paged_decode_attn (same tables, same
    grid), and the oracle's decode step within the bf16 bound. The new rows
    fall at row 0, at block starts and ends, and mid-block."""
    dev = device()
    rng = np.random.default_rng(31 + D + bs + wg)
    W = S // bs
    nb = B * W + 5
    say(f"paged fused: B={B} H={H} Hkv={Hkv} D={D} S={S} bs={bs} workgroups={wg}")
    fused, ref = make(dev, B, H, Hkv, D, S, bs, nb)
    two, _ = make(dev, B, H, Hkv, D, S, bs, nb)
    table = random_tables(rng, B, W, nb)
    tab = kvc.to_device(table, dev)
    lens = [S, S // 2, 1, bs, bs + 1][:B]
    k, v = fill_both(dev, fused, ref, rng, table, lens)
    two.paged_append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), tab,
                     kvc.to_device(np.zeros(B, dtype=np.int32), dev))
    if wg:
        fused.set_workgroups(wg)
        two.set_workgroups(wg)
    ci = np.array([S - 1, S // 2, 0, bs - 1, bs][:B], dtype=np.int32)
    kn = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
    vn = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
    q = synthetic.draw(rng, (B, H, D), "bf16")
    knd, vnd, qd, cid = (kvc.to_device(x, dev) for x in (kn, vn, q, ci))
    a = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    for rep in range(2):  # the second call reuses the cached split
        fused.paged_append_decode_attn(0, knd, vnd, qd, a, tab, cid, 0.088)
        fused.check()
    two.paged_append(0, knd, vnd, tab, cid)
    two.paged_decode_attn(0, qd, b, tab, cache_index=cid, sm_scale=0.088)
    two.check()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "fused output bits differ from the two calls"
    assert ref.append(0, kn, vn, ci, table) == []
    assert pools_equal(fused, ref), "fused pool differs from the oracle"
    assert pools_equal(two, ref)
    kg, vg = ref.gather(0, table, B)
    tol_check(to_f64(a), oatt.decode_attention(q, kg, vg, list(ci + 1), 0.088), "bf16", "paged fused")
    fused.free()
    two.free()


def test_paged_fused_skips_like_the_two_calls():
    """A new row whose block entry lies outside the pool, and a cache_index
    outside the capacity: the fused call writes nothing for them, raises the
    flag, and gives the two calls' output bits (zeros for the second)."""
    dev = device()
    rng = np.random.default_rng(41)
    B, H, Hkv, D, S, bs = 3, 8, 2, 128, 64, 16
    nb = 12
    table = np.array([[0, 1, 2, 3], [4, 5, -1, 6], [7, 8, 9, 10]], dtype=np.int32)
    tab = kvc.to_device(table, dev)
    fused, ref = make(dev, B, H, Hkv, D, S, bs, nb)
    two, _ = make(dev, B, H, Hkv, D, S, bs, nb)
    k = synthetic.draw(rng, (B, Hkv, 30, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, 30, D), "bf16")
    zero = kvc.to_device(np.zeros(B, dtype=np.int32), dev)
    for c in (fused, two):  # rows 0..29; sequence 1 stops short of its bad block (rows 32..47)
        c.paged_append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), tab, zero)
        c.check()
    ci = np.array([20, 35, S + 3], dtype=np.int32)  # b = 1: new row in the bad block; b = 2: out of range
    kn = kvc.to_device(synthetic.draw(rng, (B, Hkv, 1, D), "bf16"), dev)
    vn = kvc.to_device(synthetic.draw(rng, (B, Hkv, 1, D), "bf16"), dev)
    q = kvc.to_device(synthetic.draw(rng, (B, H, D), "bf16"), dev)
    cid = kvc.to_device(ci, dev)
    a = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    fused.paged_append_decode_attn(0, kn, vn, q, a, tab, cid, 0.1)
    assert fused.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    two.paged_append(0, kn, vn, tab, cid)
    two.paged_decode_attn(0, q, b, tab, cache_index=cid, sm_scale=0.1)
    assert two.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.count_nonzero(a[2].float()) == 0
    fk, fv = fused.layer_tensors(0)
    tk, tv = two.layer_tensors(0)
    assert torch.equal(fk.view(torch.int16), tk.view(torch.int16))
    assert torch.equal(fv.view(torch.int16), tv.view(torch.int16))
    del fk, fv, tk, tv
    fused.free()
    two.free()
