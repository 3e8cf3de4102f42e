"""The decode kernel's cached split of the work (valid for repeated calls with the same lengths, grid
and append mode) never changes a result: repeated calls give the same bits, and changing the
lengths, the grid or the mode between calls gives the oracle's result for the new inputs."""

import numpy as np
import pytest
import torch

from gpu_util import device, say, to_f64, tol_check
from oracle import attention as oatt
from oracle.buffer import RefCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def setup(dev, B, H, Hkv, D, S, seed):
    rng = np.random.default_rng(seed)
    k = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"))
    cache.prefill_fill(0, kvc.to_device(k, dev), kvc.to_device(v, dev), 0)
    ref = RefCache(1, B, Hkv, S, D, "bf16")
    ref.fill(0, k, v, 0)
    q = synthetic.draw(rng, (B, H, D), "bf16")
    return cache, ref, q, rng


def test_repeated_and_changed_lengths():
    dev = device()
    B, H, Hkv, D, S = 4, 16, 4, 128, 1024
    cache, ref, q, _ = setup(dev, B, H, Hkv, D, S, 21)
    qd = kvc.to_device(q, dev)
    scale = 1.0 / np.sqrt(D)
    L1, L2, L3 = (1000, 37, 512, 900), (1000, 38, 512, 900), (0, 100, 200, 300)
    seen = {}
    for wg in (0, 64):
        cache.set_workgroups(wg)
        for lens in (L1, L1, L2, L1, L3, L1, L1, L2, L2):
            say(f"plan: workgroups {wg} lengths {lens}")
            out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
            cache.decode_attn(0, qd, out, valid_lens=kvc.to_device(np.array(lens, dtype=np.int32), dev),
                              sm_scale=scale)
            cache.check()
            key = (wg, lens)
            if key in seen:
                assert torch.equal(out.view(torch.int16), seen[key].view(torch.int16)), key
            else:
                tol_check(to_f64(out), oatt.decode_attention(q, ref.keys(0), ref.values(0), list(lens), scale),
                          "bf16", str(key))
                seen[key] = out
    cache.free()


def test_fused_and_plain_calls_interleaved():
    """The fused call (which also appends) and the plain decode keep separate splits: interleaving
    them on one cache gives the same bits as running each alone."""
    dev = device()
    B, H, Hkv, D, S = 3, 8, 2, 128, 700
    cache, ref, q, rng = setup(dev, B, H, Hkv, D, S, 22)
    qd = kvc.to_device(q, dev)
    lens = np.array([700, 333, 64], dtype=np.int32)
    ci = kvc.to_device(lens - 1, dev)
    kn = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
    vn = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
    ref.append(0, kn, vn, lens - 1)
    want = oatt.decode_attention(q, ref.keys(0), ref.values(0), lens.tolist(), 0.1)
    outs = []
    for i in range(6):
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        if i % 2 == 0:  # the same new rows each time, so the cache ends the same
            cache.append_decode_attn(0, kvc.to_device(kn, dev), kvc.to_device(vn, dev), qd, out, ci, 0.1)
        else:
            cache.decode_attn(0, qd, out, valid_lens=kvc.to_device(lens, dev), sm_scale=0.1)
        cache.check()
        tol_check(to_f64(out), want, "bf16", f"call {i}")
        outs.append(out)
    for i in range(6):
        assert torch.equal(outs[i].view(torch.int16), outs[0].view(torch.int16)), i
    cache.free()


@pytest.mark.parametrize("workgroups", [16, 64])
def test_overflowing_plan_entries(workgroups):
    """Many short sequences on a small grid: a workgroup's range then holds more pieces than its
    cached entry keeps (8), so those workgroups work their pieces out again on every call while
    the others take theirs from the cache (with one long sequence, some workgroups hold a single
    piece of it and keep their entries). Repeated calls give identical bits, and every call
    matches the oracle, also after the lengths change."""
    dev = device()
    B, H, Hkv, D, S = 256, 8, 2, 64, 512
    cache, ref, q, rng = setup(dev, B, H, Hkv, D, S, 23)
    qd = kvc.to_device(q, dev)
    cache.set_workgroups(workgroups)
    short = rng.integers(1, 41, size=B).astype(np.int32)
    short[7] = S  # one long sequence among them
    changed = short.copy()
    changed[::3] += 1
    seen = {}
    for lens in (short, short, changed, short, changed, changed):
        key = lens.tobytes()
        say(f"overflowing entries: workgroups {workgroups}, sum of lengths {int(lens.sum())}")
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        cache.decode_attn(0, qd, out, valid_lens=kvc.to_device(lens, dev), sm_scale=0.125)
        cache.check()
        if key in seen:
            assert torch.equal(out.view(torch.int16), seen[key].view(torch.int16))
        else:
            tol_check(to_f64(out), oatt.decode_attention(q, ref.keys(0), ref.values(0), lens, 0.125), "bf16",
                      f"workgroups {workgroups}")
            seen[key] = out
    cache.free()


@pytest.mark.parametrize("D,lens", [
    (32, (512, 1, 300, 0, 512, 17, 200, 511)),    # every segment short: each goes whole to one workgroup
    (32, (513, 1, 300, 0, 512, 17, 200, 511)),    # one segment one row longer: the split over the grid
    (128, (256, 255, 3, 0, 128, 256, 1, 100)),    # 128 KB rows limit at d_h = 128: whole
    (128, (257, 255, 3, 0, 128, 256, 1, 100)),    # one row over it: split
])
def test_short_segments_whole_and_split(D, lens):
    """On the default grid, segments of at most 512 rows and 128 KB of rows are each taken whole by
    one workgroup; one row more switches to the split over the grid. Both sides of the boundary, in
    turn on one cache (the cached split follows the lengths), with ragged and empty sequences, match
    the oracle, and a forced grid (always split) matches it too."""
    dev = device()
    B, H, Hkv, S = 8, 8, 4, 520
    cache, ref, q, _ = setup(dev, B, H, Hkv, D, S, 23)
    qd = kvc.to_device(q, dev)
    scale = 1.0 / np.sqrt(D)
    want = oatt.decode_attention(q, ref.keys(0), ref.values(0), list(lens), scale)
    other = tuple(min(n + 1, S) if n else 0 for n in lens)
    want_other = oatt.decode_attention(q, ref.keys(0), ref.values(0), list(other), scale)
    for wg, seq in ((0, (lens, other, lens)), (48, (lens,))):
        cache.set_workgroups(wg)
        for cur in seq:
            say(f"short segments: d_h {D} workgroups {wg} lengths {cur}")
            out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
            cache.decode_attn(0, qd, out, valid_lens=kvc.to_device(np.array(cur, dtype=np.int32), dev),
                              sm_scale=scale)
            cache.check()
            tol_check(to_f64(out), want if cur == lens else want_other, "bf16", f"wg {wg} lens {cur}")
    cache.free()
