"""A decode step (append + attention on every layer) captured in a HIP graph
and replayed gives bit-identical outputs to eager launches on every replay,
with eager work and synchronisations between the replays."""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, oracle_decode, say, to_f64, tol_check
from oracle.buffer import RefCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    dev = device()
    L, B, H, Hkv, D, S = 3, 4, 16, 4, 128, 700
    say(f"graph replay: L={L} B={B} H={H} Hkv={Hkv} D={D} S={S}")
    rng = np.random.default_rng(61)
    valid = np.array([700, 1, 350, 129], dtype=np.int32)
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"))
    ref = RefCache(L, B, Hkv, S, D, "bf16")
    q, kn, vn, out = [], [], [], []
    for layer in range(L):
        k = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
        v = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
        cache.prefill_fill(layer, kvc.to_device(k, dev), kvc.to_device(v, dev), 0)
        ref.fill(layer, k, v, 0)
        q.append(synthetic.draw(rng, (B, H, D), "bf16"))
        kn.append(synthetic.draw(rng, (B, Hkv, 1, D), "bf16"))
        vn.append(synthetic.draw(rng, (B, Hkv, 1, D), "bf16"))
        ref.append(layer, kn[-1], vn[-1], valid - 1)
    qd = [kvc.to_device(x, dev) for x in q]
    knd = [kvc.to_device(x, dev) for x in kn]
    vnd = [kvc.to_device(x, dev) for x in vn]
    outd = [torch.empty((B, H, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    vl = kvc.to_device(valid, dev)
    ci = kvc.to_device(valid - 1, dev)

    def step():
        for layer in range(L):
            cache.append(layer, knd[layer], vnd[layer], ci)
            cache.decode_attn(layer, qd[layer], outd[layer], valid_lens=vl, cache_index=ci, sm_scale=0.088)

    step()
    torch.cuda.synchronize()
    eager = [bits_of(o, "bf16").copy() for o in outd]
    for layer in range(L):
        tol_check(to_f64(outd[layer]), oracle_decode(ref, layer, q[layer], valid, 0.088), "bf16", f"layer {layer}")

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outd:
            o.fill_(0.0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer in range(L):
            assert np.array_equal(bits_of(outd[layer], "bf16"), eager[layer]), f"replay {rep} layer {layer}"
    cache.check()
    cache.free()


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_graph_fused_step_with_index_advanced_on_device(dtype):
    """A decode loop as a caller would capture it: every layer's fused
    append + attention (kvc_append_decode_attn) in one graph, with
    cache_index advanced on the device between replays (so each replay's
    first launch meets new lengths and works the split out again, and the
    later layers reuse it). Every replay matches the oracle's decode step
    at that position, and the cache rows match the oracle's appends."""
    from oracle.quant import RefQuantCache
    dev = device()
    L, B, H, Hkv, D, S = 3, 3, 8, 2, 128, 300
    say(f"graph, fused step, advancing index: {dtype} L={L} B={B} H={H} Hkv={Hkv} D={D} S={S}")
    rng = np.random.default_rng(62)
    start = np.array([100, 1, 250], dtype=np.int32)  # rows already in the cache
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, dtype))
    ref = RefCache(L, B, Hkv, S, D, "bf16") if dtype == "bf16" else RefQuantCache(L, B, Hkv, S, D)
    q, kn, vn = [], [], []
    for layer in range(L):
        k = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
        v = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
        cache.prefill_fill(layer, kvc.to_device(k, dev), kvc.to_device(v, dev), 0)
        ref.fill(layer, k, v, 0)
        q.append(synthetic.draw(rng, (B, H, D), "bf16"))
        kn.append(synthetic.draw(rng, (B, Hkv, 1, D), "bf16"))
        vn.append(synthetic.draw(rng, (B, Hkv, 1, D), "bf16"))
    qd = [kvc.to_device(x, dev) for x in q]
    knd = [kvc.to_device(x, dev) for x in kn]
    vnd = [kvc.to_device(x, dev) for x in vn]
    outd = [torch.empty((B, H, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ci = kvc.to_device(start, dev)  # the step appends at ci and attends ci + 1 rows

    def step():
        for layer in range(L):
            cache.append_decode_attn(layer, knd[layer], vnd[layer], qd[layer], outd[layer], ci, 0.088)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(5):
        pos = start + rep
        for layer in range(L):
            ref.append(layer, kn[layer], vn[layer], pos)
        for o in outd:
            o.fill_(0.0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer in range(L):
            want = oracle_decode(ref, layer, q[layer], pos + 1, 0.088)
            tol_check(to_f64(outd[layer]), want, "bf16", f"{dtype} replay {rep} layer {layer}")
        ci.add_(1)                # the loop's index advance, on the device
        torch.cuda.synchronize()
    cache.check()
    if dtype == "bf16":
        for layer in range(L):
            k_dev, v_dev = cache.layer_tensors(layer)
            assert np.array_equal(bits_of(k_dev, "bf16"), ref.keys(layer))
            assert np.array_equal(bits_of(v_dev, "bf16"), ref.values(layer))
            del k_dev, v_dev
    else:
        for layer in range(L):
            k_dev, v_dev = cache.layer_tensors(layer)
            assert np.array_equal(k_dev.cpu().numpy(), ref.codes[layer, 0])
            assert np.array_equal(v_dev.cpu().numpy(), ref.codes[layer, 1])
            del k_dev, v_dev
    cache.free()
