"""The benchmarked decode step, checked in full against the oracle.

The step the benchmark times is 32 launches of kvc_append_decode_attn (one
per layer: append the new row at cache_index, then attend rows
[0, cache_index + 1)) of the Llama-3-8B-shaped stack (B=16, H=32, H_kv=8,
d_h=128, max_context 4096, the seeded U[1024, 4096] lengths), captured in
one HIP graph and launched on the default persistent grid. Here the same
graph is replayed twice with cache_index advanced on the device in between
and fresh queries and new rows copied into the captured buffers, as a decode
loop would. So replay 0's first layer works the split of the work out and its
other 31 layers take the cached split (and start their first piece before the
lengths are confirmed); replay 1 meets changed lengths and does the same
again. Layers 0, 15 and 31 hold their own cache rows, the others a copy of
layer 0's. Every output of every layer in both replays is compared with the
oracle ("10.3 - KV cache implementation details", section 5 step 2: append,
then attend the whole cache; "KV Cache Optimization ...", "#2 In-place KV
cache updates", "After": reads stop at the valid length), and the cache rows
with the oracle's appends, bit for bit.
"""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, oracle_decode, say, to_f64, tol_check
from oracle.buffer import RefCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu

DISTINCT = (0, 15, 31)
REPLAYS = 2


def test_benchmarked_step_graph_full_size():
    dev = device()
    cfg = synthetic.WORKLOADS["llama3_8b_gqa_bf16"]
    L, B, H, Hkv, D, S = (cfg["n_layers"], cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"],
                          cfg["head_dim"], cfg["max_context"])
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"))
    assert cache.workgroups()[0] == 0, "the default grid"
    fills, refs = {}, {}
    for layer in DISTINCT:
        c = synthetic.gqa_layer(cfg, seed_offset=layer)
        fills[layer] = c
        cache.prefill_fill(layer, kvc.to_device(c["k_fill"], dev), kvc.to_device(c["v_fill"], dev), 0)
        refs[layer] = RefCache(1, B, Hkv, S, D, "bf16")
        refs[layer].fill(0, c["k_fill"], c["v_fill"], 0)
    k0, v0 = cache.layer_tensors(0)
    for layer in range(L):
        if layer not in DISTINCT:
            kp, vp = cache.layer_ptrs(layer)
            kvc._memcpy_d2d(kp, k0.data_ptr(), k0.numel() * 2, dev)
            kvc._memcpy_d2d(vp, v0.data_ptr(), v0.numel() * 2, dev)
    del k0, v0
    group = {layer: (layer if layer in DISTINCT else 0) for layer in range(L)}
    lens = fills[0]["valid_lens"]           # the benchmark's lengths (sum 40,563)
    assert lens.max() + REPLAYS - 1 <= S
    sm_scale = fills[0]["sm_scale"]
    say(f"benchmarked step: L={L} B={B} H={H} H_kv={Hkv} D={D} S={S} lengths {lens.tolist()}")

    rng = np.random.default_rng(cfg["seed"] + 11)
    draws = [[dict(q=synthetic.draw(rng, (B, H, D), "bf16"),
                   kn=synthetic.draw(rng, (B, Hkv, 1, D), "bf16"),
                   vn=synthetic.draw(rng, (B, Hkv, 1, D), "bf16")) for _ in range(L)] for _ in range(REPLAYS)]
    qd = [torch.empty((B, H, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    knd = [torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    vnd = [torch.empty((B, Hkv, 1, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    outd = [torch.empty((B, H, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ci = kvc.to_device((lens - 1).astype(np.int32), dev)
    torch.cuda.synchronize()

    def step():
        for layer in range(L):
            cache.append_decode_attn(layer, knd[layer], vnd[layer], qd[layer], outd[layer], ci, sm_scale)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()

    worst = 0.0
    for rep in range(REPLAYS):
        for layer in range(L):
            d = draws[rep][layer]
            qd[layer].copy_(kvc.to_device(d["q"], dev))
            knd[layer].copy_(kvc.to_device(d["kn"], dev))
            vnd[layer].copy_(kvc.to_device(d["vn"], dev))
            outd[layer].fill_(0.0)
        torch.cuda.synchronize()
        say(f"  replay {rep}: cache_index = lengths - 1 + {rep}")
        g.replay()
        torch.cuda.synchronize()
        cache.check()
        for layer in range(L):
            ref = refs[group[layer]]
            for r in range(rep + 1):  # this layer's rows appended so far
                ref.append(0, draws[r][layer]["kn"], draws[r][layer]["vn"], lens - 1 + r)
            want = oracle_decode(ref, 0, draws[rep][layer]["q"], lens + rep, sm_scale)
            worst = max(worst, tol_check(to_f64(outd[layer]), want, "bf16", f"replay {rep} layer {layer}"))
        ci.add_(1)  # the loop's index advance, on the device
        torch.cuda.synchronize()
    say(f"  every output of {L} layers x {REPLAYS} replays within bounds; max abs err {worst:.3e}")

    # cache rows: the distinct layers bit for bit in full; every layer's
    # appended rows at lengths - 1 and lengths
    for layer in range(L):
        ref = refs[group[layer]]
        for r in range(REPLAYS):
            ref.append(0, draws[r][layer]["kn"], draws[r][layer]["vn"], lens - 1 + r)
        k_dev, v_dev = cache.layer_tensors(layer)
        if layer in DISTINCT:
            assert np.array_equal(bits_of(k_dev, "bf16"), ref.keys(0)), f"layer {layer} keys"
            assert np.array_equal(bits_of(v_dev, "bf16"), ref.values(0)), f"layer {layer} values"
        else:
            kb, vb = bits_of(k_dev, "bf16"), bits_of(v_dev, "bf16")
            for b in range(B):
                rows = slice(int(lens[b]) - 1, int(lens[b]) - 1 + REPLAYS)
                assert np.array_equal(kb[b, :, rows], ref.keys(0)[b, :, rows]), f"layer {layer} seq {b}"
                assert np.array_equal(vb[b, :, rows], ref.values(0)[b, :, rows]), f"layer {layer} seq {b}"
        del k_dev, v_dev
    cache.free()
