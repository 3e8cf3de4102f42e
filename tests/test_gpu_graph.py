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
