"""Decode attention on the GPU against the CPU float64 oracle.

Small cases are compared element by element over every output; the
workload shapes (DantinoX, Llama-3-8B-shaped, long context) run at their
full sizes in the launch configuration the benchmark uses and are compared
on every (b, h) of the layers that are checked.
"""

import math

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, oracle_decode, ref_cache_like, say, to_f64, tol_check
from oracle.buffer import RefCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def run_case(dev, case, L=1, layer=0, workgroups=None, S=None, dtype="bf16", fill_rows=None):
    B, Hkv = case["k_fill"].shape[:2]
    D = case["q"].shape[2]
    H = case["q"].shape[1]
    S = S or case["k_fill"].shape[2]
    desc = kvc.gqa_desc(L, B, H, Hkv, D, S, dtype)
    cache = kvc.Cache(desc)
    if workgroups is not None:
        cache.set_workgroups(workgroups)
    ref = RefCache(L, B, Hkv, S, D, dtype)
    T = case["k_fill"].shape[2]
    cache.prefill_fill(layer, kvc.to_device(case["k_fill"], dev), kvc.to_device(case["v_fill"], dev), 0)
    ref.fill(layer, case["k_fill"], case["v_fill"], 0)
    ci = case["cache_index"]
    cache.append(layer, kvc.to_device(case["k_new"], dev), kvc.to_device(case["v_new"], dev),
                 kvc.to_device(ci, dev))
    ref.append(layer, case["k_new"], case["v_new"], ci)
    out = torch.empty((B, H, D), dtype=kvc.torch_dtype(dtype), device=dev)
    cache.decode_attn(layer, kvc.to_device(case["q"], dev), out,
                      valid_lens=kvc.to_device(case["valid_lens"], dev),
                      cache_index=kvc.to_device(ci, dev), sm_scale=case["sm_scale"])
    cache.check()
    want = oracle_decode(ref, layer, case["q"], case["valid_lens"], case["sm_scale"])
    return cache, ref, out, want


def test_tiny_mha_f32_prefill_then_16_steps():
    """Tiny MHA fp32: prefill 64 tokens, then 16 decode steps appending at
    64 + i and attending 65 + i rows (q pre-scaled, sm_scale = 1). The
    buffer is compared bit for bit and the output within the fp32 bound."""
    dev = device()
    cfg = synthetic.WORKLOADS["tiny_mha_f32"]
    say(f"tiny_mha_f32: {cfg}")
    d = synthetic.tiny_sequence(cfg)
    B, H, Hkv, D, S, P = (cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                          cfg["max_context"], cfg["prefill"])
    region = torch.zeros(kvc.cache_bytes(kvc.gqa_desc(1, B, H, Hkv, D, S, "f32")), dtype=torch.uint8, device=dev)
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "f32"), external=region)
    ref = RefCache(1, B, Hkv, S, D, "f32")
    cache.prefill_fill(0, kvc.to_device(d["k"][:, :, :P], dev), kvc.to_device(d["v"][:, :, :P], dev), 0)
    ref.fill(0, d["k"][:, :, :P], d["v"][:, :, :P], 0)
    ci_dev = torch.tensor([P], dtype=torch.int32, device=dev)
    worst = 0.0
    for i in range(cfg["steps"]):
        kn = d["k"][:, :, P + i:P + i + 1]
        vn = d["v"][:, :, P + i:P + i + 1]
        cache.append(0, kvc.to_device(kn, dev), kvc.to_device(vn, dev), ci_dev)
        ref.append(0, kn, vn, [P + i])
        out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        # valid_lens omitted: n = cache_index + 1 (the appended token is attended)
        cache.decode_attn(0, kvc.to_device(d["q"][i], dev), out, cache_index=ci_dev, sm_scale=1.0)
        want = oracle_decode(ref, 0, d["q"][i], [P + i + 1], 1.0)
        worst = max(worst, tol_check(to_f64(out), want, "f32", f"step {i}"))
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(region.view(torch.float32), "f32"), ref.buf.reshape(-1).view(np.uint32))
        ci_dev += 1   # advanced on the device, as a captured decode loop would
    cache.check()
    say(f"  worst abs err {worst:.3e}")
    cache.free()


@pytest.mark.parametrize("name", ["dantinox_mha_bf16", "dantinox_gqa_bf16"])
def test_dantinox_all_layers(name):
    """12 layers, B=8, H=8, d_h=32, S=512: fill 511 rows, append at 511,
    attend 512 rows, every layer with its own data."""
    dev = device()
    cfg = synthetic.WORKLOADS[name]
    say(f"{name}: {cfg}")
    L, B, H, Hkv, D, S = (cfg["n_layers"], cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"],
                          cfg["head_dim"], cfg["max_context"])
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"))
    ref = RefCache(L, B, Hkv, S, D, "bf16")
    worst = 0.0
    for layer in range(L):
        c = synthetic.gqa_layer(cfg, seed_offset=layer, fill_rows=S - 1)
        cache.prefill_fill(layer, kvc.to_device(c["k_fill"], dev), kvc.to_device(c["v_fill"], dev), 0)
        ref.fill(layer, c["k_fill"], c["v_fill"], 0)
        ci = kvc.to_device(c["cache_index"], dev)
        cache.append(layer, kvc.to_device(c["k_new"], dev), kvc.to_device(c["v_new"], dev), ci)
        ref.append(layer, c["k_new"], c["v_new"], c["cache_index"])
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        cache.decode_attn(layer, kvc.to_device(c["q"], dev), out,
                          valid_lens=kvc.to_device(c["valid_lens"], dev), cache_index=ci,
                          sm_scale=c["sm_scale"])
        want = oracle_decode(ref, layer, c["q"], c["valid_lens"], c["sm_scale"])
        worst = max(worst, tol_check(to_f64(out), want, "bf16", f"layer {layer}"))
    cache.check()
    say(f"  worst abs err {worst:.3e}")
    cache.free()


def test_llama3_8b_shape_full_size():
    """Llama-3-8B-shaped GQA at full size (32 layers, B=16, H=32, H_kv=8,
    d_h=128, S=4096, valid_len ~ U[1024, 4096]); layers 0 and 31 hold their
    own data and every (b, h) output is compared."""
    dev = device()
    cfg = synthetic.WORKLOADS["llama3_8b_gqa_bf16"]
    say(f"llama3_8b_gqa_bf16: {cfg}")
    L, B, H, Hkv, D, S = (cfg["n_layers"], cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"],
                          cfg["head_dim"], cfg["max_context"])
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"))
    for layer in (0, L - 1):
        c = synthetic.gqa_layer(cfg, seed_offset=layer)
        say(f"  layer {layer}: valid_lens {c['valid_lens'].tolist()}")
        ref = RefCache(1, B, Hkv, S, D, "bf16")
        cache.prefill_fill(layer, kvc.to_device(c["k_fill"], dev), kvc.to_device(c["v_fill"], dev), 0)
        ref.fill(0, c["k_fill"], c["v_fill"], 0)
        ci = kvc.to_device(c["cache_index"], dev)
        cache.append(layer, kvc.to_device(c["k_new"], dev), kvc.to_device(c["v_new"], dev), ci)
        ref.append(0, c["k_new"], c["v_new"], c["cache_index"])
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        cache.decode_attn(layer, kvc.to_device(c["q"], dev), out,
                          valid_lens=kvc.to_device(c["valid_lens"], dev), cache_index=ci,
                          sm_scale=c["sm_scale"])
        cache.check()
        want = oracle_decode(ref, 0, c["q"], c["valid_lens"], c["sm_scale"])
        err = tol_check(to_f64(out), want, "bf16", f"layer {layer}")
        say(f"  layer {layer}: max abs err {err:.3e}")
        k_dev, v_dev = cache.layer_tensors(layer)
        assert np.array_equal(bits_of(k_dev, "bf16"), ref.keys(0))
        assert np.array_equal(bits_of(v_dev, "bf16"), ref.values(0))
        del k_dev, v_dev
    cache.free()


def test_long_context_full_size():
    """Long-context GQA: cache sized for 80 layers (10,737,418,240 bytes),
    H=64, H_kv=8, d_h=128, B=1, S=32768, valid 32768; layer 79 checked."""
    dev = device()
    cfg = synthetic.WORKLOADS["longctx_gqa_bf16"]
    say(f"longctx_gqa_bf16: {cfg}")
    L, B, H, Hkv, D, S = (cfg["n_layers"], cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"],
                          cfg["head_dim"], cfg["max_context"])
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"))
    assert cache.nbytes == 10737418240
    layer = L - 1
    c = synthetic.gqa_layer(cfg, seed_offset=layer, fill_rows=S - 1)
    ref = RefCache(1, B, Hkv, S, D, "bf16")
    cache.prefill_fill(layer, kvc.to_device(c["k_fill"], dev), kvc.to_device(c["v_fill"], dev), 0)
    ref.fill(0, c["k_fill"], c["v_fill"], 0)
    ci = kvc.to_device(c["cache_index"], dev)
    cache.append(layer, kvc.to_device(c["k_new"], dev), kvc.to_device(c["v_new"], dev), ci)
    ref.append(0, c["k_new"], c["v_new"], c["cache_index"])
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    cache.decode_attn(layer, kvc.to_device(c["q"], dev), out, valid_lens=kvc.to_device(c["valid_lens"], dev),
                      cache_index=ci, sm_scale=c["sm_scale"])
    cache.check()
    want = oracle_decode(ref, 0, c["q"], c["valid_lens"], c["sm_scale"])
    err = tol_check(to_f64(out), want, "bf16", "long context")
    say(f"  max abs err {err:.3e}")
    cache.free()


SMALL = [
    # dtype, B, H, Hkv, D, S
    ("f32", 3, 4, 4, 32, 97),
    ("f32", 2, 8, 2, 64, 130),
    ("f32", 2, 4, 1, 128, 77),
    ("f32", 1, 8, 8, 256, 45),
    ("bf16", 3, 8, 8, 32, 300),
    ("bf16", 2, 12, 4, 64, 129),
    ("bf16", 4, 32, 8, 128, 520),
    ("bf16", 2, 16, 2, 128, 257),
    ("bf16", 2, 32, 1, 128, 100),    # MQA, 32 heads per kv head
    ("bf16", 2, 6, 2, 256, 66),      # 3 heads per group
    ("bf16", 2, 64, 8, 128, 1000),
]


@pytest.mark.parametrize("dtype,B,H,Hkv,D,S", SMALL)
def test_small_shapes_ragged(dtype, B, H, Hkv, D, S):
    """Ragged valid lengths including 0, 1, tile edges and S on small shapes."""
    dev = device()
    rng = np.random.default_rng(S * 7 + D)
    special = [0, 1, 2, 15, 16, 17, 63, 64, 65, S - 1, S]
    valid = np.array([special[i % len(special)] if i % 2 == 0 else rng.integers(1, S + 1)
                      for i in range(B)], dtype=np.int32)
    valid = np.clip(valid, 0, S)
    valid[-1] = S
    say(f"small ragged: {dtype} B={B} H={H} Hkv={Hkv} D={D} S={S} valid={valid.tolist()}")
    case = synthetic.random_gqa_case(int(S + D), B, H, Hkv, D, S, dtype, valid_lens=np.maximum(valid, 1))
    case["valid_lens"] = valid
    case["cache_index"] = np.maximum(valid - 1, 0).astype(np.int32)
    cache, ref, out, want = run_case(dev, case, dtype=dtype)
    tol_check(to_f64(out), want, dtype, "ragged")
    assert not to_f64(out)[valid == 0].any(), "empty sequence must give zeros"
    cache.free()


@pytest.mark.parametrize("workgroups", [1, 2, 3, 7, 64, 333, 1024, 2048])
def test_workgroup_count_invariance(workgroups):
    """Any persistent grid size gives the oracle's result within tolerance:
    one workgroup streams everything; large counts split every segment into
    many pieces (and, with fewer rows than workgroups, leave some empty)."""
    dev = device()
    B, H, Hkv, D, S = 3, 16, 4, 128, 1000
    case = synthetic.random_gqa_case(77, B, H, Hkv, D, S, "bf16", valid_lens=[1000, 333, 17])
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"))
    mx = cache.workgroups()[1]
    cache.free()
    wg = min(workgroups, mx)
    say(f"workgroup invariance: workgroups={wg}")
    cache, ref, out, want = run_case(dev, case, workgroups=wg)
    assert cache.workgroups()[0] == wg
    tol_check(to_f64(out), want, "bf16", f"workgroups {wg}")
    cache.free()


@pytest.mark.parametrize("workgroups", [5, 97, 2048])
def test_fewer_rows_than_workgroups(workgroups):
    """Tiny total row counts with many workgroups: empty workgroup ranges and
    pieces of one or two rows."""
    dev = device()
    B, H, Hkv, D, S = 4, 8, 2, 64, 40
    case = synthetic.random_gqa_case(78, B, H, Hkv, D, S, "f32", valid_lens=[1, 0, 3, 2])
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "f32"))
    wg = min(workgroups, cache.workgroups()[1])
    cache.free()
    say(f"fewer rows than workgroups: workgroups={wg}")
    case["cache_index"] = np.maximum(case["valid_lens"] - 1, 0).astype(np.int32)
    cache, ref, out, want = run_case(dev, case, workgroups=wg, dtype="f32")
    tol_check(to_f64(out), want, "f32", f"workgroups {wg}")
    cache.free()


@pytest.mark.parametrize("dtype,H,Hkv,D,S,workgroups", [
    ("bf16", 8, 1, 128, 8192, 64),     # 8 pieces or so: the batch merge
    ("bf16", 8, 1, 128, 8192, 256),    # ~32 pieces: two rounds of the wide merge
    ("bf16", 16, 2, 64, 6000, 1024),   # ~500 pieces per segment
    ("f32", 8, 2, 256, 4000, 512),     # the fp32 piece, 256-wide heads
    ("bf16", 64, 8, 128, 12345, 300),  # eight heads per kv head, ragged rows
])
def test_one_long_sequence_wide_merge(dtype, H, Hkv, D, S, workgroups):
    """One sequence split over the grid: each segment's pieces (more than 8
    past 64 workgroups) are merged four dims per thread in rounds of loads."""
    dev = device()
    case = synthetic.random_gqa_case(81, 1, H, Hkv, D, S, dtype, valid_lens=[S])
    cache = kvc.Cache(kvc.gqa_desc(1, 1, H, Hkv, D, S, dtype))
    wg = min(workgroups, cache.workgroups()[1])
    cache.free()
    say(f"one long sequence: {dtype} H={H} H_kv={Hkv} D={D} S={S} workgroups={wg}")
    cache, ref, out, want = run_case(dev, case, workgroups=wg, dtype=dtype)
    tol_check(to_f64(out), want, dtype, "long sequence")
    cache.free()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_skewed_lengths_many_pieces(dtype):
    """One full-length sequence among many of one to three rows, with the
    largest grid: the long segment is cut into the most pieces the grid cap
    allows (about 65), all merged by the last one to arrive."""
    dev = device()
    B, H, Hkv, D, S = 64, 8, 1, 128, 4096
    valid = np.array([S] + [1 + i % 3 for i in range(B - 1)], dtype=np.int32)
    case = synthetic.random_gqa_case(79, B, H, Hkv, D, S, dtype, valid_lens=valid)
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, dtype))
    wg = cache.workgroups()[1]
    cache.free()
    say(f"skewed lengths: {dtype} workgroups={wg}")
    cache, ref, out, want = run_case(dev, case, workgroups=wg, dtype=dtype)
    tol_check(to_f64(out), want, dtype, "skewed")
    cache.free()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_row_is_exact(dtype):
    """n = 1: softmax of one logit is exactly 1, so out = V row 0 bit for bit."""
    dev = device()
    B, H, Hkv, D, S = 2, 8, 2, 128, 64
    case = synthetic.random_gqa_case(3, B, H, Hkv, D, S, dtype, valid_lens=[1, 1])
    for wg in (1, 64):
        cache, ref, out, want = run_case(dev, case, workgroups=wg, dtype=dtype)
        got = bits_of(out, dtype)
        G = H // Hkv
        for h in range(H):
            assert np.array_equal(got[:, h], ref.values(0)[:, h // G, 0]), f"head {h}"
        cache.free()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_garbage_beyond_valid_is_bit_identical(dtype):
    """Rows at or past n_b filled with zeros, NaN, +-inf or 1e30 give the same
    output bits (those rows are never read)."""
    dev = device()
    B, H, Hkv, D, S = 3, 8, 2, 128, 300
    valid = np.array([300, 129, 5], dtype=np.int32)
    base = synthetic.random_gqa_case(41, B, H, Hkv, D, S, dtype, valid_lens=valid)
    outs = []
    for junk in (0.0, np.nan, np.inf, -np.inf, 1e30):
        c = dict(base)
        kf, vf = base["k_fill"].copy(), base["v_fill"].copy()
        jb = np.float32(junk)
        jbits = synthetic.f32_to_bf16_bits(np.array([jb]))[0] if dtype == "bf16" else jb
        for b in range(B):
            kf[b, :, valid[b]:] = jbits
            vf[b, :, valid[b]:] = jbits
        c["k_fill"], c["v_fill"] = kf, vf
        say(f"garbage {junk} {dtype}")
        cache, ref, out, want = run_case(dev, c, dtype=dtype)
        tol_check(to_f64(out), want, dtype, f"garbage {junk}")
        outs.append(bits_of(out, dtype))
        cache.free()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_multi_step_decode_advances_on_device():
    """Eight consecutive steps on 2 layers with cache_index advanced by a
    device op between steps; each step checked against the oracle."""
    dev = device()
    B, H, Hkv, D, S, L = 4, 16, 4, 64, 160, 2
    rng = np.random.default_rng(8)
    start = np.array([100, 3, 150, 40], dtype=np.int32)
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"))
    ref = RefCache(L, B, Hkv, S, D, "bf16")
    for layer in range(L):
        k = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
        v = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
        cache.prefill_fill(layer, kvc.to_device(k, dev), kvc.to_device(v, dev), 0)
        ref.fill(layer, k, v, 0)
    ci = kvc.to_device(start, dev)
    for step in range(8):
        cur = start + step
        for layer in range(L):
            kn = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
            vn = synthetic.draw(rng, (B, Hkv, 1, D), "bf16")
            q = synthetic.draw(rng, (B, H, D), "bf16")
            cache.append(layer, kvc.to_device(kn, dev), kvc.to_device(vn, dev), ci)
            ref.append(layer, kn, vn, cur)
            out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
            cache.decode_attn(layer, kvc.to_device(q, dev), out, cache_index=ci, sm_scale=0.125)
            tol_check(to_f64(out), oracle_decode(ref, layer, q, cur + 1, 0.125), "bf16",
                      f"step {step} layer {layer}")
        ci += 1
    cache.check()
    cache.free()
