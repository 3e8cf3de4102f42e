"""The bf16 parity check can fail where it matters: at the exact inputs of the
full-size GPU tests, plausible kernel mistakes are rejected by it.

For the long-context shape (B=1, H=64, H_kv=8, d_h=128, 32,768 valid rows;
the inputs of the GPU test's layer 79) and the Llama-3-8B-shaped layer
(B=16, H=32, H_kv=8, ragged lengths), the oracle's own output rounded to bf16
(what a perfect kernel would store) must pass the check, and each planted
mistake, also rounded to bf16, must fail it:
  * the appended row left out (attend n - 1 rows instead of n);
  * one 64-row tile left out of every (sequence, kv head)'s rows.
The element-wise bound alone passes both mistakes at long context, whose
output RMS (~0.009) is below its absolute term; the per-row L2 bound in
``tol_check`` is what catches them. The mistakes are computed by the oracle
on altered inputs, on the CPU; the oracle itself is untouched.
"""

import numpy as np
import pytest

from gpu_util import tol_check
from oracle import attention as oatt
from oracle.buffer import RefCache
from static_kv_cache_amd import synthetic


def as_bf16(x):
    """float64 -> the value stored as bf16 (round to nearest even), as float64."""
    bits = synthetic.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def layer_inputs(name, layer, fill_rows):
    cfg = synthetic.WORKLOADS[name]
    B, Hkv, D, S = cfg["batch"], cfg["n_kv_heads"], cfg["head_dim"], cfg["max_context"]
    c = synthetic.gqa_layer(cfg, seed_offset=layer, fill_rows=fill_rows)
    ref = RefCache(1, B, Hkv, S, D, "bf16")
    ref.fill(0, c["k_fill"], c["v_fill"], 0)
    ref.append(0, c["k_new"], c["v_new"], c["cache_index"])
    return c, ref


def tile_dropped(c, ref, tile=64):
    """Decode with rows [t0, t0 + tile) of every (sequence, kv head) left out,
    t0 the tile boundary nearest the middle of the valid rows."""
    k, v = ref.keys(0), ref.values(0)
    out = []
    for b, n in enumerate(c["valid_lens"]):
        t0 = (int(n) // 2) // tile * tile
        keep = np.r_[0:t0, t0 + tile:int(n)]
        out.append(oatt.decode_attention(c["q"][b:b + 1], k[b][:, keep][None], v[b][:, keep][None],
                                         [len(keep)], c["sm_scale"])[0])
    return np.stack(out)


@pytest.mark.parametrize("name,layer,fill_rows", [
    ("longctx_gqa_bf16", 79, 32767),
    ("llama3_8b_gqa_bf16", 0, None),
])
def test_check_rejects_planted_mistakes(name, layer, fill_rows):
    c, ref = layer_inputs(name, layer, fill_rows)
    want = oatt.decode_attention(c["q"], ref.keys(0), ref.values(0), c["valid_lens"], c["sm_scale"])
    tol_check(as_bf16(want), want, "bf16", "exact output stored as bf16")
    mistakes = {
        "appended row left out": oatt.decode_attention(c["q"], ref.keys(0), ref.values(0),
                                                       c["valid_lens"] - 1, c["sm_scale"]),
        "one 64-row tile left out": tile_dropped(c, ref),
    }
    for what, got in mistakes.items():
        with pytest.raises(AssertionError):
            tol_check(as_bf16(got), want, "bf16", what)
