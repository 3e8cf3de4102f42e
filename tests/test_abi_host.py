"""The C-ABI library on the host (no GPU needed): it loads, exports every
entry point include/kvc.h declares, and its pure-host byte accounting
matches the oracle. No call here touches the device."""

import ctypes
import os
import re

import pytest

from oracle import cache_bytes as cb
from static_kv_cache_amd import kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvc.LIB_PATH):
        pytest.fail("libkvc.so is not built (run __graft_entry__.build())")
    return kvc.load()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for required in ("kvc_alloc", "kvc_prefill_fill", "kvc_append", "kvc_decode_attn",
                     "kvc_mla_decode", "kvc_bytes", "kvc_free", "kvc_check"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(kvc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, f"not exported: {missing}"
    assert set(declared_functions()) == set(kvc._SIGS), "binding and header disagree"


@pytest.mark.parametrize("shape", [
    (1, 1, 4, 4, 32, 128, "f32"),        # tiny MHA
    (12, 8, 8, 8, 32, 512, "bf16"),      # DantinoX MHA
    (12, 8, 8, 2, 32, 512, "bf16"),      # DantinoX GQA
    (32, 16, 32, 8, 128, 4096, "bf16"),  # Llama-3-8B-shaped
    (80, 1, 64, 8, 128, 32768, "bf16"),  # long context (80 layers)
    (80, 1, 64, 64, 128, 4096, "bf16"),  # the Llama-2-70B printed example
    (32, 1, 32, 32, 128, 1024, "f32"),   # the Llama-3 fp32 printed example
])
def test_kvc_bytes_matches_oracle(lib, shape):
    L, B, H, Hkv, D, S, dt = shape
    got = kvc.cache_bytes(kvc.gqa_desc(L, B, H, Hkv, D, S, dt))
    assert got == cb.kv_cache_bytes(L, Hkv, D, S, B, 4 if dt == "f32" else 2)


@pytest.mark.parametrize("shape", [
    (1, 2, 8, 2, 64, 100), (32, 16, 32, 8, 128, 4096), (2, 3, 16, 1, 256, 70),
])
def test_kvc_bytes_int8_matches_oracle(lib, shape):
    """int8 cache: codes at p_cache = 1 (section 4.4) plus one float32 scale per K and V row."""
    from oracle import quant
    L, B, H, Hkv, D, S = shape
    got = kvc.cache_bytes(kvc.gqa_desc(L, B, H, Hkv, D, S, "i8"))
    assert got == quant.int8_cache_bytes(L, Hkv, D, S, B)
    assert got == cb.kv_cache_bytes(L, Hkv, D, S, B, 1) + 2 * L * Hkv * S * B * 4


def test_kvc_bytes_printed_examples(lib):
    assert kvc.cache_bytes(kvc.gqa_desc(80, 1, 64, 64, 128, 4096, "bf16")) == 10737418240
    assert kvc.cache_bytes(kvc.gqa_desc(32, 1, 32, 32, 128, 1024, "f32")) == 1073741824
    assert kvc.cache_bytes(kvc.gqa_desc(80, 1, 64, 8, 128, 32768, "bf16")) == 10737418240


def test_kvc_bytes_latent(lib):
    got = kvc.cache_bytes(kvc.mla_desc(1, 32, 16, 4096))
    assert got == cb.mla_cache_bytes(1, 512, 4096, 32, 2, rope_dim=64) == 150994944


@pytest.mark.parametrize("bad", [
    dict(n_heads=6, n_kv_heads=4),      # H not a multiple of H_kv
    dict(n_layers=0), dict(batch=0), dict(max_context=0), dict(n_kv_heads=0),
    dict(dtype=7), dict(attn=3), dict(latent_dim=8), dict(batch=-4),
])
def test_kvc_bytes_rejects_bad_descriptors(lib, bad):
    fields = dict(attn=0, dtype=1, n_layers=2, batch=2, n_heads=8, n_kv_heads=2, head_dim=32,
                  max_context=64, latent_dim=0, rope_dim=0)
    fields.update(bad)
    d = kvc.Desc(**fields)
    out = ctypes.c_uint64(0)
    assert lib.kvc_bytes(ctypes.byref(d), ctypes.byref(out)) == kvc.KVC_ERR_INVALID_ARG


def test_unsupported_head_dim_and_null(lib):
    d = kvc.gqa_desc(1, 1, 4, 4, 48, 16, "bf16")
    out = ctypes.c_uint64(0)
    assert lib.kvc_bytes(ctypes.byref(d), ctypes.byref(out)) == kvc.KVC_ERR_UNSUPPORTED
    assert lib.kvc_bytes(None, ctypes.byref(out)) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_bytes(ctypes.byref(kvc.gqa_desc(1, 1, 4, 4, 32, 16, "bf16")), None) == kvc.KVC_ERR_INVALID_ARG


@pytest.mark.parametrize("desc", [
    kvc.mla_desc(1, 2, 24, 64),                 # latent heads: <= 16 or a multiple of 16
    kvc.mla_desc(1, 1, 16, 1 << 20),            # latent rows of one sequence >= 2^30 bytes
    kvc.gqa_desc(1, 1, 8, 8, 256, 1 << 21, "bf16"),   # one (sequence, kv head) block >= 2^30 bytes
    kvc.gqa_desc(1, 2048, 8, 8, 32, 1 << 20, "bf16"),  # row space of all sequences >= 2^31
    kvc.gqa_desc(1, 2, 8, 8, 32, 64, "i8"),            # int8 rows need head_dim >= 64
    kvc.mla_desc(1, 2, 16, 64, dtype="i8"),            # int8 latent cache
], ids=["mla_heads", "mla_rows", "gqa_block", "row_space", "i8_head_dim", "i8_latent"])
def test_unsupported_sizes(lib, desc):
    out = ctypes.c_uint64(0)
    assert lib.kvc_bytes(ctypes.byref(desc), ctypes.byref(out)) == kvc.KVC_ERR_UNSUPPORTED


def test_host_only_calls_reject_null_handles(lib):
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.kvc_layer_ptrs(None, 0, ctypes.byref(k), ctypes.byref(v)) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_set_workgroups(None, 64) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_free(None) == kvc.KVC_OK
    for s in range(7):
        assert lib.kvc_strerror(s)


@pytest.mark.parametrize("shape", [
    (1, 2, 8, 2, 128, 64, 16, 9),        # small: 9 blocks of 16 rows
    (32, 16, 32, 8, 128, 4096, 16, 4096),  # Llama-3-8B-shaped, 4096 blocks of 16
    (2, 1, 4, 4, 64, 1024, 256, 5),       # largest block size
])
def test_kvc_bytes_paged_matches_pool_model(lib, shape):
    """Block-table cache bytes equal the oracle pool's size: [L][2][num_blocks][H_kv][block_size][D] bf16."""
    from oracle.paged import RefPagedCache
    L, B, H, Hkv, D, S, bs, nb = shape
    got = kvc.paged_cache_bytes(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"), bs, nb)
    assert got == 2 * L * nb * Hkv * bs * D * 2
    if L * nb * bs <= 1 << 16:
        assert got == RefPagedCache(L, nb, Hkv, bs, D, "bf16", S).pool.nbytes


@pytest.mark.parametrize("desc,bs,nb,status", [
    (kvc.gqa_desc(1, 2, 8, 2, 128, 64, "bf16"), 24, 8, kvc.KVC_ERR_INVALID_ARG),   # 64 % 24 != 0
    (kvc.gqa_desc(1, 2, 8, 2, 128, 64, "bf16"), 0, 8, kvc.KVC_ERR_INVALID_ARG),
    (kvc.gqa_desc(1, 2, 8, 2, 128, 64, "bf16"), 16, 0, kvc.KVC_ERR_INVALID_ARG),
    (kvc.gqa_desc(1, 2, 8, 2, 128, 64, "bf16"), 8, 8, kvc.KVC_ERR_UNSUPPORTED),    # tiles span <= 2 blocks
    (kvc.gqa_desc(1, 2, 8, 2, 128, 96, "bf16"), 48, 8, kvc.KVC_ERR_UNSUPPORTED),   # not a power of two
    (kvc.gqa_desc(1, 2, 8, 2, 128, 1024, "bf16"), 512, 8, kvc.KVC_ERR_UNSUPPORTED),
    (kvc.gqa_desc(1, 2, 8, 2, 128, 16 * 4097, "bf16"), 16, 8, kvc.KVC_ERR_UNSUPPORTED),  # table > 4096
    (kvc.gqa_desc(1, 2, 8, 8, 128, 64, "bf16"), 16, 1 << 16, kvc.KVC_ERR_UNSUPPORTED),   # pool >= 2^30
    (kvc.gqa_desc(1, 2, 8, 2, 128, 64, "f32"), 16, 8, kvc.KVC_ERR_UNSUPPORTED),
    (kvc.gqa_desc(1, 2, 8, 2, 128, 64, "i8"), 16, 8, kvc.KVC_ERR_UNSUPPORTED),
    (kvc.mla_desc(1, 2, 16, 64), 16, 8, kvc.KVC_ERR_UNSUPPORTED),
], ids=["ragged", "bs0", "nb0", "bs8", "bs48", "bs512", "wide_table", "big_pool", "f32", "i8", "latent"])
def test_kvc_bytes_paged_rejects(lib, desc, bs, nb, status):
    out = ctypes.c_uint64(0)
    assert lib.kvc_bytes_paged(ctypes.byref(desc), bs, nb, ctypes.byref(out)) == status


def test_paged_calls_reject_null_handles(lib):
    z = ctypes.c_void_p(16)
    assert lib.kvc_paged_append(None, 0, z, z, z, z, 1, None) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_paged_decode_attn(None, 0, z, z, z, z, z, ctypes.c_float(0.1), None) == kvc.KVC_ERR_INVALID_ARG
    assert (lib.kvc_paged_append_decode_attn(None, 0, z, z, z, z, z, z, ctypes.c_float(0.1), None)
            == kvc.KVC_ERR_INVALID_ARG)
    assert lib.kvc_bytes_paged(None, 16, 4, ctypes.byref(ctypes.c_uint64())) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_alloc_paged(None, 16, 4, None, None) == kvc.KVC_ERR_INVALID_ARG


def test_prefix_calls_reject_null_handles(lib):
    z = ctypes.c_void_p(16)
    n = ctypes.c_uint64(0)
    lens = (ctypes.c_int32 * 2)(1, 1)
    assert lib.kvc_prefix_bytes(None, lens, ctypes.byref(n)) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_save_prefix(None, lens, z, 4096, None) == kvc.KVC_ERR_INVALID_ARG
    assert lib.kvc_load_prefix(None, z, 4096, lens, lens, None) == kvc.KVC_ERR_INVALID_ARG


def test_noalloc_decode_rejects_before_any_device_call(lib):
    """kvc_decode_attn_noalloc checks its descriptor and arguments on the host
    first: bad ones return a status without touching the device."""
    fn = lib.kvc_decode_attn_noalloc
    p = ctypes.c_void_p(16)  # never dereferenced: every call below is rejected first
    good = kvc.gqa_desc(1, 2, 8, 2, 128, 64, "bf16")
    assert fn(None, p, p, p, p, p, p, 0.125, None, None) == kvc.KVC_ERR_INVALID_ARG
    assert fn(ctypes.byref(good), None, p, p, p, p, p, 0.125, None, None) == kvc.KVC_ERR_INVALID_ARG
    assert fn(ctypes.byref(good), p, p, p, None, p, p, 0.125, None, None) == kvc.KVC_ERR_INVALID_ARG
    assert fn(ctypes.byref(good), p, p, p, p, None, None, 0.125, None, None) == kvc.KVC_ERR_INVALID_ARG
    assert fn(ctypes.byref(good), p, p, p, p, p, p, 0.0, None, None) == kvc.KVC_ERR_INVALID_ARG
    i8 = kvc.gqa_desc(1, 2, 8, 2, 128, 64, "i8")
    assert fn(ctypes.byref(i8), p, p, p, p, p, p, 0.125, None, None) == kvc.KVC_ERR_UNSUPPORTED
    mla = kvc.mla_desc(1, 2, 16, 64)
    assert fn(ctypes.byref(mla), p, p, p, p, p, p, 0.125, None, None) == kvc.KVC_ERR_UNSUPPORTED
    wide = kvc.gqa_desc(1, 2048, 64, 8, 128, 64, "bf16")  # 131,072 (sequence, head) pairs
    assert fn(ctypes.byref(wide), p, p, p, p, p, p, 0.125, None, None) == kvc.KVC_ERR_UNSUPPORTED
