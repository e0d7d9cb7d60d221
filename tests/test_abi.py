"""CPU tests of the C ABI: the library loads, exports every function include/zha.h declares,
and rejects bad arguments on the host before touching the GPU (state left unchanged)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zha.h")


@pytest.fixture(scope="module")
def zha():
    from hierarchical_tree_indexed_03_amd import build_lib
    if not os.path.exists(build_lib.OUT):
        build_lib.build()
    from hierarchical_tree_indexed_03_amd import zha as z
    return z


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zha_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header(zha):
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(zha.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in zha.h but not exported"
    assert set(names) == set(zha.EXPORTED)


def good(zha, **kw):
    base = dict(head_dim=128, num_kv_heads=4, num_q_heads=32, block=4, levels=6, num_ref=16,
                capacity=1 << 18, dtype="bf16", top_p=0.95, keep_sink=True)
    base.update(kw)
    return zha.make_config(**base)


BAD = [
    (dict(head_dim=96), 2), (dict(num_kv_heads=0), 1), (dict(num_q_heads=30), 1),
    (dict(num_q_heads=4 * 9), 2), (dict(block=1), 1), (dict(block=257), 1), (dict(levels=0), 1),
    (dict(levels=17), 1), (dict(num_ref=3), 2), (dict(capacity=0), 1), (dict(capacity=1 << 31), 1),
    (dict(dtype=5), 1), (dict(top_p=0.0), 1), (dict(top_p=1.5), 1), (dict(top_p=float("nan")), 1),
    (dict(dtype="f32", block=256), 2), (dict(planes=3), 1), (dict(planes=-1), 1),
    (dict(block=6), 2), (dict(block=100), 2), (dict(block=255), 2),
]


@pytest.mark.parametrize("kw,status", BAD, ids=[str(k) for k, _ in BAD])
def test_invalid_configs(zha, kw, status):
    cfg = good(zha, **kw)
    assert zha.zha_workspace_bytes(cfg) == 0
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_create(cfg, 0x100000, 1 << 40)
    assert e.value.status == status
    assert zha.zha_last_error()


def test_workspace_and_handle_checks(zha):
    cfg = good(zha)
    need = zha.zha_workspace_bytes(cfg)
    assert need > 0 and need % 256 == 0
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_create(cfg, 0x100000, need - 1)
    assert e.value.status == 4
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_create(cfg, 0x100001, need)
    assert e.value.status == 1
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_create(cfg, None, need)
    assert e.value.status == 1


def test_workspace_grows_with_capacity(zha):
    a = zha.zha_workspace_bytes(good(zha, capacity=1 << 16))
    b = zha.zha_workspace_bytes(good(zha, capacity=1 << 18))
    assert b > 3 * a


def test_level1_key_form_choice(zha):
    """Key-form level-1 scoring only where the b keys plus R x b weights take fewer bytes
    than the R planes (bf16 keys, b a power of two up to 16)."""
    assert zha.zha_level1_key_form(good(zha, block=4, num_ref=16, dtype=zha.ZHA_BF16)) == 1
    assert zha.zha_level1_key_form(good(zha, block=8, num_ref=1, dtype=zha.ZHA_BF16)) == 0
    assert zha.zha_level1_key_form(good(zha, block=256, num_ref=16, dtype=zha.ZHA_BF16)) == 0
    assert zha.zha_level1_key_form(good(zha, block=4, num_ref=16, dtype=zha.ZHA_F32)) == 0
    assert zha.zha_level1_key_form(good(zha, block=16, num_ref=16, dtype=zha.ZHA_BF16)) == 1
    assert zha.zha_level1_key_form(good(zha, block=32, num_ref=16, dtype=zha.ZHA_BF16)) == 0
    assert zha.zha_level1_key_form(good(zha, block=6, num_ref=16, dtype=zha.ZHA_BF16)) == -1   # not a power of two
    assert zha.zha_level1_key_form(good(zha, block=0)) == -1
    # the token weights take extra workspace
    ws_key = zha.zha_workspace_bytes(good(zha, block=4, num_ref=16, dtype=zha.ZHA_BF16))
    ws_f32 = zha.zha_workspace_bytes(good(zha, block=4, num_ref=16, dtype=zha.ZHA_F32))
    assert ws_key > ws_f32


def test_route_keys_choice(zha):
    """Every level is scored from the keys by default on block-4 key-form trees of at least
    four levels whose level 1 fits the selection (131,072 nodes at capacity), with every
    plane format; never on trees whose router reads planes at level 1."""
    assert zha.zha_route_keys(good(zha)) == 1
    assert zha.zha_route_keys(good(zha, planes="bf16")) == 1
    assert zha.zha_route_keys(good(zha, planes="fp4")) == 1
    assert zha.zha_route_keys(good(zha, head_dim=64, num_ref=4, levels=4)) == 1
    assert zha.zha_route_keys(good(zha, levels=3)) == 0                      # fewer than 4 levels
    assert zha.zha_route_keys(good(zha, block=8, num_ref=1, levels=7)) == 0  # planes at level 1
    assert zha.zha_route_keys(good(zha, block=256, levels=1)) == 0
    assert zha.zha_route_keys(good(zha, block=2, levels=8)) == 0             # block 2
    assert zha.zha_route_keys(good(zha, dtype="f32")) == 0
    assert zha.zha_route_keys(good(zha, capacity=1 << 20)) == 0              # 262,144 level-1 nodes
    assert zha.zha_route_keys(good(zha, capacity=1 << 19)) == 1              # 131,072
    assert zha.zha_route_keys(good(zha, block=0)) == -1


def test_route_mode_setting(zha):
    """zha_set_route_mode is checked on the host; a refused mode leaves the old one."""
    cfg = good(zha, capacity=1000)
    t = zha.zha_create(cfg, 0x100000, zha.zha_workspace_bytes(cfg))
    try:
        assert zha.zha_route_mode(t) == 2
        zha.zha_set_route_mode(t, 1)
        assert zha.zha_route_mode(t) == 1
        for bad in (3, -1):
            with pytest.raises(zha.ZhaError) as e:
                zha.zha_set_route_mode(t, bad)
            assert e.value.status == 1
        assert zha.zha_route_mode(t) == 1
        zha.zha_set_route_mode(t, 2)
        assert zha.zha_route_mode(t) == 2
        zha.zha_set_route_mode(t, 0)
        assert zha.zha_route_mode(t) == 2
    finally:
        zha.zha_destroy(t)
    cfg = good(zha, capacity=1000, block=8, num_ref=1, levels=3)
    t = zha.zha_create(cfg, 0x100000, zha.zha_workspace_bytes(cfg))
    try:
        assert zha.zha_route_mode(t) == 1
        with pytest.raises(zha.ZhaError) as e:
            zha.zha_set_route_mode(t, 2)
        assert e.value.status == 2
        assert zha.zha_route_mode(t) == 1
    finally:
        zha.zha_destroy(t)
    assert zha.zha_route_mode(None) == -1
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_set_route_mode(None, 0)
    assert e.value.status == 1


@pytest.mark.parametrize("fmt", ["bf16", "fp4"])
def test_quantised_router_planes_workspace(zha, fmt):
    """Quantised router planes add one copy of s per level the router reads planes at: every
    level but a key-form level 1 (whose planes the router never reads).  bf16: R x d x 2
    bytes per node; MX FP4: R x d / 2 bytes of codes plus R x d / 32 scale bytes."""
    D, H, cap = 128, 4, 1 << 18

    def slot(nbytes):
        return -(-nbytes // 256) * 256

    def planes_bytes(levels, b, R):
        # per-level node capacity rounded to 64 nodes, 256-byte aligned slots
        tot = 0
        for lv in levels:
            n = -(-cap // b ** lv)
            n = -(-n // 64) * 64
            tot += slot(H * n * R * D * 2) if fmt == "bf16" else slot(H * n * R * D // 2) + slot(H * n * R * D // 32)
        return tot
    # key-form level 1 (bf16, b 4, R 16): levels 2..6 get a copy
    f = zha.zha_workspace_bytes(good(zha))
    q = zha.zha_workspace_bytes(good(zha, planes=fmt))
    assert q - f == planes_bytes(range(2, 7), 4, 16)
    # planes read at level 1 too (b 8, R 1)
    f = zha.zha_workspace_bytes(good(zha, block=8, num_ref=1, levels=7))
    q = zha.zha_workspace_bytes(good(zha, block=8, num_ref=1, levels=7, planes=fmt))
    assert q - f == planes_bytes(range(1, 8), 8, 1)


def test_call_order_and_arguments(zha):
    """Handle created on a fake (never dereferenced) address: every call below must fail
    validation on the host and leave the handle as it was."""
    cfg = good(zha, capacity=1000)
    t = zha.zha_create(cfg, 0x100000, zha.zha_workspace_bytes(cfg))
    try:
        fake = 0x200000
        for call, status in [
            (lambda: zha.zha_decode(t, fake, fake), 5),
            (lambda: zha.zha_decode_dense(t, fake, fake), 5),
            (lambda: zha.zha_tree_append(t, fake, fake), 5),
            (lambda: zha.zha_debug_level(t, 1, fake, fake), 5),
            (lambda: zha.zha_debug_router_planes(t, 2, fake), 5),
            (lambda: zha.zha_tree_append_n(t, fake, fake, 4), 5),
            (lambda: zha.zha_prefill(t, fake, fake, fake, fake, 4), 5),
            (lambda: zha.zha_prefill_batched(t, fake, fake, fake, fake, 4, 4, fake, 1 << 30), 5),
            (lambda: zha.zha_debug_prefill_trace(t, 1, fake, fake), 5),
            (lambda: zha.zha_tree_build(t, fake, fake, 1001, fake), 3),
            (lambda: zha.zha_tree_build(t, fake, fake, 0, fake), 1),
            (lambda: zha.zha_tree_build(t, None, fake, 10, fake), 1),
            (lambda: zha.zha_tree_build(t, fake + 2, fake, 10, fake), 1),
        ]:
            with pytest.raises(zha.ZhaError) as e:
                call()
            assert e.value.status == status
            assert zha.zha_num_tokens(t) == 0
    finally:
        zha.zha_destroy(t)


def test_top_p_levels_validation(zha):
    """The per-level p schedule is checked on the host; a bad schedule leaves the old one."""
    cfg = good(zha, capacity=1000, levels=3)
    t = zha.zha_create(cfg, 0x100000, zha.zha_workspace_bytes(cfg))
    try:
        zha.zha_set_top_p_levels(t, [0.5, 0.9, 1.0])
        zha.zha_set_top_p_levels(t, None)
        for bad in ([0.5, 0.0, 1.0], [0.5, 1.5, 1.0], [float("nan"), 0.9, 0.9], [-0.1, 0.9, 0.9]):
            with pytest.raises(zha.ZhaError) as e:
                zha.zha_set_top_p_levels(t, bad)
            assert e.value.status == 1
    finally:
        zha.zha_destroy(t)
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_set_top_p_levels(None, [0.5])
    assert e.value.status == 1


def test_status_strings(zha):
    for s in range(7):
        assert zha.zha_status_string(s)


def test_dense_static_argument_errors(zha):
    """The allocation-free dense decode validates on the host before any HIP call."""
    import ctypes as C
    cfg = good(zha)
    buf = C.create_string_buffer(64)
    p = C.addressof(buf) + (-C.addressof(buf)) % 16
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_decode_dense_static(cfg, None, p, 10, p, p)
    assert e.value.status == 1
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_decode_dense_static(cfg, p, p, 0, p, p)
    assert e.value.status == 1
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_decode_dense_static(cfg, p, p, (1 << 18) + 1, p, p)
    assert e.value.status == 3
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_decode_dense_static(good(zha, head_dim=96), p, p, 10, p, p)
    assert e.value.status == 2
    # one split's partials over 8,800 query heads exceed the 4 MiB static scratch
    with pytest.raises(zha.ZhaError) as e:
        zha.zha_decode_dense_static(good(zha, num_kv_heads=1100, num_q_heads=8800), p, p, 10, p, p)
    assert e.value.status == 4 and "static scratch" in str(e.value)


def test_prefill_workspace_bytes(zha):
    """The batched-prefill workspace: 0 for a bad config or a batch outside 1..128, else
    256-byte granular and growing with the batch and with the capacity."""
    cfg = good(zha)
    assert zha.zha_prefill_workspace_bytes(cfg, 0) == 0
    assert zha.zha_prefill_workspace_bytes(cfg, 129) == 0
    assert zha.zha_prefill_workspace_bytes(good(zha, head_dim=96), 4) == 0
    a, b = zha.zha_prefill_workspace_bytes(cfg, 1), zha.zha_prefill_workspace_bytes(cfg, 128)
    assert a > 0 and a % 256 == 0 and b % 256 == 0 and b > 64 * a
    assert zha.zha_prefill_workspace_bytes(good(zha, capacity=1 << 20), 16) > \
        3 * zha.zha_prefill_workspace_bytes(cfg, 16)
