"""Host-side checks of libhisa.so that need no GPU: the library loads, exports
every function include/hisa.h declares, sizes workspaces, and turns bad
arguments into the documented error codes before anything is enqueued."""
import ctypes
import os
import re

import pytest

from top_kv_indexer_amd import hisa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hisa.LIB_PATH):
        from top_kv_indexer_amd import build
        build.build()
    return hisa.lib()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(hisa.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.hisa_abi_version() == 3


def dims(**kw):
    base = dict(B=1, L=1, ratio=4, window=128, topk=512, index_block=64, index_keep=16, H_i=64, D_i=128,
                H=64, Dk=512, Dv=512, Np_cap=16384, Wl_cap=128, kI=512, mode=0, idx_dtype=hisa.BF16,
                attn_dtype=hisa.BF16)
    base.update(kw)
    return hisa.hisa_dims(**base)


def test_workspace_sizes(lib):
    d = dims()
    # decode: the arrival counters (1 sequence + 16 slab-group counters, 64
    # bytes each, rounded up to 256), f32 scores of every pooled row + one
    # coarse score per block
    assert hisa.workspace_bytes(hisa.OP_SELECT_DECODE, d) == 1280 + 16384 * 4 + 256 * 4
    # 32 sequences of up to 512 slabs: 32 sequence counters + 32 x 32 group counters
    assert hisa.workspace_bytes(hisa.OP_SELECT_DECODE, dims(B=32, Np_cap=32768)) == (
        32 * 33 * 64 + 32 * 32768 * 4 + 32 * 512 * 4)
    assert hisa.workspace_bytes(hisa.OP_FLAT_TOPK, dims(L=4, Np_cap=1000)) == ((4 * 1000 * 4 + 255) // 256) * 256
    # the flat top-k needs the scores only, at decode as in prefill
    assert hisa.workspace_bytes(hisa.OP_FLAT_TOPK, dims(B=2, ratio=1, topk=2048, Np_cap=32768)) == 2 * 32768 * 4
    assert hisa.workspace_bytes(hisa.OP_FLAT_TOPK, dims(B=2, L=2, ratio=1, topk=2048, Np_cap=32768)) == 4 * 32768 * 4
    assert hisa.workspace_bytes(hisa.OP_FLAT_TOPK, dims(ratio=1, Np_cap=8192)) == 8192 * 4
    assert hisa.workspace_bytes(hisa.OP_FLAT_TOPK, dims(ratio=1, Np_cap=32768, idx_dtype=hisa.F32)) == 32768 * 4
    # single-row attention splits the 640 rows into 10 parts of 64
    assert hisa.workspace_bytes(hisa.OP_ATTENTION, d) == 10 * 64 * (2 * 512 + 8)
    # decode step: sync words (error word, then per sequence one line each of
    # "seen" and threshold, 16 split descriptors of 8 bytes: 320 bytes,
    # rounded to 512),
    # the decode selection's workspace, and the partials of 16 pooled + 2 local
    # splits of 64 heads (more than the attention call's 10)
    assert hisa.workspace_bytes(hisa.OP_DECODE_STEP, d) == 512 + (1280 + 16384 * 4 + 256 * 4) + 18 * 64 * (2 * 512 + 8)
    # many rows: no split, no workspace
    assert hisa.workspace_bytes(hisa.OP_ATTENTION, dims(L=2048, Wl_cap=2175)) == 0
    # batched selection, sized by the kernels that run: one query row per wave
    # needs only the block means (f32 + three bf16 parts) ...
    rep = 256 * 128 * 4 + 3 * 256 * 128 * 2
    assert hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, dims(L=2048)) == rep
    # ... plus the flat scores of every row when the flat scan runs (forced flat)
    assert hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, dims(L=2048, mode=hisa.MODE_FORCE_FLAT)) == (
        rep + 2048 * 16384 * 4)
    # candidates past one wave's registers: coarse scores per row and the flat scan
    assert hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, dims(L=2048, index_keep=64)) == (
        rep + 2048 * 256 * 4 + 2048 * 16384 * 4)
    # a short chunk (B * L <= 192 rows): every block mean (f32), then per row
    # the cached-means selection (counters, block scores, kept blocks, candidates)
    assert hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, dims(L=4)) == (
        256 * 128 * 4 + r256(cached_counter_bytes(4)) + 4 * 256 * 4 + 256 + 4 * 1024 * 4)
    assert hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, dims(L=192)) == (
        256 * 128 * 4 + r256(cached_counter_bytes(192)) + 192 * 256 * 4 + 192 * 16 * 4 + 192 * 1024 * 4)
    # one row more: one query row per wave
    assert hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, dims(L=193)) == rep
    # no hierarchy: only the flat scan
    assert hisa.workspace_bytes(hisa.OP_SELECT_PREFILL, dims(L=4, index_block=0, Np_cap=1000)) == (
        (4 * 1000 * 4 + 255) // 256 * 256)
    # the dense fallback fills I and needs nothing
    for op in (hisa.OP_SELECT_DECODE, hisa.OP_SELECT_PREFILL):
        assert hisa.workspace_bytes(op, dims(topk=16384, mode=hisa.MODE_FORCE_DENSE)) == 0


def test_force_dense_needs_room_for_every_pooled_row(lib):
    d = dims(topk=512, mode=hisa.MODE_FORCE_DENSE)
    for op in (hisa.OP_SELECT_DECODE, hisa.OP_SELECT_PREFILL):
        assert lib.hisa_workspace_bytes(op, ctypes.byref(d)) == ctypes.c_size_t(-1).value
        assert "FORCE_DENSE" in hisa.last_error()
    fake = ctypes.c_void_p(256)
    rc = lib.hisa_select_decode(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, None, 0, None)
    assert rc == -1
    # the switches do not apply to the coarse stage alone or to the flat indexer
    assert hisa.workspace_bytes(hisa.OP_BLOCK_SCORES, d) > 0
    assert hisa.workspace_bytes(hisa.OP_FLAT_TOPK, d) > 0


@pytest.mark.parametrize("op,kw,code", [
    (hisa.OP_SELECT_DECODE, dict(L=2), -1),
    (hisa.OP_SELECT_DECODE, dict(index_block=48), -1),
    (hisa.OP_SELECT_DECODE, dict(index_keep=0), -1),
    (hisa.OP_SELECT_DECODE, dict(index_keep=2000), -1),
    (hisa.OP_SELECT_DECODE, dict(idx_dtype=7), -2),
    (hisa.OP_SELECT_DECODE, dict(topk=0), -1),
    (hisa.OP_SELECT_DECODE, dict(mode=3), -1),
    (hisa.OP_SELECT_DECODE, dict(B=0), -1),
    (hisa.OP_SELECT_DECODE, dict(Np_cap=0), -1),
    (hisa.OP_SELECT_DECODE, dict(ratio=4, Np_cap=600000000), -4),
    (hisa.OP_BLOCK_SCORES, dict(index_block=0), -1),
    (hisa.OP_ATTENTION, dict(Dv=600), -1),
    (hisa.OP_ATTENTION, dict(attn_dtype=3), -2),
    (hisa.OP_ATTENTION, dict(attn_dtype=hisa.F32, Dk=2048, Dv=2048), -1),
    (hisa.OP_ATTENTION, dict(kI=-1), -1),
])
def test_bad_dims_are_rejected(lib, op, kw, code):
    d = dims(**kw)
    assert lib.hisa_workspace_bytes(op, ctypes.byref(d)) == ctypes.c_size_t(-1).value
    assert hisa.last_error() != ""
    fake = ctypes.c_void_p(256)  # never dereferenced: the checks fail first
    if op == hisa.OP_SELECT_DECODE:
        rc = lib.hisa_select_decode(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, fake, 1 << 30, None)
    elif op == hisa.OP_BLOCK_SCORES:
        rc = lib.hisa_block_scores(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, 1 << 30, None)
    else:
        rc = lib.sparse_local_pooled_attention(ctypes.byref(d), fake, fake, fake, fake, None, fake, fake, fake,
                                               1 << 30, None)
    assert rc == code, hisa.last_error()


def test_small_workspace_and_null_pointers(lib):
    d = dims()
    fake = ctypes.c_void_p(256)
    rc = lib.hisa_select_decode(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, fake, 16, None)
    assert rc == -3 and "workspace" in hisa.last_error()
    rc = lib.hisa_select_decode(ctypes.byref(d), fake, fake, fake, fake, None, None, None, fake, 1 << 30, None)
    assert rc == -1 and "NULL" in hisa.last_error()
    rc = lib.hisa_select_decode(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, ctypes.c_void_p(257),
                                1 << 30, None)
    assert rc == -1 and "aligned" in hisa.last_error()
    rc = lib.flat_topk_select(None, fake, fake, fake, fake, fake, fake, 1 << 30, None)
    assert rc == -1


def test_noalloc_decode_rejects_dims_past_its_workspace(lib):
    # 16 MiB of library-held workspace: B = 32 at Np_cap = 32768 (4.3 MB) fits,
    # B = 128 at Np_cap = 65536 (about 34 MB) does not and fails before any
    # GPU call.
    assert hisa.workspace_bytes(hisa.OP_SELECT_DECODE, dims(B=32, Np_cap=32768)) <= hisa.NOALLOC_MAX_BYTES
    d = dims(B=128, Np_cap=65536)
    assert hisa.workspace_bytes(hisa.OP_SELECT_DECODE, d) > hisa.NOALLOC_MAX_BYTES
    fake = ctypes.c_void_p(256)
    rc = lib.hisa_select_decode_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, None)
    assert rc == -3 and "noalloc" in hisa.last_error()
    rc = lib.hisa_select_decode_noalloc(ctypes.byref(dims(L=2)), fake, fake, fake, fake, fake, None, None, None)
    assert rc == -1


def r256(n):
    return (n + 255) // 256 * 256


def cached_counter_bytes(rows, groups=1):
    # per row one coarse counter and the group counters, one fine counter (each
    # on its own 64-byte line), then the error line and 16 descriptor words per
    # row (the one-launch form's hand-off of the kept blocks)
    return rows * (1 + groups) * 64 + rows * 64 + 64 + rows * 16 * 8


def test_cached_decode_workspace_and_limits(lib):
    # counters (1 sequence + 1 group counter for 16 workgroups, + 1 for the
    # fine stage, the error line and the descriptors, rounded to 256), block
    # scores, kept blocks, 1024 candidate scores
    d = dims()
    assert hisa.workspace_bytes(hisa.OP_SELECT_DECODE_CACHED, d) == (
        r256(cached_counter_bytes(1)) + 256 * 4 + 256 + 1024 * 4)
    assert hisa.workspace_bytes(hisa.OP_BLOCK_MEANS_UPDATE, d) == 0
    for kw in (dict(index_block=0), dict(Np_cap=64 * 4097), dict(index_keep=32), dict(mode=hisa.MODE_FORCE_FLAT),
               dict(index_keep=4), dict(idx_dtype=hisa.F32), dict(H_i=32), dict(B=40000, L=2)):
        bad = dims(**kw)
        assert lib.hisa_workspace_bytes(hisa.OP_SELECT_DECODE_CACHED, ctypes.byref(bad)) == ctypes.c_size_t(-1).value, kw
    fake = ctypes.c_void_p(256)
    rc = lib.hisa_select_decode_cached(ctypes.byref(dims(index_keep=32)), fake, fake, fake, fake, fake, fake, None, None,
                                       fake, 1 << 30, None)
    assert rc == -1 and "hisa_select_decode_cached needs" in hisa.last_error()
    rc = lib.hisa_block_means_update(ctypes.byref(dims(index_block=0)), fake, fake, fake, None)
    assert rc == -1
    rc = lib.hisa_block_means_update(ctypes.byref(dims()), fake, fake, None, None)
    assert rc == -1 and "NULL" in hisa.last_error()


def test_ring_attention_needs_room_for_the_window(lib):
    fake = ctypes.c_void_p(256)
    d = dims(L=4, Wl_cap=130)  # window 128 + L - 1 = 131 positions
    rc = lib.sparse_local_pooled_attention_ring(ctypes.byref(d), fake, fake, fake, fake, None, fake, None, fake, fake,
                                                1 << 30, None)
    assert rc == -1 and "ring" in hisa.last_error()
