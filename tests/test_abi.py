"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before launching anything.

Pointers passed here are fake (aligned, never dereferenced): every checked
error returns before any device work.
"""

import ctypes
import os
import re

import pytest

from kv_cached_gqa_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

FAKE = 1 << 20  # 16-byte aligned, never dereferenced


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libkvc.so is not built; run __graft_entry__.build() first")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    declared = _header_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layout_matches_header():
    # 3 pointers + 3 int64 + 6 int32, no padding
    assert ctypes.sizeof(_lib.KvcCache) == 3 * 8 + 3 * 8 + 6 * 4
    assert _lib.KvcCache.stride_seq.offset == 24
    assert _lib.KvcCache.dtype.offset == 48


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        s = lib.kvc_status_string(code).decode()
        assert s.startswith("KVC_")
    assert "unknown" in lib.kvc_status_string(7).decode()


def test_header_constants_match_the_binding():
    import re

    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "kvc.h")).read()
    assert int(re.search(r"#define KVC_MAX_T (\d+)", hdr).group(1)) == _lib.KVC_MAX_T


def test_workspace_bytes(lib):
    assert lib.kvc_workspace_bytes(64, 1, 32, 8, 128, 4097, 0) > 0
    assert lib.kvc_workspace_bytes(64, 1, 32, 8, 96, 4097, 0) == 0  # H
    assert lib.kvc_workspace_bytes(64, 1, 30, 8, 128, 4097, 0) == 0  # N % K
    assert lib.kvc_workspace_bytes(64, 2049, 32, 8, 128, 4097, 0) == 0  # T > KVC_MAX_T
    assert lib.kvc_workspace_bytes(8, 512, 32, 8, 128, 4097, 0) > 0  # chunked prefill
    assert lib.kvc_workspace_bytes(0, 1, 32, 8, 128, 4097, 0) == 0  # B
    a = lib.kvc_workspace_bytes(8, 5, 64, 8, 128, 9000, 100)
    b = lib.kvc_workspace_bytes(8, 5, 64, 8, 128, 9000, 1000)
    assert 0 < a < b


def test_workspace_layout_follows_the_row_block_rule(lib):
    """The workspace is the counter array, then per slot (worker or unit) the
    row statistics and the fp32 rows of a partial. Row blocks hold all G*T
    rows up to 64 (vector path up to 4 at H = 128) and 128 rows beyond, so
    the size pins the rule the header states."""
    counters = 1 << 18

    def expect(units, workers, rmax, H):
        up = lambda x: (x + 255) // 256 * 256
        slots = workers + units
        return counters * 4 + up(slots * rmax * 2 * 4) + up(slots * rmax * H * 4)

    W = 100  # an explicit grid: the automatic one depends on the device
    B, K, H = 8, 8, 128
    for T, N, rmax, rb in [(1, 32, 4, 1), (5, 64, 48, 1), (16, 32, 64, 1), (17, 32, 128, 1),
                           (32, 32, 128, 1), (33, 32, 128, 2), (512, 32, 128, 16)]:
        got = lib.kvc_workspace_bytes(B, T, N, K, H, 4097, W)
        assert got == expect(B * K * rb, W, rmax, H), (T, N)


def _cache(**kw):
    c = _lib.KvcCache()
    c.k = FAKE
    c.v = FAKE * 2
    c.block_table = None
    c.stride_seq = 8 * 4096 * 128
    c.stride_head = 4096 * 128
    c.stride_tok = 128
    c.dtype = _lib.KVC_BF16
    c.capacity = 4096
    c.block_size = 0
    c.max_blocks_per_seq = 0
    c.num_blocks = 0
    c.reserved = 0
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _decode(lib, cache, B=64, N=32, K=8, H=128, max_seq_len=4096, out_dtype=_lib.KVC_F32, q=FAKE,
            ws=FAKE, ws_bytes=1 << 30, scale=0.088, nwg=0, seq_lens=FAKE):
    cp = ctypes.byref(cache) if cache is not None else None
    return lib.kvc_attn_decode(cp, q, FAKE, out_dtype, None, B, N, K, H, seq_lens, max_seq_len,
                               scale, nwg, ws, ws_bytes, None)


def test_decode_host_errors(lib):
    E = _lib
    assert _decode(lib, None) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(k=None)) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(reserved=1)) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(dtype=E.KVC_F32)) == E.KVC_ERR_UNSUPPORTED
    assert _decode(lib, _cache(), H=96) == E.KVC_ERR_UNSUPPORTED
    assert _decode(lib, _cache(), N=30) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), max_seq_len=4097) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), max_seq_len=0) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), out_dtype=9) == E.KVC_ERR_UNSUPPORTED
    assert _decode(lib, _cache(), q=FAKE + 2) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), B=0, max_seq_len=4097) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), q=None) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), seq_lens=None) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(stride_tok=100)) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(k=FAKE + 8)) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), scale=float("nan")) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), nwg=-1) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(), B=5000) == E.KVC_ERR_UNSUPPORTED
    assert _decode(lib, _cache(), ws=None) == E.KVC_ERR_WORKSPACE
    assert _decode(lib, _cache(), ws_bytes=16) == E.KVC_ERR_WORKSPACE
    # B == 0 is a successful no-op (nothing launched; empty buffers may be null)
    assert _decode(lib, _cache(), B=0) == E.KVC_OK
    assert _decode(lib, _cache(), B=0, q=None, seq_lens=None) == E.KVC_OK


def test_paged_descriptor_errors(lib):
    E = _lib
    paged = dict(block_table=FAKE * 3, block_size=16, max_blocks_per_seq=8192, num_blocks=100,
                 stride_seq=8 * 16 * 128, stride_head=16 * 128)
    assert _decode(lib, _cache(**paged), B=0, max_seq_len=131072) == E.KVC_OK
    assert _decode(lib, _cache(**{**paged, "block_size": 12}), B=0) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(**{**paged, "num_blocks": 0}), B=0) == E.KVC_ERR_INVALID
    assert _decode(lib, _cache(**paged), B=0, max_seq_len=131073) == E.KVC_ERR_INVALID


def test_verify_and_append_host_errors(lib):
    E = _lib
    c = _cache()
    v = lambda T, **kw: lib.kvc_attn_verify(ctypes.byref(c), FAKE, FAKE, E.KVC_F32, None, 8, T,
                                            kw.get("N", 64), 8, 128, FAKE, kw.get("L", 4096), 0.1, 0,
                                            FAKE, 1 << 30, None)
    assert v(0) == E.KVC_ERR_INVALID
    assert v(2049) == E.KVC_ERR_INVALID  # T > KVC_MAX_T
    assert v(5, L=4) == E.KVC_ERR_INVALID  # max_seq_len < T
    ap = lambda **kw: lib.kvc_append(ctypes.byref(kw.get("c", c)), kw.get("kn", FAKE), FAKE,
                                     kw.get("B", 8), kw.get("T", 1), 8, kw.get("H", 128), FAKE, None)
    assert ap(T=0) == E.KVC_ERR_INVALID
    assert ap(B=-1) == E.KVC_ERR_INVALID
    assert ap(kn=None) == E.KVC_ERR_INVALID
    assert ap(kn=FAKE + 4) == E.KVC_ERR_INVALID
    assert ap(H=80) == E.KVC_ERR_UNSUPPORTED
    assert ap(B=0) == E.KVC_OK
    g = lambda cc: lib.kvc_gather(ctypes.byref(cc), FAKE, FAKE, 0, 8, 128, FAKE, 16, None)
    assert g(c) == E.KVC_ERR_INVALID  # gather needs a paged cache


def test_append_attend_host_errors(lib):
    E = _lib
    c = _cache()

    def aa(**kw):
        return lib.kvc_append_attend(ctypes.byref(kw.get("c", c)), kw.get("kn", FAKE),
                                     kw.get("vn", FAKE), kw.get("q", FAKE), FAKE, E.KVC_F32, None,
                                     kw.get("B", 8), kw.get("T", 1), kw.get("N", 64), 8,
                                     kw.get("H", 128), FAKE, kw.get("L", 4096), 0.1, 0,
                                     kw.get("ws", FAKE), 1 << 30, None)

    # everything the two separate calls reject is rejected before any launch
    assert aa(kn=None) == E.KVC_ERR_INVALID
    assert aa(vn=None) == E.KVC_ERR_INVALID
    assert aa(kn=FAKE + 4) == E.KVC_ERR_INVALID
    assert aa(vn=FAKE + 8) == E.KVC_ERR_INVALID
    assert aa(T=0) == E.KVC_ERR_INVALID
    assert aa(T=2049) == E.KVC_ERR_INVALID
    assert aa(N=60) == E.KVC_ERR_INVALID
    assert aa(H=80) == E.KVC_ERR_UNSUPPORTED
    assert aa(L=4097) == E.KVC_ERR_INVALID
    assert aa(q=None) == E.KVC_ERR_INVALID
    assert aa(ws=None) == E.KVC_ERR_WORKSPACE
    assert aa(c=_cache(dtype=E.KVC_F32)) == E.KVC_ERR_UNSUPPORTED
    # an empty batch is a successful no-op, with or without buffers
    assert aa(B=0) == E.KVC_OK
    assert aa(B=0, kn=None, vn=None, q=None) == E.KVC_OK


def test_attn_options_layout_and_errors(lib):
    E = _lib
    assert ctypes.sizeof(_lib.KvcAttnOptions) == 32  # 3 pointers, 2 int32
    c = _cache()

    def at(window=0, reserved=0, tree=None, opts=True, **kw):
        o = _lib.KvcAttnOptions()
        o.window = window
        o.reserved = reserved
        o.tree_mask = tree
        return lib.kvc_attn(ctypes.byref(c), ctypes.byref(o) if opts else None, FAKE, FAKE,
                            E.KVC_F32, None, kw.get("B", 8), kw.get("T", 5), 64, 8, 128, FAKE,
                            4096, 0.1, 0, kw.get("ws", FAKE), 1 << 30, None)

    assert at(window=-1) == E.KVC_ERR_INVALID
    assert at(reserved=3) == E.KVC_ERR_INVALID
    assert at(tree=FAKE + 2) == E.KVC_ERR_INVALID
    assert at(T=2049) == E.KVC_ERR_INVALID
    assert at(T=257, tree=FAKE) == E.KVC_ERR_INVALID  # mask rows up to KVC_MAX_TREE_T tokens
    assert at(B=0, T=256, tree=FAKE) == E.KVC_OK
    assert at(ws=None) == E.KVC_ERR_WORKSPACE
    assert at(B=0) == E.KVC_OK
    assert at(B=0, opts=False) == E.KVC_OK
    assert at(B=0, window=7, tree=FAKE) == E.KVC_OK


def test_noalloc_host_errors(lib):
    """kvc_attn_noalloc checks what kvc_attn checks, and rejects a call whose
    scratch need exceeds its static array before touching the device."""
    E = _lib
    import re

    hdr = open(HEADER).read()
    m = re.search(r"#define KVC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.KVC_NOALLOC_SCRATCH_BYTES
    c = _cache(capacity=8192, stride_seq=8 * 8192 * 128, stride_head=8192 * 128)

    def na(B=8, T=5, N=64, L=4096, window=0, tree=None, nwg=0, q=FAKE):
        o = _lib.KvcAttnOptions()
        o.window = window
        o.tree_mask = tree
        return lib.kvc_attn_noalloc(ctypes.byref(c), ctypes.byref(o), q, FAKE, E.KVC_F32, None, B,
                                    T, N, 8, 128, FAKE, L, 0.1, nwg, None)

    assert na(T=0) == E.KVC_ERR_INVALID
    assert na(N=60) == E.KVC_ERR_INVALID
    assert na(window=-1) == E.KVC_ERR_INVALID
    assert na(tree=FAKE + 2) == E.KVC_ERR_INVALID
    assert na(q=None) == E.KVC_ERR_INVALID
    assert na(L=8193) == E.KVC_ERR_INVALID
    # a 512-token chunk of prefill for 8 sequences needs more than the array
    need = lib.kvc_workspace_bytes(8, 512, 32, 8, 128, 4608, 0)
    assert need > _lib.KVC_NOALLOC_SCRATCH_BYTES
    assert na(T=512, N=32, L=4608) == E.KVC_ERR_WORKSPACE
    # the decode and verify workloads fit
    assert lib.kvc_workspace_bytes(64, 1, 32, 8, 128, 4097, 0) <= _lib.KVC_NOALLOC_SCRATCH_BYTES
    assert lib.kvc_workspace_bytes(32, 5, 64, 8, 128, 8197, 0) <= _lib.KVC_NOALLOC_SCRATCH_BYTES
    assert lib.kvc_workspace_bytes(32, 8, 64, 8, 128, 8200, 0) <= _lib.KVC_NOALLOC_SCRATCH_BYTES
    assert na(B=0) == E.KVC_OK


def test_plan_kernel_names_the_kernel_by_rows(lib):
    """Vector ALUs up to 4 query rows per (b, k) at H = 128 (8 at H = 64),
    matrix cores up to 64 rows, units of 128 rows beyond."""
    k = lambda *a: (lib.kvc_plan_kernel(*a) or b"").decode()
    assert k(64, 1, 32, 8, 128, 4097, 0) == "attn_valu_kernel"   # G = 4
    assert k(8, 1, 64, 8, 128, 4097, 0) == "attn_mfma_kernel"    # G = 8
    assert k(8, 1, 16, 2, 64, 4097, 0) == "attn_valu_kernel"     # G = 8 at H = 64
    assert k(32, 5, 64, 8, 128, 8197, 0) == "attn_mfma_kernel"   # 40 rows
    assert k(32, 8, 64, 8, 128, 8200, 0) == "attn_mfma_kernel"   # 64 rows
    assert k(8, 9, 64, 8, 128, 8200, 0) == "attn_wide_kernel"    # 72 rows
    assert k(8, 512, 32, 8, 128, 4608, 0) == "attn_wide_kernel"
    assert lib.kvc_plan_kernel(8, 1, 30, 8, 128, 4097, 0) is None  # N % K
