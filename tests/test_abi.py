"""The C-ABI library: it loads, exports what include/miattn.h declares, and its host-side
validation and planning behave as documented (CPU only; no kernel is launched)."""
import ctypes
import os
import re

import pytest

import io_aware_exact_attention_amd as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miattn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
P = ctypes.c_void_p(4096)        # a non-null, 16-byte aligned dummy pointer (never dereferenced)
MIS = ctypes.c_void_p(4096 + 2)  # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mi.LIB_PATH):
        pytest.fail("libmiattn.so is not built; run __graft_entry__.build() first")
    return mi.load_library()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["attn_fwd_prefill", "attn_fwd_prefill_paged",
                                           "attn_fwd_prefill_f16", "attn_fwd_prefill_paged_f16",
                                           "attn_fwd_prefill_fp8", "attn_fwd_prefill_paged_fp8",
                                           "attn_fwd_prefill_varlen_fp8",
                                           "attn_fwd_decode", "attn_fwd_decode_f16",
                                           "attn_fwd_decode_fp8", "attn_bwd", "attn_bwd_f16",
                                           "attn_fwd_prefill_varlen",
                                           "attn_fwd_prefill_varlen_f16",
                                           "attn_bwd_workspace_bytes",
                                           "attn_decode_workspace_bytes",
                                           "attn_fwd_decode_noalloc",
                                           "attn_decode_num_splits", "attn_status_string"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert mi.attn_status_string(OK) == "ok"
    for s in (INVALID, UNSUPPORTED, WORKSPACE, HIPERR):
        assert mi.attn_status_string(s) not in ("ok", "unknown status")
    assert mi.attn_status_string(99) == "unknown status"


def prefill(lib, q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Nq=4, Nk=4, d=64, causal=1,
            scale=0.125):
    return lib.attn_fwd_prefill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal,
                                ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(q=MIS), INVALID), (dict(o=MIS), INVALID),
    (dict(lse=ctypes.c_void_p(4098)), INVALID),
    (dict(B=0), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID), (dict(Nq=0), INVALID),
    (dict(Nk=0), INVALID), (dict(Hq=3, Hkv=2), INVALID), (dict(Nq=5, Nk=4, causal=1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(B=65536, Hq=65536, Hkv=1, Nq=128, Nk=128), UNSUPPORTED),
    (dict(Nq=16, Nk=(1 << 23) + 1, d=128), UNSUPPORTED),
])
def test_prefill_validation(lib, kw, status):
    assert prefill(lib, **kw) == status


def prefill_paged(lib, q=P, kc=P, vc=P, table=P, kv_lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2,
                  Nq=16, d=128, max_kv=100, page_size=16, max_blocks=7, num_pages=10, causal=1,
                  scale=0.1):
    return lib.attn_fwd_prefill_paged(q, kc, vc, table, kv_lens, o, lse, B, Hq, Hkv, Nq, d, max_kv,
                                      page_size, max_blocks, num_pages, causal,
                                      ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(vc=None), INVALID),
    (dict(table=None), INVALID), (dict(kv_lens=None), INVALID), (dict(o=None), INVALID),
    (dict(q=MIS), INVALID), (dict(kv_lens=ctypes.c_void_p(4098)), INVALID),
    (dict(lse=ctypes.c_void_p(4098)), INVALID), (dict(B=0), INVALID), (dict(Nq=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(max_kv=0), INVALID), (dict(Nq=101), INVALID),
    (dict(num_pages=0), INVALID), (dict(max_blocks=6), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(page_size=32), UNSUPPORTED),
    (dict(B=65536, Hq=65536, Hkv=1), UNSUPPORTED),
])
def test_prefill_paged_validation(lib, kw, status):
    assert prefill_paged(lib, **kw) == status


def decode(lib, q=P, kc=P, vc=P, table=None, seqlens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, d=128,
           max_seqlen=100, page_size=16, max_blocks=7, num_pages=10, scale=0.1, splits=1,
           ws=None, ws_bytes=0):
    return lib.attn_fwd_decode(q, kc, vc, table, seqlens, o, lse, B, Hq, Hkv, d, max_seqlen,
                               page_size, max_blocks, num_pages, ctypes.c_float(scale), splits,
                               ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kc=None), INVALID), (dict(vc=None), INVALID),
    (dict(seqlens=None), INVALID), (dict(o=None), INVALID), (dict(kc=MIS), INVALID),
    (dict(seqlens=ctypes.c_void_p(4098)), INVALID), (dict(B=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(max_seqlen=0), INVALID), (dict(splits=-1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(table=P, page_size=32), UNSUPPORTED), (dict(table=P, max_blocks=6), INVALID),
    (dict(table=P, num_pages=0), INVALID), (dict(B=70000), UNSUPPORTED),
    # more than one chunk needs a workspace of the advertised size
    (dict(max_seqlen=4096, splits=4), WORKSPACE),
    (dict(max_seqlen=4096, splits=4, ws=P, ws_bytes=100), WORKSPACE),
])
def test_decode_validation(lib, kw, status):
    assert decode(lib, **kw) == status


def decode_fp8(lib, k_scale=0.02, v_scale=0.03, **kw):
    a = dict(q=P, kc=P, vc=P, table=None, seqlens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, d=128,
             max_seqlen=100, page_size=16, max_blocks=7, num_pages=10, scale=0.1, splits=1,
             ws=None, ws_bytes=0)
    a.update(kw)
    return lib.attn_fwd_decode_fp8(a["q"], a["kc"], a["vc"], a["table"], a["seqlens"], a["o"],
                                   a["lse"], a["B"], a["Hq"], a["Hkv"], a["d"], a["max_seqlen"],
                                   a["page_size"], a["max_blocks"], a["num_pages"],
                                   ctypes.c_float(a["scale"]), ctypes.c_float(k_scale),
                                   ctypes.c_float(v_scale), a["splits"], a["ws"], a["ws_bytes"],
                                   None)


@pytest.mark.parametrize("kw,status", [
    (dict(k_scale=0.0), INVALID), (dict(k_scale=-0.5), INVALID),
    (dict(v_scale=0.0), INVALID), (dict(v_scale=-1.0), INVALID),
    (dict(k_scale=float("nan")), INVALID), (dict(v_scale=float("inf")), INVALID),
    (dict(scale=1e30, k_scale=1e30), INVALID),          # |scale| * k_scale overflows
    # every check of attn_fwd_decode applies as well
    (dict(kc=None), INVALID), (dict(vc=MIS), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(table=P, page_size=8), UNSUPPORTED),
    (dict(table=P, max_blocks=6), INVALID), (dict(max_seqlen=4096, splits=4), WORKSPACE),
])
def test_decode_fp8_validation(lib, kw, status):
    assert decode_fp8(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(B=0), INVALID), (dict(Hq=3, Hkv=2), INVALID),
    (dict(Nq=5, Nk=4, causal=1), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(d=96), UNSUPPORTED)])
def test_f16_entry_points_validate_like_bf16(lib, kw, status):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Nq=4, Nk=4, d=64, causal=1,
             scale=0.125)
    a.update(kw)
    assert lib.attn_fwd_prefill_f16(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                    a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"],
                                    ctypes.c_float(a["scale"]), None) == status
    assert prefill(lib, **kw) == status


def prefill_fp8(lib, q_scale=0.02, k_scale=0.03, v_scale=0.04, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Nq=4, Nk=4, d=64, causal=1,
             scale=0.125)
    a.update(kw)
    return lib.attn_fwd_prefill_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                    a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"],
                                    ctypes.c_float(a["scale"]), ctypes.c_float(q_scale),
                                    ctypes.c_float(k_scale), ctypes.c_float(v_scale), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_scale=0.0), INVALID), (dict(q_scale=-0.5), INVALID),
    (dict(k_scale=0.0), INVALID), (dict(v_scale=-1.0), INVALID),
    (dict(q_scale=float("nan")), INVALID), (dict(k_scale=float("inf")), INVALID),
    (dict(v_scale=float("inf")), INVALID),
    (dict(scale=1e20, q_scale=1e20, k_scale=1e10), INVALID),   # the product overflows
    # every check of attn_fwd_prefill applies as well
    (dict(q=None), INVALID), (dict(v=MIS), INVALID), (dict(B=0), INVALID),
    (dict(Hq=3, Hkv=2), INVALID), (dict(Nq=5, Nk=4, causal=1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(d=96), UNSUPPORTED),
    # one byte per element: one head's K may reach 2^31 - 1 bytes, not 2^31
    (dict(Nq=4, Nk=1 << 24, d=128), UNSUPPORTED),
])
def test_prefill_fp8_validation(lib, kw, status):
    assert prefill_fp8(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q_scale=0.0), INVALID), (dict(k_scale=-1.0), INVALID), (dict(v_scale=float("nan")), INVALID),
    (dict(scale=1e20, q_scale=1e20, k_scale=1e10), INVALID),
    (dict(table=None), INVALID), (dict(page_size=32), UNSUPPORTED), (dict(max_blocks=6), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(Nq=101), INVALID), (dict(kc=MIS), INVALID)])
def test_prefill_paged_fp8_validation(lib, kw, status):
    a = dict(q=P, kc=P, vc=P, table=P, kv_lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, Nq=16, d=128,
             max_kv=100, page_size=16, max_blocks=7, num_pages=10, causal=1, scale=0.1,
             q_scale=0.02, k_scale=0.03, v_scale=0.04)
    a.update(kw)
    args = [a[n] for n in ("q", "kc", "vc", "table", "kv_lens", "o", "lse", "B", "Hq", "Hkv",
                           "Nq", "d", "max_kv", "page_size", "max_blocks", "num_pages", "causal")]
    args += [ctypes.c_float(a[n]) for n in ("scale", "q_scale", "k_scale", "v_scale")] + [None]
    assert lib.attn_fwd_prefill_paged_fp8(*args) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q_scale=-1.0), INVALID), (dict(k_scale=float("inf")), INVALID), (dict(v_scale=0.0), INVALID),
    (dict(scale=1e20, q_scale=1e20, k_scale=1e10), INVALID),
    (dict(cu_q=None), INVALID), (dict(Hq=3, Hkv=2), INVALID), (dict(max_q=300), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(q=MIS), INVALID)])
def test_prefill_varlen_fp8_validation(lib, kw, status):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cu_q=P, cu_k=P, B=2, Hq=4, Hkv=2, total_q=200,
             total_k=250, max_q=150, max_k=200, d=128, causal=1, scale=0.1, q_scale=0.02,
             k_scale=0.03, v_scale=0.04)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "cu_q", "cu_k", "B", "Hq", "Hkv", "total_q",
                           "total_k", "max_q", "max_k", "d", "causal")]
    args += [ctypes.c_float(a[n]) for n in ("scale", "q_scale", "k_scale", "v_scale")] + [None]
    assert lib.attn_fwd_prefill_varlen_fp8(*args) == status


def test_f16_paged_and_decode_validate_like_bf16(lib):
    for kw, status in ((dict(table=None), INVALID), (dict(page_size=32), UNSUPPORTED),
                       (dict(max_blocks=6), INVALID), (dict(d=80), UNSUPPORTED)):
        a = dict(q=P, kc=P, vc=P, table=P, kv_lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, Nq=16,
                 d=128, max_kv=100, page_size=16, max_blocks=7, num_pages=10, causal=1, scale=0.1)
        a.update(kw)
        args = [a[n] for n in ("q", "kc", "vc", "table", "kv_lens", "o", "lse", "B", "Hq", "Hkv",
                               "Nq", "d", "max_kv", "page_size", "max_blocks", "num_pages",
                               "causal")] + [ctypes.c_float(a["scale"]), None]
        assert lib.attn_fwd_prefill_paged_f16(*args) == status
        assert lib.attn_fwd_prefill_paged(*args) == status
    for kw, status in ((dict(kc=None), INVALID), (dict(d=80), UNSUPPORTED),
                       (dict(max_seqlen=4096, splits=4), WORKSPACE)):
        a = dict(q=P, kc=P, vc=P, table=None, seqlens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, d=128,
                 max_seqlen=100, page_size=16, max_blocks=7, num_pages=10, scale=0.1, splits=1,
                 ws=None, ws_bytes=0)
        a.update(kw)
        args = [a[n] for n in ("q", "kc", "vc", "table", "seqlens", "o", "lse", "B", "Hq", "Hkv",
                               "d", "max_seqlen", "page_size", "max_blocks", "num_pages")]
        args += [ctypes.c_float(a["scale"]), a["splits"], a["ws"], a["ws_bytes"], None]
        assert lib.attn_fwd_decode_f16(*args) == status
        assert lib.attn_fwd_decode(*args) == status


def bwd(lib, ws_bytes=1 << 20, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, B=1, Hq=2, Hkv=1, Nq=4, Nk=4,
             d=64, causal=1, scale=0.125, ws=P)
    a.update(kw)
    args = [a[n] for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "B", "Hq", "Hkv",
                           "Nq", "Nk", "d", "causal")]
    args += [ctypes.c_float(a["scale"]), a["ws"], ws_bytes, None]
    st = lib.attn_bwd(*args)
    assert lib.attn_bwd_f16(*args) == st
    return st


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(dout=None), INVALID),
    (dict(dq=None), INVALID), (dict(dk=MIS), INVALID), (dict(lse=ctypes.c_void_p(4096 + 2)), INVALID),
    (dict(B=0), INVALID), (dict(Nk=0), INVALID), (dict(Hq=3, Hkv=2), INVALID),
    (dict(Nq=5, Nk=4, causal=1), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(Nq=16, Nk=(1 << 23) + 1, d=128), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
])
def test_backward_validation(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_backward_workspace_arithmetic(lib):
    assert mi.attn_bwd_workspace_bytes(2, 8, 100) == (2 * 8 * 100 * 8 + 255) // 256 * 256
    assert mi.attn_bwd_workspace_bytes(0, 8, 100) == 0


def varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cu_q=P, cu_k=P, B=2, Hq=4, Hkv=2, total_q=100,
             total_k=120, max_q=60, max_k=70, d=128, causal=1, scale=0.1)
    a.update(kw)
    return lib.attn_fwd_prefill_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu_q"],
                                       a["cu_k"], a["B"], a["Hq"], a["Hkv"], a["total_q"],
                                       a["total_k"], a["max_q"], a["max_k"], a["d"], a["causal"],
                                       ctypes.c_float(a["scale"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(cu_q=None), INVALID), (dict(cu_k=None), INVALID),
    (dict(k=MIS), INVALID), (dict(cu_k=ctypes.c_void_p(4098)), INVALID),
    (dict(lse=ctypes.c_void_p(4098)), INVALID), (dict(B=0), INVALID), (dict(total_q=0), INVALID),
    (dict(max_k=0), INVALID), (dict(Hq=3, Hkv=2), INVALID), (dict(max_q=101), INVALID),
    (dict(max_k=121), INVALID), (dict(scale=float("nan")), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(B=65536, Hq=65536, Hkv=1, total_q=1 << 20, max_q=1 << 20), UNSUPPORTED),
])
def test_varlen_validation(lib, kw, status):
    assert varlen(lib, **kw) == status


def test_decode_split_plan(lib):
    # explicit split counts: chunk = ceil(L / s) rounded up to 32 keys
    assert mi.attn_decode_num_splits(2, 8, 2, 128, 4096, 4) == 4
    assert mi.attn_decode_num_splits(2, 8, 2, 128, 100, 4) == 4      # chunk 32 -> 4 chunks
    assert mi.attn_decode_num_splits(2, 8, 2, 128, 100, 50) == 4     # never more than needed
    assert mi.attn_decode_num_splits(2, 8, 2, 128, 1, 0) == 1
    # automatic plan fills the machine but keeps >= 256 keys per chunk
    s = mi.attn_decode_num_splits(64, 32, 8, 128, 8192, 0)
    assert 1 <= s <= 32
    assert mi.attn_decode_num_splits(1, 1, 1, 128, 1000, 0) == 4
    assert mi.attn_decode_num_splits(0, 8, 2, 128, 100, 0) == 0      # invalid -> 0


def test_decode_workspace_arithmetic(lib):
    # the signature is (B, Hq, d, max_seqlen, num_splits), with no KV-head count
    assert list(lib.attn_decode_workspace_bytes.argtypes) == [ctypes.c_int] * 5
    assert mi.attn_decode_workspace_bytes(2, 8, 128, 100, 1) == 0
    n = 2 * 8 * 4
    want = (n * 128 * 4 + n * 4 + 255) // 256 * 256
    assert mi.attn_decode_workspace_bytes(2, 8, 128, 4096, 4) == want
    assert mi.attn_decode_workspace_bytes(0, 8, 128, 4096, 4) == 0     # invalid sizes
    assert mi.attn_decode_workspace_bytes(2, 8, 128, 4096, -1) == 0


@pytest.mark.parametrize("B,Hq,L", [(8, 32, 131072), (64, 32, 8192), (1, 1, 1000), (3, 12, 5000),
                                    (2, 64, 300)])
def test_decode_workspace_covers_every_kv_head_count(lib, B, Hq, L):
    # the automatic plan's need for every valid Hkv, the largest of them returned
    needs = []
    for hkv in [h for h in range(1, Hq + 1) if Hq % h == 0]:
        s = mi.attn_decode_num_splits(B, Hq, hkv, 128, L, 0)
        n = B * Hq * s
        needs.append(0 if s <= 1 else (n * 128 * 4 + n * 4 + 255) // 256 * 256)
    assert mi.attn_decode_workspace_bytes(B, Hq, 128, L, 0) == max(needs)


def test_binding_rejects_host_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mi.attn_fwd_prefill(x, x, x, x, None, True, 0.125)


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="the accepted call would launch a kernel on dummy pointers")
def test_prefill_grid_guard_counts_256_query_tiles(lib):
    # 2^20 heads: 2047 query tiles of 256 rows fit in 2^31 - 1 workgroups (validation
    # passes; without a device the launch then fails), 2048 do not
    H = 1 << 20
    assert prefill(lib, Hq=H, Hkv=H, Nq=2047 * 256, Nk=2047 * 256, d=64, causal=0) == HIPERR
    assert prefill(lib, Hq=H, Hkv=H, Nq=2047 * 256 + 1, Nk=2047 * 256 + 1, d=64,
                   causal=0) == UNSUPPORTED


def decode_noalloc(lib, q=P, kc=P, vc=P, table=None, seqlens=P, o=P, lse=None, B=2, Hq=8, Hkv=2,
                   d=128, max_seqlen=100, page_size=16, max_blocks=7, num_pages=10, scale=0.1,
                   splits=1):
    return lib.attn_fwd_decode_noalloc(q, kc, vc, table, seqlens, o, lse, B, Hq, Hkv, d,
                                       max_seqlen, page_size, max_blocks, num_pages,
                                       ctypes.c_float(scale), splits, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(seqlens=None), INVALID), (dict(kc=MIS), INVALID),
    (dict(B=0), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(splits=-1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(table=P, page_size=32), UNSUPPORTED),
    # partials beyond the static array: B*Hq*splits*(d+1)*4 > 32 MiB
    (dict(B=64, Hq=64, Hkv=8, max_seqlen=1 << 17, splits=128), WORKSPACE),
])
def test_decode_noalloc_validation(lib, kw, status):
    assert decode_noalloc(lib, **kw) == status


def test_decode_noalloc_limit_is_the_header_constant(lib):
    assert "#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)" in open(HEADER).read()
    assert mi.ATTN_DECODE_NOALLOC_MAX_BYTES == 32 << 20
    # the workloads' needs fit: paged (B=8, Hq=32, up to 128K keys) and contiguous
    # (B=64, Hq=32, 8K keys) decode at the automatic split count
    assert 0 < mi.attn_decode_workspace_bytes(8, 32, 128, 131072, 0) <= 32 << 20
    assert 0 < mi.attn_decode_workspace_bytes(64, 32, 128, 8192, 0) <= 32 << 20
