"""The C ABI without a GPU: the library loads, exports what include/fa.h
declares, and rejects invalid arguments on the host before any launch.

Only calls that must fail validation are made here (fake, never-dereferenced
device addresses); nothing computes.
"""
import ctypes
import os
import re

import pytest

from transformer_attention_fa_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

INVALID, UNSUPPORTED = api.FA_ERR_INVALID_ARGUMENT, api.FA_ERR_UNSUPPORTED
P = 0x10000          # fake 16-byte-aligned device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        from transformer_attention_fa_amd import build
        build.build()
    return api.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(api.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert lib.fa_status_string(0) == b"FA_OK"
    assert lib.fa_status_string(1) == b"FA_ERR_INVALID_ARGUMENT"
    assert lib.fa_status_string(2) == b"FA_ERR_UNSUPPORTED"
    assert lib.fa_status_string(3) == b"FA_ERR_HIP"
    assert lib.fa_status_string(99) == b"FA_ERR_UNKNOWN"


def test_workspace_bytes(lib):
    B, H, d, S = 32, 32, 128, 16
    o_bytes = B * H * S * d * 4
    o_bytes = (o_bytes + 255) // 256 * 256
    assert lib.fa_decode_workspace_bytes(B, H, d, S) == o_bytes + B * H * S * 4
    assert lib.fa_decode_workspace_bytes(3, 5, 64, 7) == (3 * 5 * 7 * 64 * 4 + 255) // 256 * 256 + 3 * 5 * 7 * 4
    for bad in [(0, 1, 64, 1), (1, 0, 64, 1), (1, 1, 0, 1), (1, 1, 64, 0), (1, 1, 64, 257)]:
        assert lib.fa_decode_workspace_bytes(*bad) == 0


GOOD_FWD = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=8, H_kv=2, N_q=64, N_k=64, d=128, scale=0.088, causal=1)

FWD_CASES = [
    ("null_q", dict(q=None), INVALID),
    ("null_o", dict(o=None), INVALID),
    ("B_zero", dict(B=0), INVALID),
    ("H_negative", dict(H=-1), INVALID),
    ("N_q_zero", dict(N_q=0), INVALID),
    ("N_k_zero", dict(N_k=0), INVALID),
    ("H_not_multiple_of_H_kv", dict(H=6, H_kv=4), INVALID),
    ("d_zero", dict(d=0), INVALID),
    ("d_96_unsupported", dict(d=96), UNSUPPORTED),
    ("d_256_unsupported", dict(d=256), UNSUPPORTED),
    ("scale_nan", dict(scale=float("nan")), INVALID),
    ("scale_inf", dict(scale=float("inf")), INVALID),
    ("scale_negative", dict(scale=-0.5), UNSUPPORTED),
    ("q_misaligned", dict(q=P + 8), INVALID),
    ("v_misaligned", dict(v=P + 2), INVALID),
    ("lse_misaligned", dict(lse=P + 2), INVALID),
    ("too_large", dict(B=1 << 20, H=1 << 10, N_q=1 << 12, N_k=1 << 12), UNSUPPORTED),
    # B*H is exactly at the 2^40 cap and N_q is huge: the size check must not
    # form the 2^70 product (signed overflow) on its way to rejecting it
    ("too_large_no_overflow", dict(B=1 << 20, H=1 << 20, H_kv=1 << 20, N_q=1 << 30, N_k=1), UNSUPPORTED),
]


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32", "fa_fwd_window"])
@pytest.mark.parametrize("name,change,expect", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_rejects_before_launch(lib, fn, name, change, expect):
    a = dict(GOOD_FWD, **change)
    st = getattr(lib, fn)(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"], a["N_q"],
                          a["N_k"], a["d"], a["scale"], a["causal"], None)
    assert st == expect, (name, st, lib.fa_last_error())
    assert lib.fa_last_error()


GOOD_DEC = dict(q=P, k=P, v=P, lens=P, o=P, lse=P, B=4, H=8, H_kv=2, N_max=100, d=128, scale=0.1, S=16,
                ws=P, ws_bytes=1 << 20)

DEC_CASES = [
    ("null_seq_lens", dict(lens=None), INVALID),
    ("seq_lens_misaligned", dict(lens=P + 2), INVALID),
    ("splits_zero", dict(S=0), INVALID),
    ("splits_257", dict(S=257), INVALID),
    ("workspace_null", dict(ws=None), INVALID),
    ("workspace_misaligned", dict(ws=P + 4), INVALID),
    ("workspace_small", dict(ws_bytes=1000), INVALID),
    ("N_max_zero", dict(N_max=0), INVALID),
    ("H_not_multiple", dict(H=8, H_kv=3), INVALID),
    ("d_unsupported", dict(d=80), UNSUPPORTED),
    ("null_k_cache", dict(k=None), INVALID),
]


@pytest.mark.parametrize("name,change,expect", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_rejects_before_launch(lib, name, change, expect):
    a = dict(GOOD_DEC, **change)
    st = lib.fa_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                       a["N_max"], a["d"], a["scale"], a["S"], a["ws"], a["ws_bytes"], None)
    assert st == expect, (name, st, lib.fa_last_error())
    assert lib.fa_last_error()
    st = lib.fa_decode_window(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                              a["N_max"], a["d"], a["scale"], 64, a["S"], a["ws"], a["ws_bytes"], None)
    assert st == expect, (name, st, lib.fa_last_error())


@pytest.mark.parametrize("window", [0, -1, -(1 << 30)])
def test_window_must_be_positive(lib, window):
    a = GOOD_FWD
    st = lib.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"], a["N_q"],
                           a["N_k"], a["d"], a["scale"], window, None)
    assert st == INVALID and b"window" in lib.fa_last_error()
    d = GOOD_DEC
    st = lib.fa_decode_window(d["q"], d["k"], d["v"], d["lens"], d["o"], d["lse"], d["B"], d["H"], d["H_kv"],
                              d["N_max"], d["d"], d["scale"], window, d["S"], d["ws"], d["ws_bytes"], None)
    assert st == INVALID and b"window" in lib.fa_last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "missing" / "libfa.so"))
    with pytest.raises(FileNotFoundError):
        api.load()


GOOD_PAGED = dict(q=P, kp=P, vp=P, bt=P, max_blocks=8, lens=P, o=P, lse=P, B=4, H=8, H_kv=2, num_pages=64,
                  page_size=32, d=128, scale=0.1, S=16, ws=P, ws_bytes=1 << 20)

PAGED_CASES = [
    ("null_block_table", dict(bt=None), INVALID),
    ("block_table_misaligned", dict(bt=P + 2), INVALID),
    ("max_blocks_zero", dict(max_blocks=0), INVALID),
    ("num_pages_zero", dict(num_pages=0), INVALID),
    ("page_size_zero", dict(page_size=0), INVALID),
    ("page_size_24", dict(page_size=24), UNSUPPORTED),
    ("null_seq_lens", dict(lens=None), INVALID),
    ("splits_zero", dict(S=0), INVALID),
    ("workspace_small", dict(ws_bytes=1000), INVALID),
    ("H_not_multiple", dict(H=8, H_kv=3), INVALID),
    ("d_unsupported", dict(d=80), UNSUPPORTED),
    ("null_pool", dict(kp=None), INVALID),
]


@pytest.mark.parametrize("name,change,expect", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_decode_paged_rejects_before_launch(lib, name, change, expect):
    a = dict(GOOD_PAGED, **change)
    st = lib.fa_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["max_blocks"], a["lens"], a["o"], a["lse"],
                             a["B"], a["H"], a["H_kv"], a["num_pages"], a["page_size"], a["d"], a["scale"], a["S"],
                             a["ws"], a["ws_bytes"], None)
    assert st == expect, (name, st, lib.fa_last_error())
    assert lib.fa_last_error()



@pytest.mark.parametrize("k_scale,v_scale", [(0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))])
def test_decode_fp8_rejects_bad_scales(lib, k_scale, v_scale):
    a = GOOD_DEC
    st = lib.fa_decode_fp8(a["q"], a["k"], a["v"], k_scale, v_scale, a["lens"], a["o"], a["lse"], a["B"], a["H"],
                           a["H_kv"], a["N_max"], a["d"], a["scale"], a["S"], a["ws"], a["ws_bytes"], None)
    assert st == INVALID and b"scale" in lib.fa_last_error()


@pytest.mark.parametrize("name,change,expect", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_fp8_rejects_before_launch(lib, name, change, expect):
    a = dict(GOOD_DEC, **change)
    st = lib.fa_decode_fp8(a["q"], a["k"], a["v"], 0.5, 0.5, a["lens"], a["o"], a["lse"], a["B"], a["H"],
                           a["H_kv"], a["N_max"], a["d"], a["scale"], a["S"], a["ws"], a["ws_bytes"], None)
    assert st == expect, (name, st, lib.fa_last_error())


@pytest.mark.parametrize("n", [-1, -100])
def test_fwd_max_workgroups_rejects_negative(lib, n):
    assert lib.fa_fwd_set_max_workgroups(n) == INVALID
    assert b"n must be >= 0" in lib.fa_last_error()


def test_fwd_max_workgroups_accepts_caps(lib):
    for n in (5, 1, 0):          # ends at 0: no cap for the rest of the session
        assert lib.fa_fwd_set_max_workgroups(n) == api.FA_OK
