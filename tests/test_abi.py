"""The C ABI of libfocus on the CPU: it loads, exports every declared
symbol, and rejects bad host arguments before any device work.

No call here reaches a kernel launch: each one fails validation first (or
is a size query / an empty retained call), so no GPU is needed.
"""
import ctypes
import os
import re
import threading

import pytest

import attention_delta_token_focus_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "focus.h")

# A fake, 16-byte aligned, never dereferenced device address.
FAKE = 0x10000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(focus_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 16, names
    for name in names:
        assert hasattr(F.lib, name), name
        assert callable(getattr(F, name)), name


def test_version_and_status_strings():
    assert "gfx950" in F.focus_version()
    for code, name in [(0, "FOCUS_OK"), (1, "FOCUS_ERR_INVALID_ARG"),
                       (2, "FOCUS_ERR_UNSUPPORTED"),
                       (3, "FOCUS_ERR_WORKSPACE"), (4, "FOCUS_ERR_HIP")]:
        assert F.focus_status_string(code) == name


def _attn(**kw):
    a = dict(dt=1, batch=2, B=32, Hq=32, Hkv=8, d=128, scale=0.0, q=FAKE,
             k_blk=FAKE, v_blk=FAKE, k_cache=FAKE, v_cache=FAKE,
             cu_prefix=FAKE, order=None, max_prefix=16, out=FAKE, imp=FAKE,
             lse=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return F.lib.focus_block_attn_importance(
        a["dt"], a["batch"], a["B"], a["Hq"], a["Hkv"], a["d"], a["scale"],
        a["q"], a["k_blk"], a["v_blk"], a["k_cache"], a["v_cache"],
        a["cu_prefix"], a["order"], a["max_prefix"], a["out"], a["imp"],
        a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(B=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(B=129), F.FOCUS_ERR_INVALID_ARG),
    (dict(Hkv=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(max_prefix=-1), F.FOCUS_ERR_INVALID_ARG),
    (dict(Hq=30), F.FOCUS_ERR_UNSUPPORTED),
    (dict(d=96), F.FOCUS_ERR_UNSUPPORTED),
    (dict(dt=7), F.FOCUS_ERR_UNSUPPORTED),
    (dict(q=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(imp=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(out=None, k_blk=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(v_blk=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(v_cache=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(out=None, k_cache=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(out=FAKE + 2), F.FOCUS_ERR_INVALID_ARG),
    (dict(Hq=8192, Hkv=8), F.FOCUS_ERR_INVALID_ARG),
    (dict(cu_prefix=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(k_cache=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(q=FAKE + 4), F.FOCUS_ERR_INVALID_ARG),
    (dict(lse=FAKE + 8), F.FOCUS_ERR_INVALID_ARG),
    (dict(order=FAKE + 4), F.FOCUS_ERR_INVALID_ARG),
    (dict(ws=None, ws_bytes=0), F.FOCUS_ERR_WORKSPACE),
])
def test_block_attention_rejects_bad_arguments(kw, code):
    assert _attn(**kw) == code
    assert F.focus_last_error().startswith("focus_block_attn_importance")


def _paged(**kw):
    a = dict(dt=1, batch=2, B=32, Hq=32, Hkv=8, d=128, scale=0.0, q=FAKE,
             k_blk=FAKE, v_blk=FAKE, k_pages=FAKE, v_pages=FAKE, table=FAKE,
             page_size=64, pps=4, cu_prefix=FAKE, order=None, max_prefix=256,
             out=FAKE, imp=FAKE, lse=None, ws=None, ws_bytes=0)
    a.update(kw)
    return F.lib.focus_block_attn_importance_paged(
        a["dt"], a["batch"], a["B"], a["Hq"], a["Hkv"], a["d"], a["scale"],
        a["q"], a["k_blk"], a["v_blk"], a["k_pages"], a["v_pages"], a["table"],
        a["page_size"], a["pps"], a["cu_prefix"], a["order"], a["max_prefix"],
        a["out"], a["imp"], a["lse"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=0), F.FOCUS_ERR_UNSUPPORTED),
    (dict(page_size=48), F.FOCUS_ERR_UNSUPPORTED),
    (dict(page_size=16), F.FOCUS_ERR_UNSUPPORTED),
    (dict(pps=3), F.FOCUS_ERR_INVALID_ARG),
    (dict(pps=-1), F.FOCUS_ERR_INVALID_ARG),
    (dict(table=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(table=FAKE + 4), F.FOCUS_ERR_INVALID_ARG),
    (dict(k_pages=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(batch=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(d=96), F.FOCUS_ERR_UNSUPPORTED),
    (dict(ws=None, ws_bytes=0), F.FOCUS_ERR_WORKSPACE),
])
def test_paged_block_attention_rejects_bad_arguments(kw, code):
    assert _paged(**kw) == code
    assert F.focus_last_error().startswith("focus_block_attn_importance_paged")


def _noalloc(**kw):
    a = dict(dt=1, batch=2, B=32, Hq=32, Hkv=8, d=128, scale=0.0, q=FAKE,
             k_blk=FAKE, v_blk=FAKE, k_cache=FAKE, v_cache=FAKE,
             cu_prefix=FAKE, max_prefix=16, out=FAKE, imp=FAKE, lse=None,
             stream=None)
    a.update(kw)
    return F.lib.focus_block_attn_importance_noalloc(
        a["dt"], a["batch"], a["B"], a["Hq"], a["Hkv"], a["d"], a["scale"],
        a["q"], a["k_blk"], a["v_blk"], a["k_cache"], a["v_cache"],
        a["cu_prefix"], a["max_prefix"], a["out"], a["imp"], a["lse"],
        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(B=129), F.FOCUS_ERR_INVALID_ARG),
    (dict(Hq=30), F.FOCUS_ERR_UNSUPPORTED),
    (dict(q=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(imp=FAKE + 4), F.FOCUS_ERR_INVALID_ARG),
    (dict(v_cache=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(batch=65537), F.FOCUS_ERR_WORKSPACE),
])
def test_noalloc_block_attention_rejects_bad_arguments(kw, code):
    """Argument errors, and a batch beyond the static scratch, are reported
    before any device call."""
    assert _noalloc(**kw) == code
    assert F.focus_last_error()


def test_paged_retained_attention_checks_pages():
    args = [1, 2, 32, 32, 8, 128, 0.0, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 5,
            FAKE, FAKE, FAKE, 64, 1, FAKE, None, 256, FAKE, None, 0, None]
    assert F.lib.focus_retained_attn_paged(*args) == F.FOCUS_ERR_INVALID_ARG
    assert "pages_per_seq" in F.focus_last_error()
    args[17] = 40
    assert F.lib.focus_retained_attn_paged(*args) == F.FOCUS_ERR_UNSUPPORTED


def _topk(**kw):
    a = dict(batch=2, B=32, Hq=32, pool_k=3, imp0=FAKE, imp1=FAKE,
             k_keep=FAKE, keep=FAKE, dI=None, stream=None)
    a.update(kw)
    return F.lib.focus_delta_topk(a["batch"], a["B"], a["Hq"], a["pool_k"],
                                  a["imp0"], a["imp1"], a["k_keep"],
                                  a["keep"], a["dI"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(B=200), F.FOCUS_ERR_INVALID_ARG),
    (dict(Hq=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(pool_k=4), F.FOCUS_ERR_UNSUPPORTED),
    (dict(pool_k=0), F.FOCUS_ERR_UNSUPPORTED),
    (dict(pool_k=257), F.FOCUS_ERR_UNSUPPORTED),
    (dict(imp1=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(k_keep=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(keep=None), F.FOCUS_ERR_INVALID_ARG),
])
def test_delta_topk_rejects_bad_arguments(kw, code):
    assert _topk(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((0, 32, FAKE, FAKE, FAKE, None), F.FOCUS_ERR_INVALID_ARG),
    ((2, 0, FAKE, FAKE, FAKE, None), F.FOCUS_ERR_INVALID_ARG),
    ((2, 32, None, FAKE, FAKE, None), F.FOCUS_ERR_INVALID_ARG),
    ((2, 32, FAKE, None, FAKE, None), F.FOCUS_ERR_INVALID_ARG),
    ((2, 32, FAKE, FAKE, None, None), F.FOCUS_ERR_INVALID_ARG),
])
def test_compact_rejects_bad_arguments(args, code):
    assert F.lib.focus_compact(*args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(B=129), F.FOCUS_ERR_INVALID_ARG),
    (dict(pool_k=2), F.FOCUS_ERR_UNSUPPORTED),
    (dict(idx=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(cu_ret=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(imp0=FAKE + 2), F.FOCUS_ERR_INVALID_ARG),
])
def test_select_rejects_bad_arguments(kw, code):
    a = dict(batch=2, B=32, Hq=32, pool_k=3, imp0=FAKE, imp1=FAKE,
             k_keep=FAKE, keep=FAKE, dI=None, idx=FAKE, cu_ret=FAKE)
    a.update(kw)
    assert F.lib.focus_select(a["batch"], a["B"], a["Hq"], a["pool_k"],
                              a["imp0"], a["imp1"], a["k_keep"], a["keep"],
                              a["dI"], a["idx"], a["cu_ret"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(B=129), F.FOCUS_ERR_INVALID_ARG),
    (dict(pool_k=2), F.FOCUS_ERR_UNSUPPORTED),
    (dict(rules=4), F.FOCUS_ERR_UNSUPPORTED),
    (dict(rules=-1), F.FOCUS_ERR_UNSUPPORTED),
    (dict(keep=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(k_keep=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(idx=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(cu_ret=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(imp1=FAKE + 4), F.FOCUS_ERR_INVALID_ARG),
])
def test_select_masked_rejects_bad_arguments(kw, code):
    a = dict(batch=2, B=32, Hq=32, pool_k=3, imp0=FAKE, imp1=FAKE, masked=FAKE,
             k_keep=FAKE, rules=3, keep=FAKE, cand=None, dI=None, idx=FAKE,
             cu_ret=FAKE)
    a.update(kw)
    assert F.lib.focus_select_masked(
        a["batch"], a["B"], a["Hq"], a["pool_k"], a["imp0"], a["imp1"],
        a["masked"], a["k_keep"], a["rules"], a["keep"], a["cand"], a["dI"],
        a["idx"], a["cu_ret"], None) == code
    assert F.focus_last_error().startswith("focus_select_masked")


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(B=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(pool_k=4), F.FOCUS_ERR_UNSUPPORTED),
    (dict(rules=8), F.FOCUS_ERR_UNSUPPORTED),
    (dict(alpha=0.0), F.FOCUS_ERR_INVALID_ARG),
    (dict(alpha=-1.0), F.FOCUS_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), F.FOCUS_ERR_INVALID_ARG),
    (dict(yield_hist=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(keep=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(idx=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(imp0=None), F.FOCUS_ERR_INVALID_ARG),
])
def test_select_dynamic_rejects_bad_arguments(kw, code):
    a = dict(batch=2, B=32, Hq=32, pool_k=3, imp0=FAKE, imp1=FAKE, masked=None,
             yield_hist=FAKE, alpha=1.5, rules=3, k_used=None, keep=FAKE,
             cand=None, dI=None, idx=FAKE, cu_ret=FAKE)
    a.update(kw)
    assert F.lib.focus_select_dynamic(
        a["batch"], a["B"], a["Hq"], a["pool_k"], a["imp0"], a["imp1"],
        a["masked"], a["yield_hist"], a["alpha"], a["rules"], a["k_used"],
        a["keep"], a["cand"], a["dI"], a["idx"], a["cu_ret"], None) == code
    assert F.focus_last_error().startswith("focus_select_dynamic")


def _ret(**kw):
    a = dict(dt=1, batch=2, B=32, Hq=32, Hkv=8, d=128, scale=0.0, q=FAKE,
             k=FAKE, v=FAKE, idx=FAKE, cu_ret=FAKE, n_ret=10, max_ret=5,
             k_cache=FAKE, v_cache=FAKE, cu_prefix=FAKE, order=None,
             max_prefix=16, out=FAKE, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return F.lib.focus_retained_attn(
        a["dt"], a["batch"], a["B"], a["Hq"], a["Hkv"], a["d"], a["scale"],
        a["q"], a["k"], a["v"], a["idx"], a["cu_ret"], a["n_ret"],
        a["max_ret"], a["k_cache"], a["v_cache"], a["cu_prefix"], a["order"],
        a["max_prefix"], a["out"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(n_ret=-1), F.FOCUS_ERR_INVALID_ARG),
    (dict(max_ret=33), F.FOCUS_ERR_INVALID_ARG),
    (dict(max_ret=0), F.FOCUS_ERR_INVALID_ARG),
    (dict(idx=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(out=None), F.FOCUS_ERR_INVALID_ARG),
    (dict(d=80), F.FOCUS_ERR_UNSUPPORTED),
    (dict(Hkv=5), F.FOCUS_ERR_UNSUPPORTED),
    (dict(n_ret=0, max_ret=0, idx=None, cu_ret=None, out=None), F.FOCUS_OK),
])
def test_retained_attention_arguments(kw, code):
    assert _ret(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((0, FAKE, FAKE, None), F.FOCUS_ERR_INVALID_ARG),
    ((4, None, FAKE, None), F.FOCUS_ERR_INVALID_ARG),
    ((4, FAKE, None, None), F.FOCUS_ERR_INVALID_ARG),
])
def test_schedule_rejects_bad_arguments(args, code):
    assert F.lib.focus_schedule(*args) == code


def test_workspace_queries():
    n = ctypes.c_size_t(123)
    assert F.lib.focus_block_attn_importance_workspace(
        256, 32, 32, 8, 128, 4096, ctypes.byref(n)) == F.FOCUS_OK
    assert F.focus_block_attn_importance_workspace(256, 32, 32, 8, 128,
                                                   4096) >= 0
    assert F.focus_retained_attn_workspace(128, 32, 8, 128, 8192, 1152,
                                           9) >= 0
    assert F.lib.focus_block_attn_importance_workspace(
        256, 32, 32, 8, 128, 4096, None) == F.FOCUS_ERR_INVALID_ARG
    with pytest.raises(F.FocusError) as ei:
        F.focus_block_attn_importance_workspace(256, 32, 30, 8, 128, 10)
    assert ei.value.status == F.FOCUS_ERR_UNSUPPORTED


def test_last_error_is_thread_local():
    assert _attn(batch=0) == F.FOCUS_ERR_INVALID_ARG
    seen = []
    t = threading.Thread(target=lambda: seen.append(F.focus_last_error()))
    t.start()
    t.join()
    assert seen == [""]
    assert "batch" in F.focus_last_error()


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(16)
    with pytest.raises(ValueError):
        F.focus_compact(1, 16, x, x, x)
