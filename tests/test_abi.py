"""Host-side checks of the C ABI (no GPU work is launched).

The library must load, export every function include/mattn.h declares, and
reject invalid arguments synchronously, before touching the device.  Pointer
arguments here are fake aligned addresses: every call either fails
validation or describes an empty problem, so nothing is ever dereferenced.
"""
import ctypes
import os
import re

import pytest

import flash_attention_transformers_amd as fa
from flash_attention_transformers_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mattn.h")
P = 0x10000  # fake, 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mattn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["mattn_fwd", "mattn_bwd", "mattn_bwd_stages", "mattn_bwd_workspace_size", "mattn_strerror",
         "mattn_version", "mattn_fwd_kvcache", "mattn_fwd_kvcache_workspace_size",
         "mattn_bwd_noalloc"])


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strerror():
    assert fa.mattn_version() >= 100
    assert fa.mattn_strerror(0) == "success"
    for s in (1, 2, 3, 4):
        assert fa.mattn_strerror(s) and fa.mattn_strerror(s) != "success"
    assert fa.mattn_strerror(99) == "unknown status"


def fwd_status(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, Sq=128, Skv=128, D=64, causal=0,
               scale=0.125, dtype=0):
    lib = fa.load_library()
    return lib.mattn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, dtype, None)


def bwd_status(ws=P, ws_bytes=1 << 40, B=1, Hq=2, Hkv=2, Sq=128, Skv=128, D=64, causal=0,
               scale=0.125, dtype=0, dq=P, q=P):
    lib = fa.load_library()
    return lib.mattn_bwd(q, P, P, P, P, P, dq, P, P, B, Hq, Hkv, Sq, Skv, D, causal, scale, dtype,
                         ws, ws_bytes, None)


INVALID = [
    dict(B=-1), dict(Sq=-3), dict(Hkv=0), dict(Hq=6, Hkv=4), dict(causal=2),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(dtype=7), dict(Skv=0),
    dict(q=0), dict(lse=0), dict(o=P + 8),
]


@pytest.mark.parametrize("kw", INVALID)
def test_fwd_rejects_invalid(kw):
    assert fwd_status(**kw) == fa.MATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=96), dict(D=256), dict(causal=1, Sq=129, Skv=128),
                                dict(B=1 << 12, Hq=1 << 8, Hkv=1 << 8, Sq=1 << 8, D=128)])
def test_fwd_rejects_unsupported(kw):
    assert fwd_status(**kw) == fa.MATTN_ERR_UNSUPPORTED


def test_empty_problem_is_a_noop():
    assert fwd_status(B=0) == fa.MATTN_OK
    assert fwd_status(Sq=0, q=0, o=0, lse=0, k=0, v=0, Skv=0) == fa.MATTN_OK


@pytest.mark.parametrize("kw", [dict(ws=0), dict(ws_bytes=16), dict(ws=P + 4), dict(dq=0),
                                dict(Hq=3, Hkv=2), dict(causal=-1)])
def test_bwd_rejects_invalid(kw):
    assert bwd_status(**kw) == fa.MATTN_ERR_INVALID_ARG


def test_bwd_rejects_unsupported():
    assert bwd_status(D=32) == fa.MATTN_ERR_UNSUPPORTED
    assert bwd_status(causal=1, Sq=300, Skv=200) == fa.MATTN_ERR_UNSUPPORTED


def test_workspace_size():
    ws = fa.mattn_bwd_workspace_size
    assert ws(0, 2, 2, 128, 128, 64) == 0
    assert ws(1, 3, 2, 128, 128, 64) == 0
    assert ws(1, 2, 2, 128, 128, 96) == 0
    # the per-row statistic only, rounded to 256 bytes
    assert ws(8, 12, 12, 1024, 1024, 64) == 8 * 12 * 1024 * 4
    assert ws(1, 1, 1, 3, 5, 64) == 256
    # short-KV cross attention adds fp32 partial dK/dV for split query chunks
    w = W.WORKLOADS["dit_cross_512"]
    n = ws(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D)
    dlt = w.B * w.Hq * w.Sq * 4
    part = n - ((dlt + 255) // 256 * 256)
    per_split = 2 * w.B * w.Hkv * 512 * w.D * 4
    assert part > 0 and part % per_split == 0
    assert ws(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D) == n  # deterministic


def test_python_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)


@pytest.mark.parametrize("stages", [0, 8, 0xFF])
def test_bwd_stages_rejects_bad_mask(stages):
    lib = fa.load_library()
    st = lib.mattn_bwd_stages(P, P, P, P, P, P, P, P, P, 1, 2, 2, 128, 128, 64, 0, 0.125, 0, P,
                              1 << 40, stages, None)
    assert st == fa.MATTN_ERR_INVALID_ARG


def test_bwd_stages_validates_like_bwd():
    lib = fa.load_library()
    st = lib.mattn_bwd_stages(P, P, P, P, P, P, P, P, P, 1, 3, 2, 128, 128, 64, 0, 0.125, 0, P,
                              1 << 40, fa.MATTN_BWD_ALL, None)
    assert st == fa.MATTN_ERR_INVALID_ARG
    st = lib.mattn_bwd_stages(P, P, P, P, P, P, P, P, P, 1, 2, 2, 128, 128, 96, 0, 0.125, 0, P,
                              1 << 40, fa.MATTN_BWD_DKDV, None)
    assert st == fa.MATTN_ERR_UNSUPPORTED


def kc_status(q=P, kc=P, vc=P, bt=P, sl=P, o=P, lse=P, B=1, Hq=8, Hkv=8, Sq=1, D=128, num_pages=100,
              page_size=64, pps=100, causal=1, scale=0.088, dtype=0, ws=P, ws_bytes=1 << 40):
    lib = fa.load_library()
    return lib.mattn_fwd_kvcache(q, kc, vc, bt, sl, o, lse, B, Hq, Hkv, Sq, D, num_pages, page_size,
                                 pps, causal, scale, dtype, ws, ws_bytes, None)


KC_INVALID = [
    dict(B=-1), dict(Sq=-1), dict(Hkv=0), dict(Hq=6, Hkv=4), dict(causal=2), dict(page_size=0),
    dict(pps=-1), dict(num_pages=-2), dict(scale=float("nan")), dict(dtype=5), dict(q=0),
    dict(o=P + 8), dict(kc=0), dict(vc=P + 4), dict(bt=0), dict(sl=P + 2), dict(ws=0),
    dict(ws_bytes=100),
]


@pytest.mark.parametrize("kw", KC_INVALID)
def test_kvcache_rejects_invalid(kw):
    # every case fails validation, so nothing is launched on the fake pointers
    assert kc_status(**kw) == fa.MATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dtype=1), dict(D=96), dict(page_size=48), dict(page_size=100),
                                dict(B=1 << 14, Hq=1 << 10, Hkv=1 << 10, Sq=1)])
def test_kvcache_rejects_unsupported(kw):
    assert kc_status(**kw) == fa.MATTN_ERR_UNSUPPORTED


def test_kvcache_empty_is_a_noop():
    assert kc_status(B=0, q=0, o=0, lse=0, kc=0, vc=0, bt=0, sl=0, ws=0, ws_bytes=0) == fa.MATTN_OK
    assert kc_status(Sq=0, ws=0, ws_bytes=0) == fa.MATTN_OK


def test_kvcache_workspace_size():
    ws = fa.mattn_fwd_kvcache_workspace_size
    assert ws(0, 8, 8, 1, 128, 64, 100) == 0
    assert ws(1, 6, 4, 1, 128, 64, 100) == 0
    # many sequences x heads: one split, no workspace
    assert ws(64, 32, 8, 1, 128, 64, 8) == 0
    # one short batch over a long cache: split along the keys
    n = ws(1, 8, 8, 1, 128, 64, 100)
    rows = 8
    assert n > 0 and n == ws(1, 8, 8, 1, 128, 64, 100)
    ns = None
    for cand in range(2, 65):
        o_b = (cand * rows * 128 * 4 + 255) // 256 * 256
        l_b = (cand * rows * 4 + 255) // 256 * 256
        if o_b + l_b == n:
            ns = cand
    assert ns is not None and ns <= 25  # at least four 64-token tiles per split


# The binding checks every tensor's shape and dtype against the sizes the C
# call will be given, before its device check and before any launch (the C
# side cannot see buffer extents).  CPU tensors reach those checks first, so
# each mismatch below must raise its own error, not the device error.
def _dense(B=1, Hq=4, Hkv=2, Sq=16, Skv=24, D=64, dtype=None):
    import torch

    dt = dtype or torch.bfloat16
    q = torch.zeros(B, Hq, Sq, D, dtype=dt)
    k = torch.zeros(B, Hkv, Skv, D, dtype=dt)
    return dict(q=q, k=k, v=k.clone(), o=torch.zeros_like(q), lse=torch.zeros(B, Hq, Sq),
                do=torch.zeros_like(q), dq=torch.zeros_like(q), dk=torch.zeros_like(k),
                dv=torch.zeros_like(k), workspace=torch.zeros(1 << 16, dtype=torch.uint8))


def _bad(name, fn):
    import torch

    t = _dense()
    return t, name, fn(t, torch)


DENSE_MISMATCH = {
    "v_shorter_than_k": lambda t, torch: torch.zeros(1, 2, 23, 64, dtype=torch.bfloat16),
    "v_other_dtype": lambda t, torch: torch.zeros(1, 2, 24, 64, dtype=torch.float32),
    "k_other_head_dim": lambda t, torch: torch.zeros(1, 2, 24, 128, dtype=torch.bfloat16),
    "k_other_batch": lambda t, torch: torch.zeros(2, 2, 24, 64, dtype=torch.bfloat16),
    "o_short": lambda t, torch: torch.zeros(1, 4, 15, 64, dtype=torch.bfloat16),
    "o_other_dtype": lambda t, torch: torch.zeros(1, 4, 16, 64, dtype=torch.float32),
    "lse_bf16": lambda t, torch: torch.zeros(1, 4, 16, dtype=torch.bfloat16),
    "lse_short": lambda t, torch: torch.zeros(1, 4, 15),
    "lse_4d": lambda t, torch: torch.zeros(1, 4, 16, 1),
    "q_3d": lambda t, torch: torch.zeros(4, 16, 64, dtype=torch.bfloat16),
}
FWD_TARGET = {"v_shorter_than_k": "v", "v_other_dtype": "v", "k_other_head_dim": "k",
              "k_other_batch": "k", "o_short": "o", "o_other_dtype": "o", "lse_bf16": "lse",
              "lse_short": "lse", "lse_4d": "lse", "q_3d": "q"}


@pytest.mark.parametrize("case", sorted(DENSE_MISMATCH))
def test_binding_fwd_rejects_mismatched_tensors(case):
    t, _, bad = _bad(case, DENSE_MISMATCH[case])
    t[FWD_TARGET[case]] = bad
    with pytest.raises(ValueError) as e:
        fa.mattn_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"])
    assert "GPU" not in str(e.value), e.value


BWD_MISMATCH = {
    "do": lambda torch: torch.zeros(1, 4, 16, 32, dtype=torch.bfloat16),
    "dq": lambda torch: torch.zeros(1, 4, 17, 64, dtype=torch.bfloat16),
    "dk": lambda torch: torch.zeros(1, 4, 24, 64, dtype=torch.bfloat16),
    "dv": lambda torch: torch.zeros(1, 2, 24, 64, dtype=torch.float32),
    "lse": lambda torch: torch.zeros(1, 4, 16, dtype=torch.float64),
    "workspace": lambda torch: torch.zeros(16, dtype=torch.uint8),
}


@pytest.mark.parametrize("name", sorted(BWD_MISMATCH))
@pytest.mark.parametrize("call", ["bwd", "bwd_stages"])
def test_binding_bwd_rejects_mismatched_tensors(name, call):
    import torch

    t = _dense()
    t[name] = BWD_MISMATCH[name](torch)
    args = [t[n] for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "workspace")]
    with pytest.raises(ValueError) as e:
        if call == "bwd":
            fa.mattn_bwd(*args)
        else:
            fa.mattn_bwd_stages(*args, fa.MATTN_BWD_ALL)
    assert "GPU" not in str(e.value), e.value


def _paged(B=2, Hq=8, Hkv=2, Sq=1, D=128, num_pages=6, page_size=64, pps=3):
    import torch

    q = torch.zeros(B, Hq, Sq, D, dtype=torch.bfloat16)
    kc = torch.zeros(num_pages, Hkv, page_size, D, dtype=torch.bfloat16)
    return dict(q=q, k_cache=kc, v_cache=kc.clone(),
                block_table=torch.zeros(B, pps, dtype=torch.int32),
                seqlens_k=torch.zeros(B, dtype=torch.int32), o=torch.zeros_like(q),
                lse=torch.zeros(B, Hq, Sq), workspace=torch.zeros(1 << 20, dtype=torch.uint8))


PAGED_MISMATCH = {
    "block_table": lambda torch: torch.zeros(3, 3, dtype=torch.int32),
    "seqlens_k": lambda torch: torch.zeros(1, dtype=torch.int32),
    "v_cache": lambda torch: torch.zeros(5, 2, 64, 128, dtype=torch.bfloat16),
    "k_cache": lambda torch: torch.zeros(6, 2, 64, 64, dtype=torch.bfloat16),
    "o": lambda torch: torch.zeros(2, 8, 2, 128, dtype=torch.bfloat16),
    "lse": lambda torch: torch.zeros(2, 8, 1, dtype=torch.bfloat16),
}


@pytest.mark.parametrize("name", sorted(PAGED_MISMATCH))
def test_binding_kvcache_rejects_mismatched_tensors(name):
    import torch

    t = _paged()
    t[name] = PAGED_MISMATCH[name](torch)
    with pytest.raises(ValueError) as e:
        fa.mattn_fwd_kvcache(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seqlens_k"],
                             t["o"], t["lse"], t["workspace"])
    assert "GPU" not in str(e.value), e.value


def test_binding_accepts_matching_tensors_up_to_the_device_check():
    # Consistent CPU tensors pass every shape check and stop at the device check.
    t = _dense()
    with pytest.raises(ValueError, match="GPU"):
        fa.mattn_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"])
    with pytest.raises(ValueError, match="GPU"):
        fa.mattn_bwd(*[t[n] for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv",
                                       "workspace")])
    p = _paged()
    with pytest.raises(ValueError, match="GPU"):
        fa.mattn_fwd_kvcache(p["q"], p["k_cache"], p["v_cache"], p["block_table"], p["seqlens_k"],
                             p["o"], p["lse"], p["workspace"])


def noalloc_status(B=1, Hq=2, Hkv=2, Sq=128, Skv=128, D=64, causal=0, scale=0.125, dtype=0, q=P,
                   dq=P, dk=P):
    lib = fa.load_library()
    return lib.mattn_bwd_noalloc(q, P, P, P, P, P, dq, dk, P, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                                 dtype, None)


@pytest.mark.parametrize("kw", [dict(B=-1), dict(Hq=3, Hkv=2), dict(causal=2), dict(q=0),
                                dict(dq=P + 4), dict(dk=0), dict(scale=float("nan"))])
def test_noalloc_rejects_invalid(kw):
    # rejected before the scratch lookup and before any launch
    assert noalloc_status(**kw) == fa.MATTN_ERR_INVALID_ARG


def test_noalloc_rejects_unsupported():
    assert noalloc_status(D=96) == fa.MATTN_ERR_UNSUPPORTED
    assert noalloc_status(causal=1, Sq=300, Skv=200) == fa.MATTN_ERR_UNSUPPORTED


def test_noalloc_rejects_problems_beyond_the_scratch():
    # Dlt of 2^25 - 1 rows (128 MiB) plus split partials exceeds the 128 MiB array.
    B, Hq, Hkv, Sq, Skv, D = 1, 1, 1, (1 << 25) - 1, 100, 64
    assert fa.mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D) > fa.MATTN_SCRATCH_BYTES
    assert noalloc_status(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D) == fa.MATTN_ERR_SCRATCH
    # the largest backward workspace among the workloads (DiT cross) fits
    assert fa.mattn_bwd_workspace_size(1, 10, 10, 32760, 257, 128) < fa.MATTN_SCRATCH_BYTES
    assert "scratch" in fa.mattn_strerror(fa.MATTN_ERR_SCRATCH)


def test_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MATTN_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.MATTN_SCRATCH_BYTES
