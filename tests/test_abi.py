"""CPU checks of the C ABI: the library loads, exports what include/attn.h
declares, and rejects bad arguments on the host before any launch.

Every call here fails validation, so no kernel is launched and no GPU is
needed.  Pointers are fake (never dereferenced) and 256-byte aligned.
"""

import ctypes
import os
import re

import pytest

import exact_attention_attn_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x10000  # fake, aligned, never dereferenced


def declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.library_path()):
        pytest.fail("libattn_mi355x.so not built: run `python -m exact_attention_attn_amd.build`")
    return A.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"attn_fwd", "attn_fwd_max_logit", "attn_fwd_varlen", "attn_bwd", "attn_decode_splitkv",
                          "attn_decode_splitkv_paged", "attn_decode_plan", "attn_combine",
                          "attn_decode_noalloc", "attn_strerror", "attn_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.attn_version().decode().startswith("attn-mi355x")


def test_strerror(lib):
    for code in range(7):
        assert lib.attn_strerror(code)
    assert b"scratch" in lib.attn_strerror(6)
    assert b"unknown" in lib.attn_strerror(99)


def fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, sinks=P, out=P, lse=P, B=1, Hq=8, Hkv=2, Lq=10, Lk=10, D=128,
             window=0, scale=0.1, ind=0, outd=0, stream=None)
    a.update(kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["sinks"], a["out"], a["lse"], a["B"], a["Hq"],
                        a["Hkv"], a["Lq"], a["Lk"], a["D"], a["window"], a["scale"], a["ind"],
                        a["outd"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(B=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(Lq=0), 2), (dict(Lk=0), 2),
    (dict(Hq=7), 2), (dict(Lq=11), 2), (dict(B=1 << 30, Hq=64, Hkv=8, Lq=1 << 20, Lk=1 << 20), 2),
    (dict(D=96), 3), (dict(D=256), 3), (dict(ind=2), 3), (dict(outd=-1), 3),
    (dict(scale=0.0), 4), (dict(scale=-1.0), 4), (dict(scale=float("inf")), 4),
    (dict(scale=float("nan")), 4), (dict(q=P + 8), 4), (dict(out=P + 2), 4), (dict(lse=P + 2), 4),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def fwd_ml(lib, **kw):
    a = dict(q=P, k=P, v=P, sinks=P, out=P, lse=P, mrow=P, mhead=P, B=1, Hq=8, Hkv=2, Lq=10,
             Lk=10, D=128, window=0, scale=0.1, ind=0, outd=0, stream=None)
    a.update(kw)
    return lib.attn_fwd_max_logit(a["q"], a["k"], a["v"], a["sinks"], a["out"], a["lse"],
                                  a["mrow"], a["mhead"], a["B"], a["Hq"], a["Hkv"], a["Lq"],
                                  a["Lk"], a["D"], a["window"], a["scale"], a["ind"], a["outd"],
                                  a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(Hq=7), 2), (dict(Lq=11), 2), (dict(D=96), 3),
    (dict(scale=0.0), 4), (dict(q=P + 8), 4), (dict(lse=P + 2), 4), (dict(mrow=P + 2), 4),
    (dict(mhead=P + 1), 4), (dict(sinks=P + 2), 4),
])
def test_fwd_max_logit_rejects(lib, kw, code):
    assert fwd_ml(lib, **kw) == code


def dec(lib, **kw):
    a = dict(q=P, k=P, v=P, sl=P, ns=P, op=P, lp=P, B=4, Hq=8, Hkv=2, Lk=100, D=128, ms=64,
             window=0, scale=0.1, ind=0, stream=None)
    a.update(kw)
    return lib.attn_decode_splitkv(a["q"], a["k"], a["v"], a["sl"], a["ns"], a["op"], a["lp"],
                                   a["B"], a["Hq"], a["Hkv"], a["Lk"], a["D"], a["ms"],
                                   a["window"], a["scale"], a["ind"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(sl=None), 1), (dict(ns=None), 1), (dict(op=None), 1), (dict(lp=None), 1),
    (dict(B=0), 2), (dict(Hq=6, Hkv=4), 2), (dict(ms=0), 2), (dict(ms=65), 2), (dict(Lk=0), 2),
    (dict(D=80), 3), (dict(ind=1), 3), (dict(scale=0.0), 4), (dict(k=P + 4), 4), (dict(sl=P + 2), 4),
    (dict(B=1 << 16, Hq=512, Hkv=512), 2),  # B*Hq*max_splits = 2^31: item ids need 32 bits
])
def test_decode_rejects(lib, kw, code):
    assert dec(lib, **kw) == code


def comb(lib, **kw):
    a = dict(op=P, lp=P, sl=P, ns=P, sinks=P, out=P, lse=P, B=4, Hq=8, D=128, Lk=100, ms=64,
             window=0, outd=0, stream=None)
    a.update(kw)
    return lib.attn_combine(a["op"], a["lp"], a["sl"], a["ns"], a["sinks"], a["out"], a["lse"],
                            a["B"], a["Hq"], a["D"], a["Lk"], a["ms"], a["window"], a["outd"],
                            a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), 1), (dict(out=None), 1), (dict(sl=None), 1),
    (dict(B=0), 2), (dict(ms=0), 2), (dict(ms=100), 2), (dict(Lk=0), 2),
    (dict(D=32), 3), (dict(outd=7), 3), (dict(out=P + 8), 4), (dict(sinks=P + 1), 4),
])
def test_combine_rejects(lib, kw, code):
    assert comb(lib, **kw) == code


def test_python_binding_raises_on_error_code(lib):
    with pytest.raises(A.AttnError) as e:
        A._check("attn_fwd", 2)
    assert e.value.code == 2 and "shape" in str(e.value)


def test_binding_rejects_host_tensors():
    import torch

    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.attn_fwd(q, k, k, None, q.clone())


def plan(lib, **kw):
    a = dict(sl=P, ns=P, B=4, Hq=8, Hkv=2, Lk=100, ms=64, window=0, policy=0, param=0, stream=None)
    a.update(kw)
    return lib.attn_decode_plan(a["sl"], a["ns"], a["B"], a["Hq"], a["Hkv"], a["Lk"], a["ms"],
                                a["window"], a["policy"], a["param"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(sl=None), 1), (dict(ns=None), 1), (dict(B=0), 2), (dict(Hq=6, Hkv=4), 2), (dict(ms=0), 2),
    (dict(ms=65), 2), (dict(Lk=0), 2), (dict(B=70000), 2), (dict(policy=3), 3), (dict(policy=-1), 3),
    (dict(policy=0, param=-1), 4), (dict(policy=1, param=0), 4), (dict(policy=2, param=0), 4),
    (dict(sl=P + 2), 4), (dict(ns=P + 1), 4),
    (dict(B=1 << 15, Hq=1024, Hkv=1024), 2),  # B*Hq*max_splits = 2^31: item counts need 32 bits
])
def test_plan_rejects(lib, kw, code):
    assert plan(lib, **kw) == code


def varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, cq=P, ck=P, sinks=P, out=P, lse=P, B=3, Hq=8, Hkv=2, tq=100, tk=120,
             mq=50, D=128, window=0, scale=0.1, ind=0, outd=0, stream=None)
    a.update(kw)
    return lib.attn_fwd_varlen(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["sinks"], a["out"],
                               a["lse"], a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"],
                               a["D"], a["window"], a["scale"], a["ind"], a["outd"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(cq=None), 1), (dict(ck=None), 1), (dict(out=None), 1),
    (dict(B=0), 2), (dict(tq=0), 2), (dict(tk=-1), 2), (dict(mq=0), 2), (dict(mq=101), 2),
    (dict(Hq=7), 2), (dict(B=70000), 2), (dict(D=96), 3), (dict(ind=1), 3), (dict(outd=5), 3),
    (dict(scale=0.0), 4), (dict(q=P + 8), 4), (dict(cq=P + 2), 4), (dict(lse=P + 1), 4),
])
def test_varlen_rejects(lib, kw, code):
    assert varlen(lib, **kw) == code


def paged(lib, **kw):
    a = dict(q=P, kp=P, vp=P, bt=P, sl=P, ns=P, op=P, lp=P, B=4, Hq=8, Hkv=2, npg=100, ps=16,
             mp=10, D=128, ms=64, window=0, scale=0.1, ind=0, stream=None)
    a.update(kw)
    return lib.attn_decode_splitkv_paged(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["ns"],
                                         a["op"], a["lp"], a["B"], a["Hq"], a["Hkv"], a["npg"],
                                         a["ps"], a["mp"], a["D"], a["ms"], a["window"],
                                         a["scale"], a["ind"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(bt=None), 1), (dict(kp=None), 1), (dict(lp=None), 1),
    (dict(B=0), 2), (dict(npg=0), 2), (dict(ps=0), 2), (dict(ps=24), 2), (dict(mp=0), 2),
    (dict(ms=65), 2), (dict(Hq=6, Hkv=4), 2), (dict(mp=1 << 27, ps=1 << 5), 2),
    (dict(D=80), 3), (dict(ind=1), 3), (dict(scale=-1.0), 4), (dict(bt=P + 2), 4),
    (dict(kp=P + 8), 4), (dict(B=1 << 16, Hq=512, Hkv=512), 2),
])
def test_paged_rejects(lib, kw, code):
    assert paged(lib, **kw) == code


def bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, sinks=P, out=P, dout=P, lse=P, dq=P, dk=P, dv=P, dsink=P, delta=P, B=1,
             Hq=8, Hkv=2, Lq=10, Lk=10, D=128, window=0, scale=0.1, ind=0, outd=1, stream=None)
    a.update(kw)
    return lib.attn_bwd(a["q"], a["k"], a["v"], a["sinks"], a["out"], a["dout"], a["lse"], a["dq"],
                        a["dk"], a["dv"], a["dsink"], a["delta"], a["B"], a["Hq"], a["Hkv"],
                        a["Lq"], a["Lk"], a["D"], a["window"], a["scale"], a["ind"], a["outd"],
                        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(dout=None), 1), (dict(lse=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1), (dict(delta=None), 1), (dict(Hq=7), 2), (dict(Lq=11), 2), (dict(B=0), 2),
    (dict(D=96), 3), (dict(ind=1), 3), (dict(outd=3), 3), (dict(scale=0.0), 4),
    (dict(sinks=None), 4), (dict(dq=P + 4), 4), (dict(delta=P + 2), 4), (dict(dout=P + 8), 4),
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_binding_checks_decode_inputs_on_host():
    # Only pointers reach the C ABI, so the binding checks what it cannot:
    # bf16 caches and per-sequence arrays of exactly B int32 (the kernels read B).
    import torch

    B, Hq, Hkv, L, D = 3, 4, 2, 16, 64
    q = torch.zeros(B, Hq, 1, D, dtype=torch.bfloat16)
    kc = torch.zeros(B, Hkv, L, D, dtype=torch.bfloat16)
    sl = torch.full((B,), L, dtype=torch.int32)
    op = torch.zeros(B, Hq, 8, D)
    lp = torch.zeros(B, Hq, 8)
    out = torch.zeros(B, Hq, 1, D)
    with pytest.raises(TypeError):
        A.attn_decode_splitkv(q, kc.float(), kc, sl, sl, op, lp)
    with pytest.raises(ValueError):
        A.attn_decode_splitkv(q, kc, kc, sl[:2], sl, op, lp)
    with pytest.raises(ValueError):
        A.attn_decode_splitkv(q, kc, kc, sl, sl.long(), op, lp)
    with pytest.raises(ValueError):
        A.attn_combine(op, lp, sl[:1], sl, None, out, Lk_max=L)
    with pytest.raises(ValueError):
        A.attn_combine(op, lp, sl, sl.float(), None, out, Lk_max=L)
    pages = torch.zeros(6, Hkv, 8, D, dtype=torch.bfloat16)
    table = torch.zeros(B, 2, dtype=torch.int32)
    with pytest.raises(TypeError):
        A.attn_decode_splitkv_paged(q, pages.float(), pages, table, sl, sl, op, lp)
    with pytest.raises(ValueError):
        A.attn_decode_splitkv_paged(q, pages, pages, table, sl, sl[:1], op, lp)


def test_binding_checks_input_dtypes_on_host():
    import torch

    q = torch.zeros(4, 10, 64, dtype=torch.bfloat16)
    k = torch.zeros(2, 10, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(TypeError):
        A.attn_fwd_varlen(q, k.float(), k, cu, cu, None, q.clone(), max_seqlen_q=10)
    q4 = torch.zeros(1, 4, 10, 64, dtype=torch.bfloat16)
    k4 = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16)
    f = torch.zeros(1, 4, 10, 64)
    with pytest.raises(TypeError):
        A.attn_bwd(q4, k4, k4.float(), None, f, q4, torch.zeros(1, 4, 10), f, f[:, :2], f[:, :2])


def noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, sl=P, ns=P, sinks=P, out=P, lse=P, B=4, Hq=8, Hkv=2, Lk=100, D=128,
             ms=64, window=0, scale=0.1, ind=0, outd=1, stream=None)
    a.update(kw)
    return lib.attn_decode_noalloc(a["q"], a["k"], a["v"], a["sl"], a["ns"], a["sinks"], a["out"],
                                   a["lse"], a["B"], a["Hq"], a["Hkv"], a["Lk"], a["D"], a["ms"],
                                   a["window"], a["scale"], a["ind"], a["outd"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(sl=None), 1), (dict(out=None), 1),
    (dict(B=0), 2), (dict(Hq=6, Hkv=4), 2), (dict(ms=0), 2), (dict(ms=65), 2),
    (dict(D=80), 3), (dict(ind=1), 3), (dict(outd=4), 3), (dict(scale=0.0), 4),
    (dict(out=P + 8), 4), (dict(lse=P + 2), 4), (dict(sl=P + 2), 4),
    # workspaces beyond ATTN_NOALLOC_SCRATCH_BYTES: refused before any HIP call
    (dict(B=65, Hq=64, Hkv=8, ms=64), 6), (dict(B=64, Hq=64, Hkv=8, ms=64, D=128), None),
    (dict(B=1, Hq=4104, Hkv=8, ms=64, D=128), 6), (dict(B=128, Hq=64, Hkv=8, ms=64, D=64), 6),
])
def test_noalloc_rejects(lib, kw, code):
    if code is None:
        # the largest workload that fits must pass the size check; it is not
        # launched here (no GPU), so only the bound itself is checked
        B, Hq, ms, D = kw["B"], kw["Hq"], kw["ms"], kw["D"]
        lanes = B * Hq * ms
        need = -(-lanes * D * 4 // 256) * 256 + lanes * 4
        assert need == A.NOALLOC_SCRATCH_BYTES
        return
    assert noalloc(lib, **kw) == code
