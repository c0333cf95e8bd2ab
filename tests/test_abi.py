"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid calls with the documented status before
making any HIP call (fake non-NULL pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest

import second_order_ssm_amd as tmb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twomamba.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EDEV, EALIAS, ESCRATCH = range(9)

pytestmark = pytest.mark.skipif(not os.path.exists(tmb.library_path), reason="libtwomamba.so not built")


@pytest.fixture(scope="module")
def lib():
    return tmb.load()


def declared_functions():
    """Every function declared by a header under include/."""
    names = set()
    inc = os.path.dirname(HEADER)
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(twomamba_\w+)\s*\(", src))
    return sorted(names)


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert {"twomamba_fwd", "twomamba_step", "twomamba_fwd_workspace_size", "twomamba_abi_version",
            "twomamba_status_str", "twomamba_fwd_noalloc", "twomamba_ceiling_copy", "twomamba_ceiling_mfma"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_version_and_status_strings(lib):
    assert lib.twomamba_abi_version() == 5
    seen = set()
    for s in range(9):
        txt = lib.twomamba_status_str(s).decode()
        assert txt and txt != "unknown status"
        seen.add(txt)
    assert len(seen) == 9
    assert lib.twomamba_status_str(99).decode() == "unknown status"


# fake, distinct, 256-aligned device addresses; validation never touches them
BASE = 0x7F0000000000
GAP = 1 << 34


def fake(i):
    return ctypes.c_void_p(BASE + i * GAP)


def desc(B=2, H=3, T=100, d=64, variant=0, dtype=1, chunk=0, scale=1.0, flags=0):
    return tmb.FwdDesc(B, H, T, d, d, chunk, scale, variant, dtype, flags)


def call_fwd(lib, dsc, q=1, k=2, v=3, z=4, si=None, ni=None, out=5, so=None, no=None, ws=9, wsb=1 << 40):
    p = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else fake(x))
    return lib.twomamba_fwd(ctypes.byref(dsc) if dsc is not None else None, p(q), p(k), p(v), p(z), p(si), p(ni),
                            p(out), p(so), p(no), p(ws), ctypes.c_size_t(wsb), None)


def ws_size(lib, dsc):
    n = ctypes.c_size_t(12345)
    s = lib.twomamba_fwd_workspace_size(ctypes.byref(dsc), ctypes.byref(n))
    return s, n.value


def test_workspace_size_reference_path(lib):
    # reference kernels: per-chunk state + normaliser + chunk decay per head
    d = desc(B=2, H=3, T=100, d=64, dtype=0, flags=tmb.FLAG_REFERENCE_KERNELS, chunk=64)
    s, n = ws_size(lib, d)
    assert s == OK
    nbh, nc, D = 6, 2, 2080
    a256 = lambda x: (x + 255) // 256 * 256
    expect = a256(a256(a256(nbh * nc * D * 64 * 4) + nbh * nc * D * 4) + nbh * nc * 4)
    assert n == expect
    assert ws_size(lib, desc(variant=1, flags=tmb.FLAG_REFERENCE_KERNELS)) == (OK, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ESHAPE), (dict(T=-5), ESHAPE), (dict(d=0), ESHAPE),
    (dict(dtype=7), EDTYPE), (dict(variant=3), EDTYPE),
    (dict(d=32), EUNSUP), (dict(d=128), EUNSUP), (dict(chunk=48), EUNSUP), (dict(flags=1 << 7), EUNSUP),
    (dict(variant=1, flags=1), EUNSUP), (dict(chunk=128, flags=2), EUNSUP), (dict(chunk=128, dtype=0), EUNSUP),
    (dict(scale=float("nan")), ESHAPE), (dict(scale=float("inf")), ESHAPE),
    (dict(B=1 << 30, H=1 << 30, T=1 << 30), ESHAPE),
])
def test_bad_descriptor(lib, kw, status):
    d = desc(**kw)
    assert ws_size(lib, d)[0] == status
    assert call_fwd(lib, d) == status


def test_null_arguments(lib):
    assert call_fwd(lib, None) == ENULL
    n = ctypes.c_size_t(0)
    assert lib.twomamba_fwd_workspace_size(ctypes.byref(desc()), None) == ENULL
    assert lib.twomamba_fwd_workspace_size(None, ctypes.byref(n)) == ENULL
    for field in ("q", "k", "v", "z", "out"):
        assert call_fwd(lib, desc(), **{field: None}) == ENULL
    # state pointers come in pairs
    assert call_fwd(lib, desc(), si=6, ni=None) == ENULL
    assert call_fwd(lib, desc(), so=7, no=None) == ENULL


def test_exp_rejects_state(lib):
    assert call_fwd(lib, desc(variant=1), si=6, ni=7) == EUNSUP
    assert call_fwd(lib, desc(variant=1), so=6, no=7) == EUNSUP


def test_workspace_checks(lib):
    d = desc(dtype=0, flags=tmb.FLAG_REFERENCE_KERNELS)
    _, need = ws_size(lib, d)
    assert need > 0
    assert call_fwd(lib, d, ws=None) == EWS
    assert call_fwd(lib, d, wsb=need - 1) == EWS
    assert call_fwd(lib, d, ws=ctypes.c_void_p(BASE + 9 * GAP + 16)) == EWS     # not 256-aligned


def test_alias_checks(lib):
    d = desc(dtype=0, flags=tmb.FLAG_REFERENCE_KERNELS)
    assert call_fwd(lib, d, out=1) == EALIAS                                  # out == q
    assert call_fwd(lib, d, out=ctypes.c_void_p(BASE + 2 * GAP + 64)) == EALIAS  # out inside k
    assert call_fwd(lib, d, ws=3) == EALIAS                                   # workspace == v
    assert call_fwd(lib, d, si=6, ni=7, so=ctypes.c_void_p(BASE + 6 * GAP + 256), no=8) == EALIAS  # partial alias
    assert call_fwd(lib, d, si=6, ni=7, so=7, no=8) == EALIAS                 # state_out over norm_in


def test_empty_batch_is_a_no_op(lib):
    assert call_fwd(lib, desc(B=0), q=None, k=None, v=None, z=None, out=None, ws=None, wsb=0) == OK


def call_step(lib, dsc, q=1, k=2, v=3, z=4, s=5, n=6, out=7):
    p = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else fake(x))
    return lib.twomamba_step(ctypes.byref(dsc) if dsc is not None else None, p(q), p(k), p(v), p(z), p(s), p(n),
                             p(out), None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ESHAPE), (dict(dk=32, dv=32), EUNSUP), (dict(dk=64, dv=16), EUNSUP), (dict(dtype=5), EDTYPE),
    (dict(flags=2), EUNSUP), (dict(scale=float("nan")), ESHAPE),
])
def test_step_bad_descriptor(lib, kw, status):
    a = dict(B=4, H=2, dk=64, dv=64, scale=1.0, dtype=1, flags=0)
    a.update(kw)
    assert call_step(lib, tmb.StepDesc(**a)) == status


def test_step_null_and_alias(lib):
    d = tmb.StepDesc(B=4, H=2, dk=64, dv=64, scale=1.0, dtype=1, flags=0)
    assert call_step(lib, None) == ENULL
    for f in ("q", "k", "v", "z", "s", "n", "out"):
        assert call_step(lib, d, **{f: None}) == ENULL
    assert call_step(lib, d, out=1) == EALIAS
    assert call_step(lib, d, n=5) == EALIAS
    assert call_step(lib, tmb.StepDesc(B=0, H=2, dk=64, dv=64, scale=1.0, dtype=1, flags=0),
                     q=None, k=None, v=None, z=None, s=None, n=None, out=None) == OK


# ---------------------------------------------------------------------------
# 2Mamba-E key/value cache entry points

def cdesc(B=2, H=3, d=64, max_len=100, pos=10, dtype=1, scale=1.0, flags=0):
    return tmb.ExpCacheDesc(B, H, d, d, max_len, pos, scale, dtype, flags)


def exp_step_call(lib, d, ws_bytes=1 << 20, **ptrs):
    p = {n: fake(i) for i, n in enumerate(["q", "k", "v", "z", "kc", "vc", "gc", "out", "ws"])}
    p.update(ptrs)
    return lib.twomamba_exp_step(ctypes.byref(d), p["q"], p["k"], p["v"], p["z"], p["kc"], p["vc"], p["gc"],
                                 p["out"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=100), ESHAPE),            # pos must be < max_len
    (dict(pos=-1), ESHAPE),
    (dict(max_len=-1), ESHAPE),
    (dict(dtype=5), EDTYPE),
    (dict(flags=1), EUNSUP),
    (dict(d=32), EUNSUP),
    (dict(scale=float("nan")), ESHAPE),
])
def test_exp_step_bad_descriptor(lib, kw, status):
    assert exp_step_call(lib, cdesc(**kw)) == status


def test_exp_step_workspace_and_pointers(lib):
    n = ctypes.c_size_t(0)
    d = cdesc(B=2, H=16, max_len=8192, pos=8191)
    assert lib.twomamba_exp_step_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert n.value == 32 * 16 * 66 * 4          # 16 splits of 512 keys, (dv + 2) floats each
    assert exp_step_call(lib, d, ws_bytes=n.value - 1) == EWS
    assert exp_step_call(lib, d, ws=None) == EWS
    assert exp_step_call(lib, d, ws=ctypes.c_void_p(BASE + 8 * GAP + 16)) == EWS   # misaligned
    assert exp_step_call(lib, d, q=None) == ENULL
    assert exp_step_call(lib, d, gc=None) == ENULL
    assert exp_step_call(lib, d, out=fake(0)) == EALIAS     # out over q
    assert exp_step_call(lib, d, vc=fake(4)) == EALIAS      # v cache over k cache
    assert lib.twomamba_exp_step_workspace_size(ctypes.byref(d), None) == ENULL
    empty = cdesc(B=0)
    assert exp_step_call(lib, empty, q=None, ws=None) == OK


def test_exp_cache_fill_validation(lib):
    def call(d, **ptrs):
        p = {n: fake(i) for i, n in enumerate(["k", "v", "z", "kc", "vc", "gc"])}
        p.update(ptrs)
        return lib.twomamba_exp_cache_fill(ctypes.byref(d), p["k"], p["v"], p["z"], p["kc"], p["vc"], p["gc"], None)
    assert call(cdesc(pos=101)) == ESHAPE        # T > max_len
    assert call(cdesc(pos=10, flags=2)) == EUNSUP
    assert call(cdesc(pos=10), z=None) == ENULL
    assert call(cdesc(pos=10), kc=fake(1)) == EALIAS
    assert call(cdesc(pos=0), k=None) == OK      # nothing to fill


# ---------------------------------------------------------------- backward
def call_bwd(lib, dsc, q=1, k=2, v=3, z=4, out=5, dout=6, rs=None, dq=10, dk=11, dv=12, dz=13, ws=14,
             wsb=1 << 40):
    p = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else fake(x))
    return lib.twomamba_bwd(ctypes.byref(dsc) if dsc is not None else None, p(q), p(k), p(v), p(z), p(out),
                            p(dout), p(rs), p(dq), p(dk), p(dv), p(dz), p(ws), ctypes.c_size_t(wsb), None)


def bwd_ws(lib, dsc):
    n = ctypes.c_size_t(12345)
    s = lib.twomamba_bwd_workspace_size(ctypes.byref(dsc), ctypes.byref(n))
    return s, n.value


def test_bwd_workspace_size(lib):
    # per token: fp64 decay prefix + four fp32 rows (statistic, dout.out, row and column sums)
    a256 = lambda x: (x + 255) // 256 * 256
    n = 2 * 3 * 100
    assert bwd_ws(lib, desc(B=2, H=3, T=100)) == (OK, a256(8 * n) + 4 * a256(4 * n))
    assert bwd_ws(lib, desc(B=0)) == (OK, 0)


def test_attention_form_flag_selects_the_quadratic_first_order_backward(lib):
    # TWOMAMBA_FLAG_ATTENTION_FORM (8): the first order's backward takes the attention
    # form, whose workspace is the per-token rows above; without it the O(T) form
    # (segment slots plus two fp32 rows).  Other variants ignore it; unknown bits fail.
    a256 = lambda x: (x + 255) // 256 * 256
    n = 2 * 3 * 1000
    s, chunked = bwd_ws(lib, desc(B=2, H=3, T=1000, variant=2))
    assert s == OK and chunked != a256(8 * n) + 4 * a256(4 * n)
    assert bwd_ws(lib, desc(B=2, H=3, T=1000, variant=2, flags=8)) == (OK, a256(8 * n) + 4 * a256(4 * n))
    assert bwd_ws(lib, desc(B=2, H=3, T=1000, variant=0, flags=8)) == bwd_ws(lib, desc(B=2, H=3, T=1000, variant=0))
    assert bwd_ws(lib, desc(B=2, H=3, T=1000, variant=2, flags=32))[0] == EUNSUP


def test_chunked_form_flag_selects_the_linear_2mamba_backward(lib):
    # TWOMAMBA_FLAG_CHUNKED_FORM (16): 2Mamba's backward in its linear-in-T form (a
    # workspace other than the attention form's per-token rows); by default that form from
    # 20480 tokens on, where TWOMAMBA_FLAG_ATTENTION_FORM (8) keeps the quadratic one.  The
    # first order and 2Mamba-E ignore the flag; fp32 and the reference kernels keep the
    # attention form.
    a256 = lambda x: (x + 255) // 256 * 256
    att = lambda n: a256(8 * n) + 4 * a256(4 * n)
    n = 2 * 3 * 1000
    assert bwd_ws(lib, desc(B=2, H=3, T=1000)) == (OK, att(n))
    s, ch = bwd_ws(lib, desc(B=2, H=3, T=1000, flags=16))
    assert s == OK and ch > att(n)
    assert bwd_ws(lib, desc(B=2, H=3, T=1000, flags=16 | 2)) == (OK, att(n))
    assert bwd_ws(lib, desc(B=2, H=3, T=1000, flags=16, dtype=0)) == (OK, att(n))
    assert bwd_ws(lib, desc(B=2, H=3, T=1000, variant=1, flags=16)) == (OK, att(n))
    assert bwd_ws(lib, desc(B=2, H=3, T=1000, variant=2, flags=16)) == bwd_ws(lib, desc(B=2, H=3, T=1000, variant=2))
    n = 1 * 2 * 20480
    s, ch = bwd_ws(lib, desc(B=1, H=2, T=20480))
    assert s == OK and ch > att(n)
    assert bwd_ws(lib, desc(B=1, H=2, T=20480, flags=8)) == (OK, att(n))
    assert bwd_ws(lib, desc(B=1, H=2, T=20480, flags=8 | 16)) == (OK, att(n))
    assert bwd_ws(lib, desc(B=1, H=2, T=20479)) == (OK, att(1 * 2 * 20479))
    # heads of 2^24 tokens or more: rows past 32-bit buffer offsets, the attention form
    assert bwd_ws(lib, desc(B=1, H=1, T=1 << 24, flags=16)) == (OK, att(1 << 24))
    s, ch = bwd_ws(lib, desc(B=1, H=1, T=(1 << 24) - 1, flags=16))
    assert s == OK and ch > att((1 << 24) - 1)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ESHAPE), (dict(dtype=7), EDTYPE), (dict(variant=3), EDTYPE), (dict(d=32), EUNSUP),
    (dict(variant=1, flags=1), EUNSUP), (dict(flags=1 << 7), EUNSUP), (dict(scale=float("nan")), ESHAPE),
    (dict(B=1 << 30, H=1 << 30, T=1 << 30), ESHAPE),
])
def test_bwd_bad_descriptor(lib, kw, status):
    d = desc(**kw)
    assert bwd_ws(lib, d)[0] == status
    assert call_bwd(lib, d) == status


def test_bwd_pointer_checks(lib):
    d = desc()
    _, need = bwd_ws(lib, d)
    assert call_bwd(lib, None) == ENULL
    for field in ("q", "k", "v", "z", "out", "dout", "dq", "dk", "dv", "dz"):
        assert call_bwd(lib, d, **{field: None}) == ENULL
    assert call_bwd(lib, d, ws=None) == EWS
    assert call_bwd(lib, d, wsb=need - 1) == EWS
    assert call_bwd(lib, d, ws=ctypes.c_void_p(BASE + 14 * GAP + 16)) == EWS
    assert call_bwd(lib, d, dq=1) == EALIAS                                  # dq == q
    assert call_bwd(lib, d, dv=ctypes.c_void_p(BASE + 6 * GAP + 64)) == EALIAS  # dv inside dout
    assert call_bwd(lib, d, dk=10) == EALIAS                                 # dk == dq
    assert call_bwd(lib, d, ws=13) == EALIAS                                 # workspace == dz
    assert call_bwd(lib, d, rs=13) == EALIAS                                 # row statistics == dz
    assert call_bwd(lib, d, rs=ctypes.c_void_p(BASE + 14 * GAP + 256)) == EALIAS   # inside the workspace
    assert call_bwd(lib, desc(B=0), q=None, k=None, v=None, z=None, out=None, dout=None, dq=None, dk=None,
                    dv=None, dz=None, ws=None, wsb=0) == OK


# ---------------------------------------------------------------- forward with row statistics
def call_fwd_stats(lib, dsc, rs=7, si=None, ni=None, so=None, no=None, ws=9, wsb=1 << 40):
    p = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else fake(x))
    return lib.twomamba_fwd_stats(ctypes.byref(dsc), p(1), p(2), p(3), p(4), p(si), p(ni), p(5), p(so), p(no), p(rs),
                                  p(ws), ctypes.c_size_t(wsb), None)


def test_fwd_stats_pointer_checks(lib):
    # the validation of the plain forward plus the statistics buffer: required,
    # [B][H][T] fp32 disjoint from everything else, none for the first order
    # (no call here gets past validation: nothing is launched)
    d = desc(T=1000)                      # needs a workspace
    n = 2 * 3 * 1000
    assert call_fwd_stats(lib, d, rs=None) == ENULL
    assert call_fwd_stats(lib, d, rs=4) == EALIAS                                        # == z
    assert call_fwd_stats(lib, d, rs=ctypes.c_void_p(BASE + 4 * GAP + 4 * (n - 1))) == EALIAS   # last float of z
    assert call_fwd_stats(lib, d, rs=ctypes.c_void_p(BASE + 4 * GAP + 4 * n), ws=None) == EWS   # just past z: taken
    assert call_fwd_stats(lib, d, rs=9) == EALIAS                                        # == workspace
    assert call_fwd_stats(lib, d, rs=5) == EALIAS                                        # == out
    assert call_fwd_stats(lib, desc(variant=1), rs=2) == EALIAS                          # 2Mamba-E: == k
    assert call_fwd_stats(lib, desc(variant=2)) == EUNSUP                                # first order: none
    assert call_fwd_stats(lib, desc(B=0), rs=None, ws=None, wsb=0) == OK


# ---------------------------------------------------------------- input convolution
def call_conv(lib, dsc, q=1, k=2, v=3, w=4, b=None, si=None, qo=6, ko=7, vo=8, so=None):
    p = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else fake(x))
    return lib.twomamba_conv2(ctypes.byref(dsc) if dsc is not None else None, p(q), p(k), p(v), p(w), p(b), p(si),
                              p(qo), p(ko), p(vo), p(so), None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ESHAPE), (dict(d=32), EUNSUP), (dict(dtype=5), EDTYPE), (dict(flags=1), EUNSUP),
    (dict(B=1 << 30, H=1 << 30, T=1 << 30), ESHAPE),
])
def test_conv_bad_descriptor(lib, kw, status):
    a = dict(B=2, H=3, T=50, d=64, dtype=1, flags=0)
    a.update(kw)
    assert call_conv(lib, tmb.ConvDesc(**a)) == status


def test_conv_pointer_checks(lib):
    dsc = tmb.ConvDesc(2, 3, 50, 64, 1, 0)
    assert call_conv(lib, None) == ENULL
    for field in ("q", "k", "v", "w", "qo", "ko", "vo"):
        assert call_conv(lib, dsc, **{field: None}) == ENULL
    assert call_conv(lib, dsc, qo=1) == EALIAS                  # q_out == q
    assert call_conv(lib, dsc, ko=6) == EALIAS                  # k_out == q_out
    assert call_conv(lib, dsc, so=4) == EALIAS                  # state out == weight
    assert call_conv(lib, dsc, w=ctypes.c_void_p(BASE + 4 * GAP + 8)) == EUNSUP   # weight not 16-byte aligned
    assert call_conv(lib, tmb.ConvDesc(0, 3, 50, 64, 1, 0), q=None, k=None, v=None, w=None, qo=None, ko=None,
                     vo=None) == OK


def test_step_conv_checks(lib):
    d = tmb.StepDesc(2, 3, 64, 64, 1.0, 1, 0)
    p = lambda x: None if x is None else fake(x)

    def call(w=10, cs=11, b=None, state=6, d_=d):
        return lib.twomamba_step_conv(ctypes.byref(d_), p(1), p(2), p(3), p(4), p(w), p(b), p(cs), p(state),
                                      p(7), p(8), None)
    assert call(w=None) == ENULL
    assert call(cs=None) == ENULL
    assert call(cs=6) == EALIAS                                 # cache over the state
    assert call(cs=1) == EALIAS                                 # cache over q
    assert call(d_=tmb.StepDesc(2, 3, 64, 16, 1.0, 1, 0)) == EUNSUP


# ---------------------------------------------------------------- first order
def test_first_order_forward_validation(lib):
    d = desc(variant=2)
    a256 = lambda x: (x + 255) // 256 * 256
    s, n = ws_size(lib, d)
    assert s == OK and n == a256(a256(6 * 2 * 64 * 64 * 4) + 6 * 2 * 4)      # per-chunk d x d states + decays
    assert call_fwd(lib, d, si=6, ni=7) == EUNSUP                           # no normaliser
    assert call_fwd(lib, d, so=6, no=7) == EUNSUP
    assert call_fwd(lib, desc(variant=2, flags=1), out=1) == EALIAS         # NO_NORM accepted, checks still run


def test_first_order_step_validation(lib):
    p = lambda x: None if x is None else fake(x)
    d = tmb.StepDesc(2, 3, 64, 64, 1.0, 1, tmb.FLAG_FIRST_ORDER)
    call = lambda norm: lib.twomamba_step(ctypes.byref(d), p(1), p(2), p(3), p(4), p(5), p(norm), p(7), None)
    assert call(6) == EUNSUP                                                # first order takes no normaliser
    bad = tmb.StepDesc(2, 3, 64, 64, 1.0, 1, 8)
    assert lib.twomamba_step(ctypes.byref(bad), p(1), p(2), p(3), p(4), p(5), p(6), p(7), None) == EUNSUP


# ---------------------------------------------------------------- no fallback
def test_missing_library_fails_loudly(tmp_path):
    # the binding has no CPU or oracle fallback: without the library it raises
    with pytest.raises(RuntimeError):
        tmb.load(str(tmp_path / "libtwomamba.so"))


def test_product_package_never_touches_the_oracle():
    # the oracle is test infrastructure: nothing under the package imports or
    # names it
    pkg = os.path.dirname(tmb.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(root, f), encoding="utf-8").read()
                assert "oracle" not in src, f"{f} refers to the oracle"


def call_fwd_noalloc(lib, dsc, q=1, k=2, v=3, z=4, si=None, ni=None, out=5, so=None, no=None):
    p = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else fake(x))
    return lib.twomamba_fwd_noalloc(ctypes.byref(dsc) if dsc is not None else None, p(q), p(k), p(v), p(z), p(si),
                                    p(ni), p(out), p(so), p(no), None)


def test_fwd_noalloc_validation_before_any_hip_call(lib):
    # the checks of twomamba_fwd, then the static scratch's limit (128 MiB), all
    # before the scratch lookup (the call's first HIP call): nothing here is launched
    assert call_fwd_noalloc(lib, None) == ENULL
    assert call_fwd_noalloc(lib, desc(T=100), q=None) == ENULL
    assert call_fwd_noalloc(lib, desc(T=100), out=1) == EALIAS
    assert call_fwd_noalloc(lib, desc(T=100, d=48)) == EUNSUP
    # fp32 reference kernels keep one state per chunk: 2 heads x 256 chunks x 532 KB > 128 MiB
    big = desc(B=1, H=2, T=16384, d=64, dtype=0)
    s, need = ws_size(lib, big)
    assert s == OK and need > (128 << 20)
    assert call_fwd_noalloc(lib, big) == ESCRATCH
    assert lib.twomamba_status_str(ESCRATCH).decode() == "workspace larger than the library's static scratch"


def test_ceiling_kernels_validate_before_any_hip_call(lib):
    vp = ctypes.c_void_p
    assert lib.twomamba_ceiling_copy(None, fake(1), ctypes.c_size_t(64), None) == ENULL
    assert lib.twomamba_ceiling_copy(fake(0), fake(1), ctypes.c_size_t(65), None) == EUNSUP     # not 16-byte sized
    assert lib.twomamba_ceiling_copy(vp(BASE + 8), fake(1), ctypes.c_size_t(64), None) == EUNSUP  # misaligned
    assert lib.twomamba_ceiling_copy(fake(0), vp(BASE + 32), ctypes.c_size_t(64), None) == EALIAS  # overlap
    assert lib.twomamba_ceiling_copy(fake(0), fake(1), ctypes.c_size_t(0), None) == OK           # nothing to do
    assert lib.twomamba_ceiling_mfma(0, 10, fake(0), None, None) == ESHAPE
    assert lib.twomamba_ceiling_mfma(4, 10, None, None, None) == ENULL


def call_fwd_conv(lib, dsc, w=20, b=None, ci=None, co=None, ws=9, wsb=1 << 40, q=1, out=5):
    p = lambda x: None if x is None else (x if isinstance(x, ctypes.c_void_p) else fake(x))
    return lib.twomamba_fwd_conv(ctypes.byref(dsc), p(q), p(2), p(3), p(4), p(w), p(b), p(ci), p(co), None, None,
                                 p(out), None, None, p(ws), ctypes.c_size_t(wsb), None)


def test_fwd_conv_validation_and_workspace(lib):
    # the forward's checks plus those of the convolution, all before any HIP call
    d = desc(T=100)
    assert call_fwd_conv(lib, d, w=None) == ENULL
    assert call_fwd_conv(lib, d, w=ctypes.c_void_p(BASE + 20 * GAP + 8)) == EUNSUP      # misaligned weight
    assert call_fwd_conv(lib, d, co=1) == EALIAS                                      # cache out == q
    assert call_fwd_conv(lib, d, co=20) == EALIAS                                     # cache out == weight
    assert call_fwd_conv(lib, d, out=20) == EALIAS                                    # out == weight
    assert call_fwd_conv(lib, d, ws=None) == EWS
    n = ctypes.c_size_t(0)
    # first order at bf16, d = 64 convolves in its kernels: no more workspace than the plain forward
    for variant, extra in ((2, 0), (1, 2), (0, 3)):
        dd = desc(B=2, H=3, T=1000, variant=variant)
        assert lib.twomamba_fwd_conv_workspace_size(ctypes.byref(dd), ctypes.byref(n)) == OK
        s, plain = ws_size(lib, dd)
        tensor = (2 * 3 * 1000 * 64 * 2 + 255) // 256 * 256
        base = (plain + 255) // 256 * 256 if extra else plain
        assert n.value == base + extra * tensor, (variant, n.value, plain)


@pytest.mark.parametrize("variant,fused", [(1, 2), (2, 0)])   # 2Mamba-E convolves k, v up front; first order none
def test_mfma_paths_stop_at_32bit_head_offsets(lib, variant, fused):
    # The 2Mamba-E and first-order MFMA kernels address a head's rows through 32-bit
    # buffer offsets; from 2^24 tokens per head (2^31 bytes at d = 64, bf16) the
    # forward takes the reference kernels instead of wrapping.  The convolution's
    # workspace shows which path a shape gets: the reference path convolves all
    # three tensors up front, the MFMA paths fewer.
    n = ctypes.c_size_t(0)
    for T, expect in (((1 << 24) - 1, fused), (1 << 24, 3)):
        dd = desc(B=1, H=1, T=T, variant=variant)
        assert lib.twomamba_fwd_conv_workspace_size(ctypes.byref(dd), ctypes.byref(n)) == OK
        s, plain = ws_size(lib, dd)
        assert s == OK
        tensor = (T * 64 * 2 + 255) // 256 * 256
        base = (plain + 255) // 256 * 256 if expect else plain
        assert n.value == base + expect * tensor, (variant, T, n.value, plain)
