"""The C-ABI library loads, exports every entry point include/dion.h
declares, and rejects bad arguments before making any HIP call (so these
run on a machine without a GPU)."""
import ctypes
import math
import os
import re

import pytest

import rank_orthonormalized_optimizer_dion_amd as dion

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dion.h")

# Distinct, aligned fake device addresses: validation never dereferences them.
FX, FG, FR, FV, FW = (k << 40 for k in range(1, 6))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dion_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return dion.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert lib.dion_version() >= 200


def test_only_dion_symbols_exported():
    out = os.popen(f"nm -D --defined-only {dion.library_path()}").read().split("\n")
    syms = [l.split()[-1] for l in out if l.strip() and l.split()[1] in "TDBR"]
    exported = [s for s in syms if not s.startswith("_")]
    assert exported and all(s.startswith("dion_") for s in exported), exported


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.dion_error_string(code)


def step(lib, X=FX, G=FG, R=FR, V=FV, m=64, n=32, r=8, eta=0.01, beta=0.95, variant=1,
         gd=0, ws=FW, nbytes=None):
    if nbytes is None:
        nbytes = lib.dion_workspace_size(m, n, r, variant, gd) if m > 0 and n > 0 else 1 << 30
    return lib.dion_step(X, G, R, V, m, n, r, eta, beta, variant, gd, ws, nbytes, None)


@pytest.mark.parametrize("kw", [
    dict(X=None), dict(G=None), dict(R=None), dict(V=None),
    dict(m=0), dict(n=0), dict(r=0), dict(r=33), dict(m=16, n=32, r=17),
    dict(variant=2), dict(variant=-1), dict(gd=2),
    dict(eta=math.nan), dict(beta=math.inf), dict(eta=-math.inf),
    dict(X=FX + 2), dict(G=FG + 2), dict(G=FG + 1, gd=1),
    dict(R=FX + 64),                       # R overlaps X
    dict(m=1 << 21), dict(m=1 << 16, n=1 << 16, r=8),
])
def test_invalid_arguments(lib, kw):
    assert step(lib, **kw) == dion.ERR_INVALID_ARG


def test_workspace_checks(lib):
    need = lib.dion_workspace_size(64, 32, 8, 1, 0)
    assert need > 0
    assert step(lib, nbytes=need - 1) == dion.ERR_WORKSPACE
    assert step(lib, ws=None) == dion.ERR_WORKSPACE
    assert step(lib, ws=FW + 8) == dion.ERR_WORKSPACE      # misaligned


def test_workspace_size_query(lib):
    assert lib.dion_workspace_size(64, 32, 33, 1, 0) == 0
    assert lib.dion_workspace_size(64, 32, 0, 1, 0) == 0
    a = lib.dion_workspace_size(3072, 8192, 768, 1, 1)
    b = lib.dion_workspace_size(3072, 8192, 192, 1, 1)
    # at least the three factor buffers (P, scratch, W) of float32
    assert a >= 4 * 768 * (3072 + 8192 + 8192)
    assert a > b > 0


def test_batched_validation(lib):
    mats = (dion.dion_matrix * 2)()
    mats[0] = dion.dion_matrix(FX, FG, FR, FV, 64, 32, 8)
    mats[1] = dion.dion_matrix(FX + (1 << 36), FG + (1 << 36), FR + (1 << 36),
                               FV + (1 << 36), 48, 96, 16)
    size = lib.dion_workspace_size_batched(mats, 2, 1, 0)
    single = (lib.dion_workspace_size(64, 32, 8, 1, 0) +
              lib.dion_workspace_size(48, 96, 16, 1, 0))
    assert size > 0 and size >= single - 4096
    assert lib.dion_workspace_size_batched(mats, 0, 1, 0) == 0
    bad = (dion.dion_matrix * 1)()
    bad[0] = dion.dion_matrix(FX, FG, FR, FV, 64, 32, 40)
    assert lib.dion_workspace_size_batched(bad, 1, 1, 0) == 0
    assert lib.dion_step_batched(bad, 1, 0.01, 0.95, 1, 0, FW, 1 << 30, None) == \
        dion.ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.dion_plan_create(bad, 1, 1, 0, ctypes.byref(h)) == dion.ERR_INVALID_ARG
    assert lib.dion_plan_create(mats, 2, 5, 0, ctypes.byref(h)) == dion.ERR_INVALID_ARG
    assert not h.value
    assert lib.dion_status(None, 1, None, None) == dion.ERR_INVALID_ARG


def test_sharded_variant_rejected_outside_plans(lib):
    sharded = 1 | 0x200
    assert step(lib, variant=sharded, nbytes=1 << 30) == dion.ERR_INVALID_ARG
    assert lib.dion_workspace_size(64, 32, 8, sharded, 0) == 0
    mats = (dion.dion_matrix * 1)(dion.dion_matrix(FX, FG, FR, FV, 64, 32, 8))
    assert lib.dion_workspace_size_batched(mats, 1, sharded, 0) == 0
    assert lib.dion_step_batched(mats, 1, 0.01, 0.95, sharded, 0, FW, 1 << 30, None) == \
        dion.ERR_INVALID_ARG


def test_shard_entry_points_reject_null_plan(lib):
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.dion_plan_shard_stage(None, 0, 0.01, 0.95, FW, 1 << 30, None) == \
        dion.ERR_INVALID_ARG
    assert lib.dion_plan_shard_buffer(None, 0, 0, ctypes.byref(off), ctypes.byref(nb)) == \
        dion.ERR_INVALID_ARG


def test_plan_buffer_rejects_bad_arguments(lib):
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    for which in (dion.BUF_P, dion.BUF_U, dion.BUF_W):
        assert lib.dion_plan_buffer(None, which, 0, ctypes.byref(off), ctypes.byref(nb)) == \
            dion.ERR_INVALID_ARG


def test_gram_variant_bit(lib):
    # the sliced Gram (default) needs its digit planes in the workspace;
    # DION_GRAM_F64 does not, and an unknown bit is rejected
    m, n, r = 3072, 8192, 768
    sliced = lib.dion_workspace_size(m, n, r, 1, 1)
    f64 = lib.dion_workspace_size(m, n, r, 1 | dion.GRAM_F64, 1)
    assert f64 > 0
    assert sliced - f64 >= 5 * r * max(m, n)
    assert lib.dion_workspace_size(m, n, r, 1 | 0x1000, 1) == 0


def test_grouped_schedule_bit(lib):
    # DION_SCHED_GROUPED is accepted and changes no workspace size
    for m, n, r in ((256, 128, 16), (3072, 8192, 768)):
        plain = lib.dion_workspace_size(m, n, r, 1, 0)
        assert plain > 0
        assert lib.dion_workspace_size(m, n, r, 1 | dion.SCHED_GROUPED, 0) == plain


def test_binding_constants_match_header():
    # the binding's flag and status values are the header's #defines
    here = os.path.dirname(os.path.abspath(__file__))
    text = open(os.path.join(here, "..", "include", "dion.h")).read()
    defs = {k: int(v, 0) for k, v in re.findall(r"#define\s+(DION_\w+)\s+\(?(-?(?:0x)?[0-9a-fA-F]+)\)?", text)}
    assert defs["DION_VARIANT_DION"] == dion.VARIANTS["dion"]
    assert defs["DION_VARIANT_ORTH"] == dion.VARIANTS["orth"]
    assert defs["DION_MATH_F32"] == dion.MATH["f32"]
    assert defs["DION_MATH_BF16X3"] == dion.MATH["bf16x3"]
    assert defs["DION_GRAM_F64"] == dion.GRAM_F64
    assert defs["DION_SHARDED"] == dion.SHARDED
    assert defs["DION_SCHED_GROUPED"] == dion.SCHED_GROUPED
    assert defs["DION_SHARD_GRAM"] == dion.SHARD_GRAM and defs["DION_SHARD_W"] == dion.SHARD_W
    assert (defs["DION_BUF_P"], defs["DION_BUF_U"], defs["DION_BUF_W"]) == \
        (dion.BUF_P, dion.BUF_U, dion.BUF_W)
    assert defs["DION_OK"] == dion.OK and defs["DION_ERR_INVALID_ARG"] == dion.ERR_INVALID_ARG
    assert defs["DION_ERR_WORKSPACE"] == dion.ERR_WORKSPACE and defs["DION_ERR_HIP"] == dion.ERR_HIP
    assert defs["DION_ERR_BREAKDOWN"] == dion.ERR_BREAKDOWN
    assert (defs["DION_STATUS_ORTH_P"], defs["DION_STATUS_ORTH_W"], defs["DION_STATUS_COLNORM"]) == \
        (dion.STATUS_ORTH_P, dion.STATUS_ORTH_W, dion.STATUS_COLNORM)
    # the three flag groups do not overlap
    assert not (defs["DION_VARIANT_MASK"] & (defs["DION_MATH_MASK"] | defs["DION_SHARDED"] | defs["DION_GRAM_F64"]))
    assert not (defs["DION_MATH_MASK"] & (defs["DION_SHARDED"] | defs["DION_GRAM_F64"]))
    assert not (defs["DION_SHARDED"] & defs["DION_GRAM_F64"])
