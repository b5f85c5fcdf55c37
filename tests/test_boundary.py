"""The C-ABI boundary, host side only (no kernel is ever launched here).

* libmoe_ep.so loads and exports every function include/moe_ep.h declares;
* the workspace queries validate their scalars and size the workspace;
* every validation error of moe_dispatch / moe_combine is returned before any
  launch. The pointers passed here are fake addresses: each call below is
  rejected on the host by a check that runs before anything dereferences or
  launches, which is exactly the property under test.
"""
import ctypes
import os
import re

import pytest

import combine_ep_recv_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")

OK, NULLPTR, SHAPE, DTYPE, QUANT, WORKSPACE, LAUNCH, SCHEDULE, ALIGN, MASK = range(10)


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) == set(moe.EXPORTS), names
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(10):
        assert moe.status_str(s) and moe.status_str(s) != "unknown status"
    assert moe.status_str(99) == "unknown status"


def _ws(*args):
    n = ctypes.c_size_t(0)
    rc = moe.library().moe_dispatch_workspace_size(*args, ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("args,want", [
    ((8, 32, 8, 7168, 8, 1, 0), OK),
    ((16, 256, 16, 7168, 8, 2, 2), OK),
    ((2, 0, 1, 1, 1, 0, 0), OK),              # bs = 0 is valid
    ((768, 1, 1, 16, 1, 1, 0), OK),           # largest world
    ((8, 1, 128, 16, 8, 1, 0), OK),           # 1024 experts
    ((1, 8, 8, 16, 2, 0, 0), SHAPE),          # ep_world below 2
    ((769, 1, 1, 16, 1, 0, 0), SHAPE),        # ep_world above 768
    ((8, 1, 129, 16, 8, 0, 0), SHAPE),        # 1032 experts
    ((2, 4, 2, 16, 5, 0, 0), SHAPE),          # topk > experts
    ((2, 4, 2, 16, 0, 0, 0), SHAPE),          # topk 0
    ((2, -1, 2, 16, 1, 0, 0), SHAPE),         # negative bs
    ((2, 4, 2, 0, 1, 0, 0), SHAPE),           # h 0
    ((2, 4, 0, 16, 1, 0, 0), SHAPE),          # no experts
    ((512, 40000, 2, 16, 1, 0, 0), SHAPE),    # N beyond the launch limit
    ((64, 2048, 2, 65536, 1, 1, 0), SHAPE),   # N * ceil(h/128) beyond the slice-grid limit
    ((8, 2 ** 27, 8, 16, 8, 0, 0), SHAPE),    # N*K >= 2^31
    ((2, 4, 2, 16, 1, 3, 0), DTYPE),
    ((2, 4, 2, 16, 1, 1, 1), OK),             # static int8
    ((2, 4, 2, 16, 1, 0, 1), QUANT),          # int32 cannot be quantised
    ((2, 4, 2, 24, 1, 2, 1), QUANT),          # static needs h % 16 == 0
    ((2, 4, 2, 16400, 1, 1, 1), QUANT),       # ... and h <= 16384
    ((2, 4, 2, 16384, 1, 1, 1), OK),
    ((8, 4, 16, 64, 65, 1, 1), QUANT),        # ... and topk <= 64
    ((2, 4, 2, 16, 1, 1, -1), QUANT),
    ((2, 4, 2, 16, 1, 0, 2), QUANT),          # int32 cannot be quantised
    ((16, 256, 16, 7168, 8, 2, 3), OK),       # per-group FP8
    ((2, 4, 2, 16, 1, 0, 3), QUANT),
    ((2, 4, 2, 7176, 1, 2, 3), QUANT),        # per-group needs h % 16 == 0
    ((2, 4, 2, 16400, 1, 2, 3), QUANT),       # ... and h <= 16384
    ((2, 4, 2, 16384, 1, 2, 3), OK),
    ((8, 4, 16, 64, 65, 2, 3), QUANT),        # ... and topk <= 64
    ((2, 4, 2, 16, 1, 1, 4), OK),             # MX (MXFP8)
    ((16, 256, 16, 7168, 8, 2, 4), OK),
    ((2, 4, 2, 16, 1, 0, 4), QUANT),          # int32 cannot be quantised
    ((2, 4, 2, 7176, 1, 2, 4), QUANT),        # MX needs h % 16 == 0
    ((2, 4, 2, 16400, 1, 2, 4), QUANT),       # ... and h <= 16384
    ((8, 4, 16, 64, 65, 2, 4), QUANT),        # ... and topk <= 64
    ((2, 4, 2, 16, 1, 1, 5), QUANT),
])
def test_dispatch_workspace_query(args, want):
    rc, n = _ws(*args)
    assert rc == want, moe.status_str(rc)
    if rc == OK:
        assert n > 0 and n % 256 == 0


def test_workspace_grows_with_shape():
    a = _ws(8, 32, 8, 7168, 8, 1, 0)[1]
    b = _ws(16, 256, 16, 7168, 8, 2, 2)[1]
    assert b > a


def test_combine_workspace_query():
    n = ctypes.c_size_t(7)
    lib = moe.library()
    assert lib.moe_combine_workspace_size(8, 32, 8, 7168, 8, 1, ctypes.byref(n)) == OK
    assert n.value == 8 * 32 * 8 * 4
    assert lib.moe_combine_workspace_size(1, 32, 8, 7168, 8, 1, ctypes.byref(n)) == SHAPE
    assert lib.moe_combine_workspace_size(8, 32, 8, 7168, 8, 5, ctypes.byref(n)) == DTYPE
    assert lib.moe_combine_workspace_size(8, 32, 8, 7168, 8, 1, None) == NULLPTR
    assert lib.moe_dispatch_workspace_size(8, 32, 8, 7168, 8, 1, 0, None) == NULLPTR


A = 1 << 20   # fake, 256-aligned "device" addresses; never dereferenced by these calls


def _dispatch(**kw):
    p = dict(x=A, ids=2 * A, esc=None, mask=None, mk=0, sp=None, W=2, bs=4, epr=2, h=16, K=2, dtype=1, quant=0,
             qs=None, qn=0, ex=3 * A, dyn=None, assist=4 * A, erc=5 * A, esc_out=None, sched=None, ws=6 * A,
             wsb=1 << 30)
    p.update(kw)
    P = lambda v: None if v is None else ctypes.c_void_p(v)
    return moe.library().moe_dispatch(
        P(p["x"]), P(p["ids"]), P(p["esc"]), P(p["mask"]), p["mk"],
        ctypes.byref(p["sp"]) if p["sp"] is not None else None, p["W"], p["bs"], p["epr"], p["h"], p["K"],
        p["dtype"], p["quant"], P(p["qs"]), ctypes.c_int64(p["qn"]),
        P(p["ex"]), P(p["dyn"]), P(p["assist"]), P(p["erc"]), P(p["esc_out"]),
        ctypes.byref(p["sched"]) if p["sched"] is not None else None, P(p["ws"]), p["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(W=1), SHAPE),
    (dict(K=5), SHAPE),
    (dict(dtype=7), DTYPE),
    (dict(quant=5), QUANT),
    (dict(quant=4), NULLPTR),                        # MX needs its scale bytes
    (dict(dtype=0, quant=4, dyn=7 * A), QUANT),
    (dict(quant=4, dyn=7 * A + 1, sched=moe.MoeSchedule(mode=1)), SCHEDULE),   # MX: token schedule only
    (dict(quant=4, dyn=7 * A + 1, x=A + 2), ALIGN),                         # MX: 16-byte rows
    (dict(quant=3), NULLPTR),                        # per-group quantising needs dynamic_scales
    (dict(dtype=0, quant=2, dyn=7 * A), QUANT),
    (dict(x=None), NULLPTR),
    (dict(ids=None), NULLPTR),
    (dict(ex=None), NULLPTR),
    (dict(assist=None), NULLPTR),
    (dict(erc=None), NULLPTR),
    (dict(ws=None), NULLPTR),
    (dict(quant=2), NULLPTR),                        # quantising needs dynamic_scales
    (dict(dyn=7 * A), NULLPTR),                      # ... and forbids it otherwise
    (dict(esc_out=7 * A), NULLPTR),                  # expand_scales needs expert_scales
    (dict(wsb=16), WORKSPACE),
    (dict(x=A + 1), ALIGN),                          # fp16 tokens at an odd address
    (dict(ids=2 * A + 2), ALIGN),
    (dict(erc=5 * A + 2), ALIGN),
    (dict(ws=6 * A + 8), ALIGN),
    (dict(sched=moe.MoeSchedule(mode=5)), SCHEDULE),
    (dict(W=128, epr=8, K=2, sched=moe.MoeSchedule(mode=1)), SCHEDULE),   # W*S = 131072 > LDS budget
    (dict(quant=3, dyn=7 * A, sched=moe.MoeSchedule(mode=1)), SCHEDULE),  # per-group: token schedule only
    (dict(quant=3, dyn=7 * A, x=A + 2), ALIGN),                           # per-group: 16-byte rows
    (dict(quant=1), NULLPTR),                                  # static needs its coefficients
    (dict(quant=1, qs=8 * A, qn=3), QUANT),                    # 1, h (16) or E*h (64) of them
    (dict(quant=1, qs=8 * A, qn=32), QUANT),
    (dict(quant=1, qs=8 * A, qn=16, dyn=7 * A), NULLPTR),      # and writes no dynamic scales
    (dict(qs=8 * A, qn=16), NULLPTR),                          # coefficients only for quant mode 1
    (dict(qn=16), NULLPTR),
    (dict(quant=2, dyn=7 * A, qs=8 * A, qn=1), NULLPTR),
    (dict(quant=1, qs=8 * A + 4, qn=64), ALIGN),               # h or E*h values: 16-byte aligned
    (dict(quant=1, qs=8 * A + 2, qn=1), ALIGN),                # one value: 4-byte aligned
    (dict(quant=1, qs=8 * A, qn=1, sched=moe.MoeSchedule(mode=1)), SCHEDULE),   # token schedule only
    (dict(quant=1, qs=8 * A, qn=1, x=A + 2), ALIGN),           # 16-byte rows
    (dict(sp=moe.MoeSpecialExperts(zero_expert_num=-1)), SHAPE),
    (dict(sp=moe.MoeSpecialExperts(const_expert_num=-1)), SHAPE),
    (dict(sp=moe.MoeSpecialExperts(zero_expert_num=2 ** 31 - 4)), SHAPE),   # E + zero = 2^31
    (dict(sp=moe.MoeSpecialExperts(copy_expert_num=2 ** 30, const_expert_num=2 ** 30 - 4)), SHAPE),   # 2^31 ids
    (dict(mk=3, mask=8 * A), MASK),                                     # unknown mask kind
    (dict(mk=1), MASK),                                                 # a kind without a mask
    (dict(mask=8 * A), MASK),                                           # a mask without a kind
])
def test_dispatch_rejects_before_launch(kw, want):
    rc = _dispatch(**kw)
    assert rc == want, (kw, rc, moe.status_str(rc))


def _combine(**kw):
    p = dict(ex=A, assist=2 * A, erc=3 * A, ids=4 * A, sc=5 * A, mask=None, mk=0, sp=None, W=2, bs=4, epr=2, h=16,
             K=2, dtype=1, out=6 * A, ws=7 * A, wsb=1 << 30)
    p.update(kw)
    P = lambda v: None if v is None else ctypes.c_void_p(v)
    return moe.library().moe_combine(P(p["ex"]), P(p["assist"]), P(p["erc"]), P(p["ids"]), P(p["sc"]),
                                     P(p["mask"]), p["mk"], ctypes.byref(p["sp"]) if p["sp"] is not None else None,
                                     p["W"],
                                     p["bs"], p["epr"], p["h"], p["K"], p["dtype"], P(p["out"]), P(p["ws"]),
                                     p["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(W=769), SHAPE),
    (dict(h=0), SHAPE),
    (dict(dtype=-1), DTYPE),
    (dict(ex=None), NULLPTR),
    (dict(assist=None), NULLPTR),
    (dict(erc=None), NULLPTR),
    (dict(ids=None), NULLPTR),
    (dict(sc=None), NULLPTR),
    (dict(out=None), NULLPTR),
    (dict(ws=None), NULLPTR),
    (dict(wsb=8 * 4 * 2 - 1), WORKSPACE),
    (dict(ex=A + 1), ALIGN),
    (dict(ws=7 * A + 4), ALIGN),
    (dict(out=6 * A + 1), ALIGN),
    (dict(dtype=0, ex=A + 2), ALIGN),
    (dict(bs=0), OK),                                # empty batch: nothing to launch
    (dict(sp=moe.MoeSpecialExperts(copy_expert_num=2)), NULLPTR),      # copy experts need ori_x
    (dict(sp=moe.MoeSpecialExperts(copy_expert_num=2, ori_x=8 * A + 1)), ALIGN),
    (dict(sp=moe.MoeSpecialExperts(const_expert_num=3)), NULLPTR),     # const experts need their outputs
    (dict(sp=moe.MoeSpecialExperts(const_expert_num=3, const_x=8 * A + 1)), ALIGN),
    (dict(sp=moe.MoeSpecialExperts(const_expert_num=-1, const_x=8 * A)), SHAPE),
    (dict(sp=moe.MoeSpecialExperts(zero_expert_num=1, const_expert_num=2 ** 31 - 5, const_x=8 * A)), SHAPE),
    (dict(mk=-1), MASK),
    (dict(mk=2), MASK),                              # a kind without a mask
    (dict(mask=8 * A), MASK),                        # a mask without a kind
])
def test_combine_rejects_before_launch(kw, want):
    rc = _combine(**kw)
    assert rc == want, (kw, rc, moe.status_str(rc))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "combine_ep_recv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".hpp", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text and "moe_oracle" not in text, f
