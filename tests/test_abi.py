"""The C ABI library without a GPU: it loads, exports every declared entry point, and rejects
bad arguments before enqueueing anything (these calls never reach a HIP API)."""
import ctypes
import os
import re

import pytest

import post_weight_quantization_group_amd as cq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_binding_names():
    assert sorted(cq.EXPORTED_SYMBOLS) == _declared()


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(cq.library_path())
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert cq.cq_abi_version() == 2
    assert cq.cq_status_string(0) == "ok"
    assert "workspace" in cq.cq_status_string(-2)
    assert cq.cq_status_string(123) == "unknown status"


def test_workspace_sizes():
    assert cq.cq_workspace_size(cq.EXHAUSTIVE, 4, 0) >= 256
    assert cq.cq_workspace_size(cq.EXHAUSTIVE, 4, 1000) >= 4000
    assert cq.cq_workspace_size(cq.CANDIDATE, 4, 1000) > cq.cq_workspace_size(cq.EXHAUSTIVE, 4, 1000)
    assert cq.cq_workspace_size(cq.EXHAUSTIVE, 0, 10) == 0
    assert cq.cq_workspace_size(cq.EXHAUSTIVE, 33, 10) == 0
    assert cq.cq_workspace_size(7, 4, 10) == 0
    assert cq.cq_workspace_size(cq.BOUNDED, 4, 1000) == cq.cq_workspace_size(cq.EXHAUSTIVE, 4, 1000)
    assert cq.cq_proxy_workspace_size(10) >= 80


FAKE = 1 << 20  # a 16-byte-aligned address that is never dereferenced: every call below fails its checks


def _quant(**kw):
    lib = cq.load()
    a = dict(w=FAKE, d=FAKE, d_period=1, E=4, n=10, method=0, scales=FAKE, codes=None, obj=None, flags=None,
             ps=None, po=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.cq_quantize_groups(a["w"], a["d"], a["d_period"], a["E"], a["n"], a["method"], a["scales"],
                                  a["codes"], a["obj"], a["flags"], a["ps"], a["po"], a["ws"], a["wsb"],
                                  a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), -1), (dict(E=33), -1), (dict(n=-1), -1), (dict(d_period=0), -1), (dict(w=None), -1),
    (dict(d=None), -1), (dict(scales=None), -1), (dict(method=5), -1), (dict(w=FAKE + 4), -1),
    (dict(method=1, ps=FAKE), -4), (dict(ws=None), -2), (dict(ws=FAKE, wsb=16), -2),
    (dict(ws=FAKE + 16, wsb=1 << 20), -2),
])
def test_quantize_rejects_before_launch(kw, status):
    assert _quant(**kw) == status


def _spec(**kw):
    lib = cq.load()
    a = dict(w=FAKE, d=FAKE, G=64, qmin=-4, qmax=3, d_period=1, E=4, n=10, method=0, scales=FAKE, ws=FAKE,
             wsb=1 << 20)
    a.update(kw)
    return lib.cq_quantize_groups_spec(a["w"], a["d"], a["G"], a["qmin"], a["qmax"], a["d_period"], a["E"], a["n"],
                                       a["method"], a["scales"], None, None, None, a.get("ps"), None, a["ws"],
                                       a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), -1), (dict(G=257), -1), (dict(qmin=1), -1), (dict(qmax=-1), -1), (dict(qmin=0, qmax=0), -1),
    (dict(qmin=-129), -1), (dict(qmax=128), -1), (dict(method=3), -1), (dict(method=2), -4),
    # the candidate solver takes at most 8 codes on each side of zero and groups of at most 128
    (dict(method=1, qmin=-9), -4), (dict(method=1, qmax=9), -4), (dict(method=1, G=129), -4),
    (dict(method=1, qmin=-16, qmax=15, G=256), -4), (dict(method=1, ps=FAKE), -4),
    (dict(method=1, ws=None), -2), (dict(method=1, w=FAKE + 2), -1),
    (dict(w=FAKE + 2), -1), (dict(E=33), -1), (dict(scales=None), -1), (dict(ws=None), -2),
    (dict(ws=FAKE, wsb=16), -2), (dict(n=0, w=None, d=None, scales=None), 0),
    # the pages' quantizer through the spec entry takes cq_quantize_groups' checks (16-byte alignment)
    (dict(G=128, qmin=-8, qmax=7, w=FAKE + 4), -1), (dict(G=128, qmin=-8, qmax=7, method=5), -1),
])
def test_quantize_spec_rejects_before_launch(kw, status):
    assert _spec(**kw) == status


def test_zero_groups_is_a_no_op():
    assert _quant(n=0, w=None, d=None, scales=None) == 0


def test_other_entry_points_reject_bad_arguments():
    lib = cq.load()
    assert lib.cq_pack_gptq_v1(FAKE, FAKE, 4, 100, FAKE, FAKE, None) == -1          # in % 128
    assert lib.cq_pack_gptq_v1(FAKE + 1, FAKE, 4, 128, FAKE, FAKE, None) == -1      # codes alignment
    assert lib.cq_pack_gptq_v1(None, FAKE, 4, 128, FAKE, FAKE, None) == -1
    assert lib.cq_pack_gptq_v1(None, None, 0, 128, None, None, None) == 0           # empty
    assert lib.cq_baseline_scales(FAKE, FAKE, 1, 4, 10, 9, FAKE, None, None, None, 0, None) == -1
    assert lib.cq_baseline_scales(FAKE, FAKE, 1, 4, 10, 1, FAKE, None, None, None, 0, None) == -2
    assert lib.cq_baseline_scales(FAKE, None, 1, 4, 10, 0, FAKE, None, FAKE, None, 0, None) == -1
    assert lib.cq_proxy_worst_env_wmse(FAKE, FAKE, 1, 4, 10, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, 0,
                                       None) == -1
    assert lib.cq_proxy_worst_env_wmse(FAKE, FAKE, 1, 4, 10, FAKE, FAKE, 2, FAKE, FAKE, None, None, 0,
                                       None) == -2
    assert lib.cq_baseline_scales(FAKE, FAKE, 1, 4, 10, 0, FAKE, FAKE + 8, None, None, 0, None) == -1  # codes


def test_pack_multi_rejects_bad_arguments():
    lib = cq.load()
    f = lib.cq_pack_gptq_v1_multi
    import ctypes as C

    def arr(*v):
        return C.cast((C.c_int64 * len(v))(*v), C.c_void_p)
    assert f(FAKE, FAKE, -1, arr(4), arr(128), FAKE, FAKE, None) == -1
    assert f(FAKE, FAKE, 257, arr(4), arr(128), FAKE, FAKE, None) == -1          # too many matrices
    assert f(FAKE, FAKE, 2, arr(4, 4), arr(128, 100), FAKE, FAKE, None) == -1    # in % 128
    assert f(FAKE, FAKE, 1, arr(-1), arr(128), FAKE, FAKE, None) == -1
    assert f(FAKE, FAKE, 1, None, arr(128), FAKE, FAKE, None) == -1
    assert f(FAKE + 1, FAKE, 1, arr(4), arr(128), FAKE, FAKE, None) == -1        # codes alignment
    assert f(None, FAKE, 1, arr(4), arr(128), FAKE, FAKE, None) == -1
    assert f(None, None, 0, None, None, None, None, None) == 0                   # nothing to pack
    assert f(None, None, 2, arr(0, 0), arr(128, 256), None, None, None) == 0     # empty matrices


def test_multi_policy_proxy_rejects_bad_arguments():
    lib = cq.load()
    f = lib.cq_proxy_worst_env_wmse_multi
    assert f(FAKE, FAKE, 1, 4, 10, 0, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 0, None) == -1     # no policy
    assert f(FAKE, FAKE, 1, 4, 10, 65, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 0, None) == -1    # too many
    assert f(FAKE, FAKE, 1, 4, 10, 3, None, FAKE, 1, FAKE, FAKE, FAKE, None, 0, None) == -1     # no scales
    assert f(FAKE, FAKE, 1, 4, 10, 3, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, 0, None) == -1     # no module
    assert f(FAKE, FAKE, 1, 4, 10, 3, FAKE, FAKE, 1, FAKE, FAKE, FAKE + 4, None, 0, None) == -1  # per_group
    # without per_group the workspace must hold n_policies * n_groups values
    # (100 groups x 3 policies x 8 bytes = 2,400 > 2,048)
    assert f(FAKE, FAKE, 1, 4, 100, 3, FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 2048, None) == -2


def test_heldout_compare_rejects_bad_arguments():
    lib = cq.load()
    f = lib.cq_heldout_compare
    ws = cq.cq_heldout_workspace_size(10, 2)
    assert ws >= (11 * 2 + 10) * 8
    ok = dict(pa=FAKE, pb=FAKE, n=100, off=FAKE, M=2, idx=FAKE, B=10, alpha=0.05, counts=FAKE, effect=FAKE,
              boot=FAKE, ci=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["pa"], a["pb"], a["n"], a["off"], a["M"], a["idx"], a["B"], a["alpha"], a["counts"],
                 a["effect"], a["boot"], a["ci"], a["ws"], a["wsb"], None)

    assert call(alpha=0.0) == -1 and call(alpha=1.0) == -1
    assert call(M=0) == -1 and call(B=-1) == -1 and call(n=-1) == -1
    assert call(pa=None) == -1 and call(off=None) == -1 and call(ci=None) == -1
    assert call(idx=None) == -1 and call(boot=None) == -1 and call(pa=FAKE + 4) == -1
    assert call(ws=None) == -2 and call(wsb=ws - 8) == -2 and call(ws=FAKE + 64) == -2


def test_environment_diagonals_rejects_bad_arguments():
    lib = cq.load()
    f = lib.cq_environment_diagonals
    ws = cq.cq_diagonals_workspace_size(4, 100, 256)
    assert ws >= 4 * 256 * 8 and cq.cq_diagonals_workspace_size(4, 100, 200) == 0
    assert f(FAKE, 0, 100, 256, FAKE, FAKE, ws, None) == -1       # E
    assert f(FAKE, 33, 100, 256, FAKE, FAKE, ws, None) == -1
    assert f(FAKE, 4, 0, 256, FAKE, FAKE, ws, None) == -1         # T
    assert f(FAKE, 4, 100, 200, FAKE, FAKE, ws, None) == -1       # in % 128
    assert f(FAKE + 8, 4, 100, 256, FAKE, FAKE, ws, None) == -1   # x alignment
    assert f(FAKE, 4, 100, 256, None, FAKE, ws, None) == -1
    assert f(FAKE, 4, 100, 256, FAKE, None, ws, None) == -2
    assert f(FAKE, 4, 100, 256, FAKE, FAKE, ws - 8, None) == -2


def test_w4a16_matmul_rejects_bad_arguments():
    lib = cq.load()
    f = lib.cq_w4a16_matmul
    assert f(FAKE, FAKE, FAKE, 4, 64, 100, FAKE, None) == -1          # in % 128
    assert f(FAKE + 8, FAKE, FAKE, 4, 64, 128, FAKE, None) == -1      # x alignment
    assert f(FAKE, None, FAKE, 4, 64, 128, FAKE, None) == -1
    assert f(FAKE, FAKE, FAKE, 64 * 65536, 64, 128, FAKE, None) == -1  # M beyond the grid
    assert f(None, None, None, 0, 64, 128, None, None) == 0           # empty


def test_pack_spec_rejects_bad_arguments():
    f = cq.load().cq_pack_gptq_v1_spec
    assert f(FAKE, FAKE, 4, 128, 3, 128, FAKE, FAKE, None) == -1         # field width
    assert f(FAKE, FAKE, 4, 128, 4, 0, FAKE, FAKE, None) == -1           # group length
    assert f(FAKE, FAKE, 4, 128, 4, 257, FAKE, FAKE, None) == -1
    assert f(FAKE, FAKE, 4, 96, 4, 64, FAKE, FAKE, None) == -1           # in % group_len
    assert f(FAKE, FAKE, 4, 24, 2, 8, FAKE, FAKE, None) == -1            # in % (32 / bits)
    assert f(FAKE, FAKE, -1, 128, 4, 128, FAKE, FAKE, None) == -1
    assert f(FAKE + 2, FAKE, 4, 128, 8, 32, FAKE, FAKE, None) == -1      # codes alignment
    assert f(FAKE, FAKE + 1, 4, 128, 8, 32, FAKE, FAKE, None) == -1      # scales alignment
    assert f(None, FAKE, 4, 128, 8, 32, FAKE, FAKE, None) == -1
    assert f(None, None, 0, 128, 2, 16, None, None, None) == 0           # empty


def test_spec_baseline_and_proxy_reject_bad_arguments():
    lib = cq.load()
    b = lib.cq_baseline_scales_spec
    assert b(FAKE, FAKE, 0, -4, 3, 1, 4, 10, 0, FAKE, None, None, None, 0, None) == -1       # group length
    assert b(FAKE, FAKE, 64, 1, 3, 1, 4, 10, 0, FAKE, None, None, None, 0, None) == -1       # qmin > 0
    assert b(FAKE, FAKE, 64, -4, 0, 1, 4, 10, 0, FAKE, None, None, None, 0, None) == -1      # AbsMax, qmax 0
    assert b(FAKE, FAKE, 64, -4, 3, 1, 4, 10, 5, FAKE, None, None, None, 0, None) == -1      # which
    assert b(FAKE, FAKE, 64, -4, 3, 1, 4, 10, 1, FAKE, None, None, None, 0, None) == -2      # pooled: workspace
    assert b(FAKE + 2, FAKE, 64, -4, 3, 1, 4, 10, 0, FAKE, None, None, None, 0, None) == -1  # w alignment
    assert b(FAKE, FAKE, 64, -4, 3, 1, 4, 0, 0, None, None, None, None, 0, None) == 0         # empty
    p = lib.cq_proxy_worst_env_wmse_multi_spec
    assert p(FAKE, FAKE, 300, -4, 3, 1, 4, 10, 1, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert p(FAKE, FAKE, 64, -4, 3, 1, 4, 10, 0, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 0, None) == -1  # policies
    assert p(FAKE, FAKE, 64, -4, 3, 1, 4, 10, 1, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, 0, None) == -1  # modules
    assert p(FAKE, FAKE, 64, -4, 3, 1, 4, 10, 1, FAKE, FAKE, 1, FAKE, FAKE, None, None, 0, None) == -2  # workspace
    assert p(FAKE, FAKE, 64, -4, 3, 1, 33, 10, 1, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 0, None) == -1  # E


def test_probe_rejects_bad_arguments():
    f = cq.load().cq_probe_valu_fma
    import ctypes
    hz = ctypes.c_double(0.0)
    assert f(0, 8, 1, FAKE, FAKE, ctypes.byref(hz), None) == -1      # iters < 1
    assert f(10, 0, 1, FAKE, FAKE, ctypes.byref(hz), None) == -1     # blocks < 1
    assert f(10, 8, 3, FAKE, FAKE, ctypes.byref(hz), None) == -1     # mode
    assert f(10, 8, -1, FAKE, FAKE, ctypes.byref(hz), None) == -1
    assert f(10, 8, 1, None, FAKE, ctypes.byref(hz), None) == -1     # out
    assert f(10, 8, 1, FAKE, None, ctypes.byref(hz), None) == -1     # clocks
    assert f(10, 8, 1, FAKE, FAKE, None, None) == -1                 # wall_clock_hz
