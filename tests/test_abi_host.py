"""The C ABI on the host: the library loads, exports every symbol that
include/*.h declare, sizes workspaces, and rejects bad arguments before
anything reaches a GPU (every call here fails validation, so no HIP call is
made)."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from block_quantized_expert_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared_functions():
    names = set()
    for fn in sorted(os.listdir(INCLUDE)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(B.EXPORTED) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    for s in range(5):
        assert B.status_string(s).startswith("MOE_")
    assert "unknown" in B.status_string(99)


def test_struct_layout_matches_c():
    # int32 x4, 3 x {int32 type; 2 pointers}, int32 x2, 3 x proj
    assert ctypes.sizeof(B.MoeProj) == 24
    assert B.MoeLayer.gate.offset == 16
    assert B.MoeLayer.has_shared.offset == 88
    assert B.MoeLayer.packed_experts.offset == 168
    assert ctypes.sizeof(B.MoeLayer) == 176


FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p(0x10004)


def _layer(hidden=4096, inter=2048, e=256, k=6, shared=True, wtype=0, swtype=0, codes=FAKE):
    L = B.MoeLayer()
    L.hidden, L.inter, L.n_experts, L.top_k = hidden, inter, e, k
    for name in ("gate", "up", "down"):
        setattr(L, name, B.MoeProj(wtype, codes.value, FAKE.value))
    L.has_shared = 1 if shared else 0
    if shared:
        L.shared_inter = inter
        for name in ("shared_gate", "shared_up", "shared_down"):
            setattr(L, name, B.MoeProj(swtype, FAKE.value, FAKE.value))
    return L


def test_ffn_workspace_bytes():
    L = _layer()
    n = 4096
    slots = n * 6 + n
    h = -(-slots * 2048 * 2 // 256) * 256
    o = -(-slots * 4096 * 3 // 256) * 256  # per-slot outputs, 24-bit floats
    xq = n * 4096 * 2          # activations as two E4M3 parts
    xs = n * 4096 // 16        # their scale bytes
    gmax = n * 6 * 4           # lazy skip: each routed slot's largest |SiLU(g)|
    qctr = 256                 # item-queue counters of the grouped GEMMs
    h6 = slots * 64 * 72 + 256 + slots * 64 * 4  # h in E2M3 parts (+ padding) for the packed down
    assert B.lib().moe_ffn_workspace_bytes(ctypes.byref(L), n) == \
        2 * h + o + xq + xs + gmax + qctr + h6
    # up to 16 tokens: also the gate outputs of the gate-first lazy pass
    n = 16
    slots = n * 6 + n
    h = -(-slots * 2048 * 2 // 256) * 256
    o = -(-slots * 4096 * 3 // 256) * 256  # per-slot outputs, 24-bit floats
    xs = -(-n * 4096 // 16 // 256) * 256
    gmax = -(-n * 6 * 4 // 256) * 256
    gbuf = n * 6 * 2048 * 4
    # (16 tokens x 6 slots: too few per expert for the E2M3 parts)
    assert B.lib().moe_ffn_workspace_bytes(ctypes.byref(L), n) == \
        2 * h + o + n * 4096 * 2 + xs + gmax + 256 + gbuf
    # the E2M3 parts from 16 slots per routed expert on
    L16 = _layer(e=16, k=2)
    for n, with_h6 in ((127, False), (128, True)):
        slots = n * 2 + n
        h6 = -(-(slots * 64 * 72 + 16) // 256) * 256 + -(-slots * 64 * 4 // 256) * 256
        plain = B.lib().moe_ffn_workspace_bytes(ctypes.byref(L16), n)
        assert plain > 0
        L16.gate = B.MoeProj(1, FAKE.value, FAKE.value)  # fp8 routed experts: no E2M3 parts
        L16.up = L16.down = L16.gate
        fp8 = B.lib().moe_ffn_workspace_bytes(ctypes.byref(L16), n)
        L16 = _layer(e=16, k=2)
        assert plain - fp8 == (h6 if with_h6 else 0)
    assert B.lib().moe_ffn_workspace_bytes(ctypes.byref(L), 0) == 0
    assert B.lib().moe_ffn_workspace_bytes(ctypes.byref(_layer(hidden=100)), 8) == 0
    assert B.lib().moe_ffn_workspace_bytes(None, 8) == 0
    assert B.lib().moe_group_workspace_bytes(8, 2, 16) == 0


def _ffn(L, x=FAKE, x_type=1, n=4, ws=FAKE, ws_bytes=1 << 40, y=FAKE, w=FAKE):
    return B.lib().moe_ffn_forward(ctypes.byref(L) if L is not None else None, x, x_type, n, w,
                                   FAKE, FAKE, FAKE, FAKE, y, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,layer_kwargs,expected", [
    ({"x": None}, {}, B.MOE_ERR_INVALID),
    ({"x": MIS}, {}, B.MOE_ERR_INVALID),
    ({"y": MIS}, {}, B.MOE_ERR_INVALID),
    ({"w": None}, {}, B.MOE_ERR_INVALID),
    ({"n": -1}, {}, B.MOE_ERR_INVALID),
    ({"n": (1 << 22) + 1}, {}, B.MOE_ERR_UNSUPPORTED),
    ({"x_type": 7}, {}, B.MOE_ERR_UNSUPPORTED),
    ({"ws": None}, {}, B.MOE_ERR_WORKSPACE),
    ({"ws_bytes": 1000}, {}, B.MOE_ERR_WORKSPACE),
    ({"ws": MIS}, {}, B.MOE_ERR_INVALID),
    ({}, {"hidden": 4000}, B.MOE_ERR_UNSUPPORTED),
    ({}, {"inter": 96}, B.MOE_ERR_UNSUPPORTED),
    ({}, {"hidden": 0}, B.MOE_ERR_INVALID),
    ({}, {"k": 9, "e": 16}, B.MOE_ERR_UNSUPPORTED),
    ({}, {"k": 17, "e": 16}, B.MOE_ERR_INVALID),
    ({}, {"e": 2000}, B.MOE_ERR_UNSUPPORTED),
    ({}, {"wtype": 5}, B.MOE_ERR_UNSUPPORTED),
    ({}, {"codes": MIS}, B.MOE_ERR_INVALID),
    ({}, {"swtype": 3}, B.MOE_ERR_UNSUPPORTED),
])
def test_ffn_rejects_bad_arguments(kwargs, layer_kwargs, expected):
    assert _ffn(_layer(**layer_kwargs), **kwargs) == expected


def test_ffn_null_layer_and_mixed_types():
    assert _ffn(None) == B.MOE_ERR_INVALID
    L = _layer()
    L.down = B.MoeProj(1, FAKE.value, FAKE.value)  # gate mxfp4, down fp8
    assert _ffn(L) == B.MOE_ERR_UNSUPPORTED
    L = _layer()
    L.has_shared = 2
    assert _ffn(L) == B.MOE_ERR_INVALID
    L = _layer()
    L.shared_inter = 0
    assert _ffn(L) == B.MOE_ERR_INVALID
    L = _layer()
    L.shared_up = B.MoeProj(0, 0, FAKE.value)
    assert _ffn(L) == B.MOE_ERR_INVALID
    # scale bytes are read with 16-byte loads and copies
    L = _layer()
    L.up = B.MoeProj(0, FAKE.value, FAKE.value + 4)
    assert _ffn(L) == B.MOE_ERR_INVALID
    L = _layer(swtype=1)
    L.shared_down = B.MoeProj(1, FAKE.value, FAKE.value + 1)
    assert _ffn(L) == B.MOE_ERR_INVALID


def test_ffn_zero_tokens_is_a_no_op():
    assert _ffn(_layer(), n=0, x=None, ws=None, y=None) == B.MOE_OK


def test_route_rejects_bad_arguments():
    R = B.lib().moe_route
    assert R(None, 4, 256, 6, 1.5, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert R(FAKE, 4, 256, 6, 0.0, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert R(FAKE, 4, 256, 6, float("nan"), FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert R(FAKE, 4, 256, 6, float("inf"), FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert R(FAKE, 4, 4, 6, 1.5, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert R(FAKE, 4, 256, 9, 1.5, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert R(FAKE, 4, 1025, 6, 1.5, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert R(FAKE, -1, 256, 6, 1.5, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert R(FAKE, 4, 256, 0, 1.5, FAKE, FAKE, None) == B.MOE_ERR_INVALID
    assert R(None, 0, 256, 6, 1.5, None, None, None) == B.MOE_OK  # nothing to do


def test_route_hash_and_group_reject_bad_arguments():
    H = B.lib().moe_route_hash
    assert H(FAKE, 4, FAKE, FAKE, 0, 256, 6, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID
    assert H(FAKE, 4, None, FAKE, 100, 256, 6, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID
    assert H(FAKE, 4, FAKE, FAKE, 100, 256, 9, FAKE, FAKE, None, None) == B.MOE_ERR_UNSUPPORTED
    G = B.lib().moe_group
    assert G(FAKE, 4, 6, 256, None, FAKE, FAKE, FAKE, None, None, 0, None) == B.MOE_ERR_INVALID
    assert G(FAKE, 4, 6, 256, FAKE, FAKE, None, FAKE, None, None, 0, None) == B.MOE_ERR_INVALID
    assert G(FAKE, 4, 6, 2048, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == B.MOE_ERR_UNSUPPORTED
    assert G(FAKE, 4, 9, 256, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == B.MOE_ERR_UNSUPPORTED
    assert G(FAKE, 4, 300, 256, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == B.MOE_ERR_INVALID
    RG = B.lib().moe_route_group
    assert RG(FAKE, 4, 256, 6, 1.5, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == \
        B.MOE_ERR_INVALID
    assert RG(FAKE, 4, 256, 6, -1.5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == \
        B.MOE_ERR_INVALID
    assert RG(FAKE, 4, 256, 9, 1.5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == \
        B.MOE_ERR_UNSUPPORTED


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_validator_under_address_and_ub_sanitizers(tmp_path):
    # The pure-host validator, built with ASan + UBSan and driven through its
    # accept and reject paths.
    csrc = os.path.join(ROOT, "block_quantized_expert_amd", "csrc")
    exe = str(tmp_path / "validator")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
           os.path.join(csrc, "moe_host.cpp"),
           os.path.join(ROOT, "tests", "native", "validator_main.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validator ok" in r.stdout


def test_forward_workspace_bytes():
    lib = B.lib()
    for n in (1, 7, 4096):
        L = _layer()
        ffn = lib.moe_ffn_workspace_bytes(ctypes.byref(L), n)
        assert lib.moe_forward_workspace_bytes(ctypes.byref(L), n) == \
            B.MOE_FORWARD_SYNC_BYTES + -(-ffn // 256) * 256
    assert lib.moe_forward_workspace_bytes(ctypes.byref(_layer(hidden=100)), 1) == 0
    assert lib.moe_forward_workspace_bytes(None, 1) == 0


@pytest.mark.parametrize("layer_kwargs,n,x_type,expected", [
    ({}, 1, B.MOE_ACT_BF16, 1),                         # the decode layer: one kernel
    ({"hidden": 512, "inter": 128, "e": 16, "k": 2}, 1, B.MOE_ACT_BF16, 1),
    ({"inter": 384, "shared": False}, 1, B.MOE_ACT_BF16, 1),
    ({}, 2, B.MOE_ACT_BF16, 0),                         # more than one token
    ({}, 1, B.MOE_ACT_F32, 0),                          # fp32 activations
    ({"hidden": 640}, 1, B.MOE_ACT_BF16, 0),            # hidden not a multiple of 512
    ({"hidden": 8192}, 1, B.MOE_ACT_BF16, 0),           # x no longer fits the staging
    ({"inter": 4224}, 1, B.MOE_ACT_BF16, 0),            # down scales no longer fit the staging
    ({"wtype": 1}, 1, B.MOE_ACT_BF16, 0),               # fp8 routed experts
    ({"swtype": 1}, 1, B.MOE_ACT_BF16, 0),              # fp8 shared expert
    ({"e": 512}, 1, B.MOE_ACT_BF16, 0),                 # more experts than the router wave holds
    ({"hidden": 100}, 1, B.MOE_ACT_BF16, -1),           # invalid layer
])
def test_forward_path_choice(layer_kwargs, n, x_type, expected):
    L = _layer(**layer_kwargs)
    assert B.lib().moe_forward_single_kernel(ctypes.byref(L), n, x_type) == expected


def test_forward_path_choice_shared_width():
    L = _layer()
    L.shared_inter = 1024  # shared expert narrower than the routed ones
    assert B.lib().moe_forward_single_kernel(ctypes.byref(L), 1, B.MOE_ACT_BF16) == 0


def _fwd(L, logits=FAKE, scale=1.5, x=FAKE, n=1, ids=FAKE, ws=FAKE, ws_bytes=1 << 40, y=FAKE):
    return B.lib().moe_forward(ctypes.byref(L) if L is not None else None, logits, scale, x,
                               B.MOE_ACT_BF16, n, ids, FAKE, FAKE, FAKE, FAKE, FAKE, y, ws,
                               ws_bytes, None, None)


@pytest.mark.parametrize("kwargs,expected", [
    ({"logits": None}, B.MOE_ERR_INVALID),
    ({"ids": None}, B.MOE_ERR_INVALID),
    ({"x": None}, B.MOE_ERR_INVALID),
    ({"y": MIS}, B.MOE_ERR_INVALID),
    ({"scale": 0.0}, B.MOE_ERR_INVALID),
    ({"ws": None}, B.MOE_ERR_WORKSPACE),
    ({"ws_bytes": B.MOE_FORWARD_SYNC_BYTES}, B.MOE_ERR_WORKSPACE),
    ({"ws": MIS}, B.MOE_ERR_INVALID),
])
def test_forward_rejects_bad_arguments(kwargs, expected):
    assert _fwd(_layer(), **kwargs) == expected


def test_forward_workspace_init_rejects_small_areas():
    lib = B.lib()
    assert lib.moe_forward_workspace_init(None, 1 << 20, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_forward_workspace_init(FAKE, B.MOE_FORWARD_SYNC_BYTES - 1, None) == \
        B.MOE_ERR_WORKSPACE


def test_opts_rejected_before_launch():
    lib = B.lib()
    P = ctypes.c_void_p
    bad = [dict(n_group=3),                    # does not divide 256 experts
           dict(n_group=128),                  # more than 64 groups
           dict(n_group=8, topk_group=9),      # more groups kept than exist
           dict(n_group=64, topk_group=1),     # 4 experts in the kept group < top-6
           dict(n_group=-1),
           dict(keep_max=7),                   # above top_k
           dict(keep_max=-1),
           dict(min_w=-0.1),
           dict(min_w=float("nan")),
           dict(lazy_tau=float("inf")),
           dict(lazy_tau=-1.0)]
    for kw in bad:
        o = B.make_opts(**kw)
        assert lib.moe_route_ex(FAKE, 4, 256, 6, 1.5, ctypes.byref(o), FAKE, FAKE, None) == \
            B.MOE_ERR_INVALID, kw
        assert lib.moe_route_group_ex(FAKE, 4, 256, 6, 1.5, ctypes.byref(o), FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, None, None) == B.MOE_ERR_INVALID, kw
    o = B.make_opts()
    o.sel_bias = 0x10002  # not 4-byte aligned
    assert lib.moe_route_ex(FAKE, 4, 256, 6, 1.5, ctypes.byref(o), FAKE, FAKE, None) == \
        B.MOE_ERR_INVALID
    # the FFN and the whole layer check the options too
    L = _layer()
    o = B.make_opts(lazy_tau=-1.0)
    assert lib.moe_ffn_forward_ex(ctypes.byref(L), FAKE, B.MOE_ACT_BF16, 4, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, ctypes.byref(o), FAKE, 1 << 40, None, None,
                                  None, None, None) == B.MOE_ERR_INVALID
    o = B.make_opts(keep_max=9)
    assert lib.moe_forward_ex(ctypes.byref(L), FAKE, 1.5, ctypes.byref(o), FAKE, B.MOE_ACT_BF16,
                              1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None,
                              None, None, None) == B.MOE_ERR_INVALID


def test_opts_struct_layout_matches_c():
    # int32 x2, pointer, int32, float x2
    assert B.MoeOpts.sel_bias.offset == 8
    assert B.MoeOpts.keep_max.offset == 16
    assert B.MoeOpts.lazy_tau.offset == 24
    assert ctypes.sizeof(B.MoeOpts) == 32


def _pack_bytes_expected(E, H, I, SI=None, shared_fp8=False):
    """The packed layout of include/moe.h, summed section by section: codes
    (half a byte per input MXFP4, a byte fp8), then R*C/32 bytes of scale
    words."""
    def up(v):
        return -(-v // 256) * 256
    mats = [(E * I, H, 2), (E * I, H, 2), (E * H, I, 2)]
    if SI is not None:
        d = 1 if shared_fp8 else 2
        mats += [(SI, H, d), (SI, H, d), (H, SI, d)]
    return sum(up(r * c // d) + up(r * c // 32) for r, c, d in mats)


def test_packed_experts_bytes():
    lib = B.lib()
    # routed and shared MXFP4: all six matrices
    L = _layer()
    assert lib.moe_packed_experts_bytes(ctypes.byref(L)) == _pack_bytes_expected(256, 4096, 2048, 2048)
    # an fp8 shared expert: a byte per input
    L = _layer(swtype=1)
    assert lib.moe_packed_experts_bytes(ctypes.byref(L)) == \
        _pack_bytes_expected(256, 4096, 2048, 2048, shared_fp8=True)
    L = _layer(shared=False, e=8, hidden=1024, inter=512)
    assert lib.moe_packed_experts_bytes(ctypes.byref(L)) == _pack_bytes_expected(8, 1024, 512)
    # cannot be packed: fp8 routed experts, H or I not a multiple of 512
    assert lib.moe_packed_experts_bytes(ctypes.byref(_layer(wtype=1, swtype=1))) == 0
    assert lib.moe_packed_experts_bytes(ctypes.byref(_layer(hidden=640))) == 0
    assert lib.moe_packed_experts_bytes(ctypes.byref(_layer(inter=384))) == 0
    assert lib.moe_packed_experts_bytes(None) == 0


def test_pack_experts_rejects_bad_arguments():
    """Host-side checks only: every call here returns before any launch."""
    lib = B.lib()
    L = _layer(shared=False, e=8, hidden=1024, inter=512)
    n = lib.moe_packed_experts_bytes(ctypes.byref(L))
    aligned = ctypes.c_void_p(0x100000)
    assert lib.moe_pack_experts(ctypes.byref(L), None, n, None) == B.MOE_ERR_INVALID
    assert lib.moe_pack_experts(ctypes.byref(L), ctypes.c_void_p(0x100010), n, None) == B.MOE_ERR_INVALID
    assert lib.moe_pack_experts(ctypes.byref(L), aligned, n - 1, None) == B.MOE_ERR_INVALID
    assert lib.moe_pack_experts(None, aligned, n, None) == B.MOE_ERR_INVALID
    fp8 = _layer(wtype=1, swtype=1, shared=False)
    assert lib.moe_pack_experts(ctypes.byref(fp8), aligned, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED
    # a layer that names a packed copy must be packable and the copy aligned
    L.packed_experts = 0x100000
    assert lib.moe_ffn_workspace_bytes(ctypes.byref(L), 8) > 0
    L.packed_experts = 0x100010
    assert lib.moe_ffn_workspace_bytes(ctypes.byref(L), 8) == 0
    fp8.packed_experts = 0x100000
    assert lib.moe_ffn_workspace_bytes(ctypes.byref(fp8), 8) == 0


def test_mfma_rate_rejects_bad_arguments():
    """moe_mfma_rate checks its arguments before touching the device."""
    L = B.lib()
    invalid = 1  # MOE_ERR_INVALID
    assert L.moe_mfma_rate(8, 0, 0, 1, None, None) == invalid       # no such shape
    assert L.moe_mfma_rate(16, 1, 0, 1, None, None) == invalid      # E5M2 is not offered
    assert L.moe_mfma_rate(32, 0, 3, 1, None, None) == invalid
    assert L.moe_mfma_rate(16, 0, 0, 0, None, None) == invalid      # no rounds
    assert L.moe_mfma_rate(16, 4, 0, 1, None, None) == invalid      # null output
