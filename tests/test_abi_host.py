"""Host-side checks of the C ABI: the library loads, exports every function
include/gha.h declares, and rejects bad arguments before touching a device.
No kernel is launched here; fake (but aligned) pointers only reach the
argument checks, which fail first."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import grouped_head_latent_amd as gha
from grouped_head_latent_amd import GhaTensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gha.library_path()):
        from grouped_head_latent_amd import build
        build.build()
    return gha.load_library()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"gqa_prefill", "gqa_decode", "gta_shared_score_prefill", "latent_absorb_decode",
            "gta_shared_score_decode", "gqla_gqa_decode", "gta_shared_score_decode_workspace_bytes",
            "gqla_gqa_decode_workspace_bytes",
            "gqa_decode_workspace_bytes", "latent_absorb_decode_workspace_bytes",
            "gqa_decode_paged", "gqa_decode_paged_workspace_bytes", "gqla_gqa_prefill",
            "gqla_absorb_decode", "gqla_absorb_decode_workspace_bytes", "gqa_decode_fp8",
            "gha_status_string", "gha_last_error", "gha_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gha_version() >= 100
    assert lib.gha_status_string(3) == b"GHA_ERR_GROUPING"


def test_debug_checks_switch(lib):
    assert lib.gha_status_string(10) == b"GHA_ERR_PRECONDITION"
    before = lib.gha_debug_checks()
    try:
        lib.gha_set_debug_checks(1)
        assert lib.gha_debug_checks() == 1 and gha.debug_checks()
        lib.gha_set_debug_checks(0)
        assert lib.gha_debug_checks() == 0 and not gha.debug_checks()
        gha.set_debug_checks(True)
        assert lib.gha_debug_checks() == 1
    finally:
        lib.gha_set_debug_checks(before)


@pytest.mark.parametrize("env,want", [("1", "True"), ("0", "False"), (None, "False")])
def test_debug_checks_follow_the_environment_until_set(lib, env, want):
    e = {k: v for k, v in os.environ.items() if k != "GHA_DEBUG_CHECKS"}
    if env is not None:
        e["GHA_DEBUG_CHECKS"] = env
    code = ("import grouped_head_latent_amd as g; a = g.debug_checks(); g.set_debug_checks(not a); "
            "print(a, g.debug_checks())")
    r = subprocess.run([sys.executable, "-c", code], env=e, cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == [want, str(want != "True")]


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def T(ptr=FAKE, sb=1 << 20, sh=1 << 14, ss=128):
    return GhaTensor(ptr, sb, sh, ss)


def prefill(lib, **kw):
    a = dict(q=T(), k=T(), v=T(), o=T(), lse=None, B=1, h_q=8, h_kv=2, S_q=16, S_k=16, d=128,
             i=gha.GHA_BF16, o_t=gha.GHA_BF16, scale=0.0, causal=1)
    a.update(kw)
    return lib.gqa_prefill(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                           ctypes.byref(a["o"]), a["lse"], a["B"], a["h_q"], a["h_kv"], a["S_q"],
                           a["S_k"], a["d"], a["i"], a["o_t"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(h_kv=3), 3),                      # 8 % 3 != 0
    (dict(d=96), 7),                        # unsupported head dim
    (dict(S_q=17, S_k=16), 2),              # causal with S_q > S_k
    (dict(B=0), 2),
    (dict(i=gha.GHA_F32, o_t=gha.GHA_BF16), 6),
    (dict(q=T(ptr=0)), 1),
    (dict(k=T(ptr=FAKE + 2)), 5),           # misaligned pointer
    (dict(v=T(ss=100)), 5),                 # 200-byte rows: not 16-byte multiples
    (dict(o=T(sh=-1)), 4),
])
def test_prefill_rejects_bad_arguments(lib, kw, status):
    assert prefill(lib, **kw) == status
    assert len(lib.gha_last_error()) > 0


def decode(lib, **kw):
    a = dict(q=T(), k=T(), v=T(), seq=FAKE, o=T(), B=2, h_q=32, h_kv=8, s_q=1, L_cap=4096,
             L_max=4096, d=128, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gqa_decode(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                          ctypes.c_void_p(a["seq"]) if a["seq"] else None, ctypes.byref(a["o"]), None,
                          a["B"], a["h_q"], a["h_kv"], a["s_q"], a["L_cap"], a["L_max"], a["d"],
                          gha.GHA_BF16, gha.GHA_BF16, 0.0,
                          ctypes.c_void_p(a["ws"]) if a["ws"] else None, a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(h_kv=5), 3),
    (dict(L_max=8192), 2),                  # hint above capacity
    (dict(s_q=3, L_max=2, L_cap=2), 2),     # s_q above the longest sequence
    (dict(seq=0), 1),
    (dict(ws=0), 8),
    (dict(ws_bytes=16), 8),
    (dict(d=256), 7),
])
def test_decode_rejects_bad_arguments(lib, kw, status):
    assert decode(lib, **kw) == status


def paged(lib, **kw):
    a = dict(q=T(), k=T(sb=1 << 16, sh=1 << 13), v=T(sb=1 << 16, sh=1 << 13), bt=FAKE, bt_stride=64,
             page=64, seq=FAKE, o=T(), B=2, h_q=32, h_kv=8, s_q=1, L_cap=4096, L_max=4096, window=0,
             d=128, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gqa_decode_paged(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                                ctypes.c_void_p(a["bt"]) if a["bt"] else None, a["bt_stride"], a["page"],
                                ctypes.c_void_p(a["seq"]) if a["seq"] else None, ctypes.byref(a["o"]), None,
                                a["B"], a["h_q"], a["h_kv"], a["s_q"], a["L_cap"], a["L_max"], a["window"],
                                a["d"], gha.GHA_BF16, gha.GHA_BF16, 0.0,
                                ctypes.c_void_p(a["ws"]) if a["ws"] else None, a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(h_kv=5), 3),
    (dict(page=48), 2),                     # not a multiple of 32
    (dict(page=0), 2),
    (dict(bt_stride=63), 2),                # 63 pages of 64 tokens do not cover 4096
    (dict(window=-1), 2),
    # 32 query heads over 8 KV heads at s_q = 2 is 8 rows per group: the row
    # check passes and the call stops at the (too small) workspace instead
    (dict(s_q=2, ws_bytes=16), 8),
    (dict(h_q=64, s_q=5), 2),               # 8 heads x 5 tokens = 40 rows > 32
    (dict(seq=0), 1),
    (dict(ws=0), 8),
    (dict(ws_bytes=16), 8),
    (dict(d=256), 7),
    (dict(k=T(sb=1 << 16, sh=1 << 13, ss=64)), 4),   # rows overlap (token stride < d)
    (dict(v=T(sb=(1 << 16) + 4)), 5),                 # page stride not a multiple of 16 bytes
])
def test_paged_decode_rejects_bad_arguments(lib, kw, status):
    assert paged(lib, **kw) == status
    assert len(lib.gha_last_error()) > 0


def test_paged_decode_workspace_follows_the_window(lib):
    # one slot per work-group and per (sequence, KV head), 16 padded rows; the
    # size covers the 8-bit caches' plan of two work-groups per CU (512)
    full = lib.gqa_decode_paged_workspace_bytes(64, 32, 8, 1, 32768, 0, 128)
    assert full == (512 + 64 * 8) * 16 * 129 * 4 + 65 * 4
    # a short window has fewer chunks: fewer work-groups are planned
    short = lib.gqa_decode_paged_workspace_bytes(1, 4, 1, 1, 32768, 100, 128)
    assert short == (3 + 1) * 16 * 129 * 4 + 2 * 4
    assert lib.gqa_decode_paged_workspace_bytes(64, 40, 8, 8, 32768, 0, 128) == 0


def gqla_prefill(lib, **kw):
    a = dict(qc=T(), qr=T(ss=64), kc=T(), kr=T(ss=64), v=T(), o=T(), B=1, h_q=16, g=2, S_q=256, S_k=256,
             d_h=128, d_r=64, i=gha.GHA_BF16, o_t=gha.GHA_F32, scale=0.07, causal=1)
    a.update(kw)
    return lib.gqla_gqa_prefill(ctypes.byref(a["qc"]), ctypes.byref(a["qr"]), ctypes.byref(a["kc"]),
                                ctypes.byref(a["kr"]), ctypes.byref(a["v"]), ctypes.byref(a["o"]), None,
                                a["B"], a["h_q"], a["g"], a["S_q"], a["S_k"], a["d_h"], a["d_r"], a["i"],
                                a["o_t"], ctypes.c_float(a["scale"]), a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=3), 3),
    (dict(d_h=64), 7),
    (dict(d_r=32), 7),
    (dict(scale=0.0), 2),                   # the expanded head width is not an argument
    (dict(S_q=300), 2),                     # causal with S_q > S_k
    (dict(i=gha.GHA_F32), 6),
    (dict(kr=T(ptr=0)), 1),
    (dict(kr=T(ss=32)), 4),                 # RoPE rows overlap
    (dict(v=T(ss=100)), 5),
])
def test_gqla_prefill_rejects_bad_arguments(lib, kw, status):
    assert gqla_prefill(lib, **kw) == status
    assert len(lib.gha_last_error()) > 0


def absorbing(lib, **kw):
    a = dict(qc=T(ss=128 * 128, sh=128), qr=T(ss=64 * 128, sh=64), wuk=FAKE, wuv=FAKE, c=T(ss=576), kr=T(ss=576),
             seq=FAKE, o=T(ss=128 * 128, sh=128), B=2, h_q=128, g=8, s_q=1, L_cap=4096, L_max=4096, d_h=128,
             r=512, d_r=64, scale=0.07, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gqla_absorb_decode(ctypes.byref(a["qc"]), ctypes.byref(a["qr"]),
                                  ctypes.c_void_p(a["wuk"]) if a["wuk"] else None,
                                  ctypes.c_void_p(a["wuv"]) if a["wuv"] else None,
                                  ctypes.byref(a["c"]), ctypes.byref(a["kr"]),
                                  ctypes.c_void_p(a["seq"]) if a["seq"] else None, ctypes.byref(a["o"]), None,
                                  a["B"], a["h_q"], a["g"], a["s_q"], a["L_cap"], a["L_max"], a["d_h"], a["r"],
                                  a["d_r"], gha.GHA_BF16, gha.GHA_BF16, ctypes.c_float(a["scale"]),
                                  ctypes.c_void_p(a["ws"]) if a["ws"] else None, a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=3), 3),
    (dict(d_h=64), 7),
    (dict(r=256), 7),
    (dict(wuk=0), 1),
    (dict(wuv=FAKE + 8), 5),                # weights not 16-byte aligned
    (dict(scale=0.0), 2),
    (dict(seq=0), 1),
    (dict(ws_bytes=4096), 8),
    (dict(ws=FAKE + 16), 5),                # workspace not 256-byte aligned
])
def test_absorbing_decode_rejects_bad_arguments(lib, kw, status):
    assert absorbing(lib, **kw) == status
    assert len(lib.gha_last_error()) > 0


def test_absorbing_decode_workspace_adds_query_and_latent_output(lib):
    lat = lib.latent_absorb_decode_workspace_bytes(64, 128, 1, 65536, 512)
    up = lambda x: (x + 255) // 256 * 256
    rows = 64 * 128
    # the latent decode's workspace, q~ and o_lat (bf16 each), W^UK transposed
    assert lib.gqla_absorb_decode_workspace_bytes(64, 128, 1, 65536, 512) == (
        up(lat) + 2 * up(rows * 512 * 2) + 128 * 128 * 512 * 2)


def fp8(lib, **kw):
    a = dict(q=T(), k=T(sb=1 << 20, sh=1 << 17, ss=128), v=T(sb=1 << 20, sh=1 << 17, ss=128), ks=0.05, vs=0.02,
             bt=0, bt_stride=0, page=0, seq=FAKE, o=T(), B=2, h_q=32, h_kv=8, s_q=1, L_cap=1024, L_max=1024,
             window=0, d=128, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.gqa_decode_fp8(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                              ctypes.c_float(a["ks"]), ctypes.c_float(a["vs"]),
                              ctypes.c_void_p(a["bt"]) if a["bt"] else None, a["bt_stride"], a["page"],
                              ctypes.c_void_p(a["seq"]) if a["seq"] else None, ctypes.byref(a["o"]), None,
                              a["B"], a["h_q"], a["h_kv"], a["s_q"], a["L_cap"], a["L_max"], a["window"], a["d"],
                              gha.GHA_BF16, ctypes.c_float(0.0),
                              ctypes.c_void_p(a["ws"]) if a["ws"] else None, a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=0.0), 2),
    (dict(vs=float("inf")), 2),
    (dict(d=96), 7),
    (dict(k=T(sb=1 << 20, sh=1 << 17, ss=112)), 4),         # 112-byte rows of 128 codes overlap
    (dict(v=T(sb=1 << 20, sh=1 << 17, ss=136)), 5),         # 136-byte rows: not 16-byte multiples
    (dict(h_kv=3), 3),
    (dict(bt=FAKE, bt_stride=16, page=48), 2),
    (dict(ws_bytes=16), 8),
])
def test_fp8_decode_rejects_bad_arguments(lib, kw, status):
    assert fp8(lib, **kw) == status
    assert len(lib.gha_last_error()) > 0


def test_workspace_sizes_cover_the_split_plan(lib):
    assert lib.gqa_decode_workspace_bytes(64, 32, 8, 1, 32768, 128) > 0
    assert lib.gqa_decode_workspace_bytes(64, 32, 7, 1, 32768, 128) == 0
    # latent: 2 row blocks of 128 rows, 128 work-groups per row block, one
    # partial (512 outputs + lse, fp32) per work-group and per sequence it
    # touches (at most n_wg + B slots), plus B + 1 tile prefix sums
    n = lib.latent_absorb_decode_workspace_bytes(64, 128, 2, 65536, 512)
    assert n == 2 * (128 + 64) * 128 * 513 * 4 + 65 * 4
    # a tiny problem has no more work-groups than tiles
    assert lib.latent_absorb_decode_workspace_bytes(1, 128, 1, 40, 512) == 1 * (2 + 1) * 128 * 513 * 4 + 2 * 4


def latent(lib, **kw):
    a = dict(r_kv=512, d_r=64, scale=0.07, L_max=1024, L_cap=1024, s_q=1)
    a.update(kw)
    return lib.latent_absorb_decode(ctypes.byref(T(ss=512 * 128)), ctypes.byref(T(ss=64 * 128)),
                                    ctypes.byref(T(ss=576)), ctypes.byref(T(ptr=FAKE + 1024, ss=576)),
                                    ctypes.c_void_p(FAKE), ctypes.byref(T(ss=512 * 128)), None, 2, 128,
                                    a["s_q"], a["L_cap"], a["L_max"], a["r_kv"], a["d_r"], gha.GHA_BF16,
                                    gha.GHA_BF16, a["scale"], ctypes.c_void_p(FAKE), 16, None)


@pytest.mark.parametrize("kw,status", [
    (dict(r_kv=256), 7), (dict(d_r=32), 7), (dict(scale=0.0), 2), (dict(L_max=2048), 2),
])
def test_latent_rejects_bad_arguments(lib, kw, status):
    assert latent(lib, **kw) == status


def test_latent_rejects_small_workspace(lib):
    assert latent(lib) == 8


def gta(lib, **kw):
    a = dict(h=16, n_grp=4, d_qk=64, d_v=64)
    a.update(kw)
    return lib.gta_shared_score_prefill(ctypes.byref(T()), ctypes.byref(T()), ctypes.byref(T()),
                                        ctypes.byref(T()), None, 1, a["h"], a["n_grp"], 64, a["d_qk"],
                                        a["d_v"], gha.GHA_BF16, gha.GHA_BF16, 0.0, 1, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_grp=3), 3), (dict(d_v=96), 7), (dict(d_v=512), 7), (dict(d_v=32), 7), (dict(d_qk=96), 7),
])
def test_gta_rejects_bad_arguments(lib, kw, status):
    assert gta(lib, **kw) == status


def gta_dec(lib, **kw):
    a = dict(h=16, n_grp=4, s_q=1, L_cap=4096, L_max=4096, d_qk=64, d_v=64, seq=FAKE, ws=FAKE, ws_bytes=1 << 40,
             k=T(), v=T())
    a.update(kw)
    return lib.gta_shared_score_decode(ctypes.byref(T()), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                                       ctypes.c_void_p(a["seq"]) if a["seq"] else None, ctypes.byref(T()), None,
                                       2, a["h"], a["n_grp"], a["s_q"], a["L_cap"], a["L_max"], a["d_qk"],
                                       a["d_v"], gha.GHA_BF16, gha.GHA_BF16, 0.0,
                                       ctypes.c_void_p(a["ws"]) if a["ws"] else None, a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_grp=3), 3), (dict(d_v=96), 7), (dict(d_v=512), 7), (dict(d_qk=96), 7),
    (dict(s_q=33, L_max=64), 2), (dict(L_max=8192), 2), (dict(seq=0), 1), (dict(ws_bytes=16), 8),
    # wider values and more heads per group are accepted; these stop at the workspace
    (dict(d_v=256, v=T(ss=256), ws_bytes=16), 8), (dict(h=32, n_grp=4, d_v=128, ws_bytes=16), 8),
    (dict(d_v=256), 4),                     # value rows of 256 elements would overlap (ss = 128)
    (dict(k=T(ss=32)), 4),                  # key rows of 64 elements would overlap
    (dict(v=T(ss=1 << 20)), 2),             # a sequence spanning 8 GiB
])
def test_gta_decode_rejects_bad_arguments(lib, kw, status):
    assert gta_dec(lib, **kw) == status


def gqla(lib, **kw):
    a = dict(h_q=128, g=8, s_q=2, L_cap=4096, L_max=4096, d_h=128, d_r=64, scale=0.07, ws=FAKE, ws_bytes=1 << 40,
             k_r=T(ss=64))
    a.update(kw)
    return lib.gqla_gqa_decode(ctypes.byref(T()), ctypes.byref(T()), ctypes.byref(T()), ctypes.byref(a["k_r"]),
                               ctypes.byref(T()), ctypes.c_void_p(FAKE), ctypes.byref(T()), None, 2, a["h_q"],
                               a["g"], a["s_q"], a["L_cap"], a["L_max"], a["d_h"], a["d_r"], gha.GHA_BF16,
                               gha.GHA_BF16, a["scale"], ctypes.c_void_p(a["ws"]) if a["ws"] else None,
                               a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=3), 3), (dict(d_h=64), 7), (dict(d_r=32), 7), (dict(scale=0.0), 2),
    (dict(s_q=3), 2),                       # 16 heads x 3 tokens: more than 32 rows per group
    (dict(ws=0), 8), (dict(k_r=T(ss=32)), 4),
])
def test_gqla_decode_rejects_bad_arguments(lib, kw, status):
    assert gqla(lib, **kw) == status


def test_stream_decode_workspace_sizes(lib):
    # one partial slot per work-group (256 of them, one per CU) and per
    # (sequence, group), padded rows of (outputs + lse), then B + 1 chunk
    # prefix sums
    # GTA: 64 x 4 (sequence, group) units, 16 padded rows of 4 x 64 outputs
    assert lib.gta_shared_score_decode_workspace_bytes(64, 16, 4, 1, 32768, 64) == (256 + 256) * 16 * 257 * 4 + 65 * 4
    # GQLA at s_q = 2: 32 teams of 8, 64 x 8 (sequence, group), 32 rows each
    assert lib.gqla_gqa_decode_workspace_bytes(64, 128, 8, 2, 65536, 128) == (256 + 512) * 32 * 129 * 4 + 65 * 4
    assert lib.gqla_gqa_decode_workspace_bytes(64, 128, 8, 3, 65536, 128) == 0
    # a tiny problem has no more work-groups than chunks
    assert lib.gta_shared_score_decode_workspace_bytes(1, 4, 1, 1, 100, 64) == (1 + 1) * 16 * 257 * 4 + 2 * 4


def test_gta_decode_workspace_follows_the_value_sources(lib):
    # value sources of 128 columns for d_v >= 128: a launch takes up to 512
    # columns when one q-tile holds the rows (s_q <= 16), else up to 256; the
    # launches over a group's sources reuse one launch's workspace
    def ws(rows_padded, dv, units=64 * 4, wgs=256):
        n = (wgs + units) * rows_padded
        return n * dv * 4 + n * 4 + 65 * 4
    assert lib.gta_shared_score_decode_workspace_bytes(64, 16, 4, 1, 32768, 64) == ws(16, 256)
    assert lib.gta_shared_score_decode_workspace_bytes(64, 16, 4, 1, 32768, 128) == ws(16, 512)
    assert lib.gta_shared_score_decode_workspace_bytes(64, 16, 4, 2, 32768, 256) == ws(16, 512)
    assert lib.gta_shared_score_decode_workspace_bytes(64, 16, 4, 17, 32768, 128) == ws(32, 256)
    assert lib.gta_shared_score_decode_workspace_bytes(64, 12, 4, 1, 32768, 64) == ws(16, 64)   # 3 heads: 1 source a launch
    assert lib.gta_shared_score_decode_workspace_bytes(64, 16, 4, 1, 32768, 96) == 0


def test_valid_call_without_device_reports_hip_error(lib):
    """On a host with no GPU a well-formed call must fail cleanly with
    GHA_ERR_HIP (never crash).  Skipped where a device exists, since the fake
    pointers would then reach a kernel."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    assert prefill(lib) == 9
    assert b"device" in lib.gha_last_error()


def test_fp8_decode_plans_two_work_groups_per_cu(lib):
    # 8-bit caches plan 512 work-groups (two per CU) where 16-bit ones plan 256,
    # so the bf16 plan's workspace is too small for them and the paged query
    # covers both
    big = dict(k=T(sb=1 << 26, sh=1 << 22, ss=128), v=T(sb=1 << 26, sh=1 << 22, ss=128),
               L_cap=32768, L_max=32768)
    full = lib.gqa_decode_paged_workspace_bytes(2, 32, 8, 1, 32768, 0, 128)
    assert full == (512 + 2 * 8) * 16 * 129 * 4 + 3 * 4
    bf16_plan = (256 + 2 * 8) * 16 * 129 * 4 + 3 * 4
    assert fp8(lib, ws_bytes=bf16_plan, **big) == 8
    assert fp8(lib, ws_bytes=full - 1, **big) == 8
    # a call with the full workspace would pass every check and launch on the
    # fake pointers, so it is never made here
