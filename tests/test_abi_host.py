"""Host-side tests of the C ABI (no GPU needed).

Every argument check in libvx runs before any HIP call, so these tests call
the entry points with host buffers standing in for device pointers and check
that each invalid argument is rejected with the documented status and that
no buffer is touched.  They also check that libvx.so exports every function
include/vx.h declares and that the header compiles as plain C.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import sliding_window_attention_vx_amd as vx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vx.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_RANGE, E_HIP = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(vx_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vx.LIB_PATH):
        from sliding_window_attention_vx_amd import build
        build.build()
    return vx.lib()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ("vx_rope_qk", "vx_swa_attn_prefill", "vx_swa_attn_stream_step", "vx_kv_ring_append",
              "vx_swa_attn_stream_step_append", "vx_rope_table", "vx_status_string",
              "vx_last_error", "vx_version", "vx_default_cfg", "vx_swa_attn_prefill_varlen",
              "vx_default_gqa_cfg", "vx_gqa_attn_prefill", "vx_gqa_attn_decode", "vx_linear",
              "vx_enc_qkv_rope", "vx_enc_attn_step", "vx_rmsnorm", "vx_enc_stem_step",
              "vx_enc_layer_step", "vx_enc_step", "vx_swa_attn_prefill_workspace_size"):
        assert f in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", vx.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (vx_\w+)", out))
    assert set(declared_functions()) <= exported


def test_header_is_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "vx.h"\n#include <stdio.h>\n'
                   "int main(void){vx_attn_cfg c; vx_default_cfg(&c);\n"
                   " vx_status s = vx_swa_attn_prefill(0,0,0,0,1,1,1,0,1,0,0,0,&c,0);\n"
                   ' printf("%d %d %s\\n", c.window, (int)s, vx_status_string(s));\n'
                   " return s == VX_E_NULL ? 0 : 1;}\n")
    exe = tmp_path / "use"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(exe), vx.LIB_PATH, f"-Wl,-rpath,{os.path.dirname(vx.LIB_PATH)}"],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split()[:2] == ["750", "1"]


def test_default_cfg(L):
    c = vx._Cfg()
    L.vx_default_cfg(ctypes.byref(c))
    assert (c.head_dim, c.window, c.rope_theta, c.softmax_scale, c.io_dtype, c.out_dtype, c.flags) \
        == (64, 750, 1e6, 0.125, vx.VX_BF16, vx.VX_BF16, 0)
    assert (c.workspace, c.workspace_bytes) == (None, 0)
    assert L.vx_version() >= 100


def test_status_strings(L):
    for code in range(7):
        assert L.vx_status_string(code).decode() == vx._STATUS[code]


class Bufs:
    """Host arrays standing in for device buffers (16-byte aligned)."""

    def __init__(self, nbytes=1 << 16):
        self.arrs = []
        self.nbytes = nbytes

    def new(self):
        a = np.full(self.nbytes // 4 + 16, 7.0, dtype=np.float32)
        off = (-a.ctypes.data) % 16 // 4
        a = a[off:off + self.nbytes // 4]
        assert a.ctypes.data % 16 == 0
        self.arrs.append(a)
        return ctypes.c_void_p(a.ctypes.data)

    def untouched(self):
        return all(np.all(a == 7.0) for a in self.arrs)


def cfg(**kw):
    c = vx._Cfg()
    vx.lib().vx_default_cfg(ctypes.byref(c))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def prefill(L, b, c, q=None, k=None, v=None, o=None, B=1, T=8, H=2, pos0=None, rope_applied=1,
            table=None, tp0=0, tlen=0):
    q = q if q is not None else b.new()
    k = k if k is not None else b.new()
    v = v if v is not None else b.new()
    o = o if o is not None else b.new()
    return L.vx_swa_attn_prefill(q, k, v, o, B, T, H, pos0, rope_applied, table, tp0, tlen,
                                 None if c is None else ctypes.byref(c), None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=32), E_SHAPE), (dict(window=0), E_RANGE), (dict(window=-5), E_RANGE),
    (dict(rope_theta=0.0), E_RANGE), (dict(rope_theta=float("nan")), E_RANGE),
    (dict(rope_theta=float("inf")), E_RANGE), (dict(softmax_scale=-1.0), E_RANGE),
    (dict(softmax_scale=float("nan")), E_RANGE), (dict(io_dtype=vx.VX_F32, out_dtype=vx.VX_BF16), E_DTYPE),
    (dict(io_dtype=7), E_DTYPE), (dict(out_dtype=-1), E_DTYPE), (dict(flags=4), E_RANGE),
])
def test_prefill_rejects_bad_cfg(L, kw, status):
    b = Bufs()
    assert prefill(L, b, cfg(**kw)) == status
    assert L.vx_last_error().decode() != ""
    assert b.untouched()


def test_prefill_argument_errors(L):
    b = Bufs()
    c = cfg()
    assert prefill(L, b, None) == E_NULL
    assert prefill(L, b, c, B=-1) == E_SHAPE
    assert prefill(L, b, c, T=-3) == E_SHAPE
    assert prefill(L, b, c, H=0) == E_SHAPE
    assert prefill(L, b, c, T=1 << 25) == E_SHAPE
    assert prefill(L, b, c, q=ctypes.c_void_p(0)) == E_NULL
    assert prefill(L, b, c, o=ctypes.c_void_p(0)) == E_NULL
    mis = ctypes.c_void_p(b.new().value + 4)
    assert prefill(L, b, c, v=mis) == E_ALIGN
    q = b.new()
    assert prefill(L, b, c, q=q, o=q) == E_RANGE  # o aliases q
    # pos0 is a device int64 array: only its alignment is checked on the host
    assert prefill(L, b, c, pos0=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    # a table must cover the chunk's positions 0 .. T-1 when pos0 is NULL
    t = b.new()
    assert prefill(L, b, c, rope_applied=0, table=t, tp0=0, tlen=7) == E_RANGE
    assert prefill(L, b, c, rope_applied=0, table=t, tp0=5, tlen=100) == E_RANGE
    assert prefill(L, b, c, rope_applied=0, table=t, tp0=-1, tlen=100) == E_RANGE
    assert prefill(L, b, c, rope_applied=0, table=ctypes.c_void_p(t.value + 4), tp0=0,
                   tlen=100) == E_ALIGN
    assert b.untouched()


def test_prefill_workspace_checks(L):
    b = Bufs()
    ws = b.new()
    assert prefill(L, b, cfg(workspace=None, workspace_bytes=64)) == E_NULL
    assert prefill(L, b, cfg(workspace=ctypes.c_void_p(ws.value + 8), workspace_bytes=64)) == E_ALIGN
    q = b.new()
    assert prefill(L, b, cfg(workspace=q, workspace_bytes=64), q=q) == E_RANGE  # overlaps q
    assert b.untouched()


def test_prefill_workspace_size(L):
    size = L.vx_swa_attn_prefill_workspace_size
    c = cfg()
    # a cos/sin table of B*T rows of 256 bytes (rounded up to 256), then, where
    # the split walk is taken (only with VX_FLAG_SPLIT_WALK, on grids of at
    # most 1.5 128-query tiles per compute unit: 256 CUs without a device), a
    # flag word per (b, h, query tile, wave), 256-byte aligned, and two
    # 9216-byte partial results per flag
    # grids of at least 8 query tiles per CU also keep the keys rotated
    # ahead of the kernel there (B*T*H rows of 128 bytes)
    assert size(8, 6000, 32, ctypes.byref(c)) == 8 * 6000 * 256 + 8 * 6000 * 32 * 128
    assert size(8, 1500, 32, ctypes.byref(c)) == 8 * 1500 * 256 + 8 * 1500 * 32 * 128
    assert size(8, 1024, 32, ctypes.byref(c)) == 8 * 1024 * 256 + 8 * 1024 * 32 * 128  # 8 per CU
    assert size(7, 1024, 32, ctypes.byref(c)) == 7 * 1024 * 256  # 7 tiles per CU: not
    assert size(4, 1500, 32, ctypes.byref(c)) == 4 * 1500 * 256
    assert size(2, 1500, 32, ctypes.byref(c)) == 2 * 1500 * 256  # 768 query tiles: neither
    assert size(1, 1500, 32, ctypes.byref(c)) == 1500 * 256  # 384 query tiles: not split
    assert size(1, 1500, 16, ctypes.byref(c)) == 1500 * 256  # no split without the flag
    force = cfg(flags=2)
    slots = 12 * 16 * 4
    assert size(1, 1500, 16, ctypes.byref(force)) == 1500 * 256 + slots * 8 + slots * 2 * 9216
    slots = 12 * 32 * 4
    assert size(1, 1500, 32, ctypes.byref(force)) == 1500 * 256 + slots * 8 + slots * 2 * 9216
    assert size(2, 1500, 32, ctypes.byref(force)) == 2 * 1500 * 256  # 768 tiles: never split
    assert size(1, 3, 1, ctypes.byref(c)) == 3 * 256  # a one-tile band: not split
    assert size(1, 3, 1, ctypes.byref(force)) == 3 * 256 + 256 + 4 * 2 * 9216
    assert size(1, 1500, 16, ctypes.byref(cfg(window=64))) == 1500 * 256  # 3-tile bands
    assert size(1, 1500, 32, None) == 0
    assert size(-1, 1500, 32, ctypes.byref(c)) == 0
    assert size(1, 1500, 32, ctypes.byref(cfg(window=0))) == 0


def test_prefill_noalloc_host_checks(L):
    """The allocation-free prefill refuses more rows than its static scratch
    holds (before any HIP call) and validates like vx_swa_attn_prefill."""
    b = Bufs()
    c = cfg()
    q, k, v, o = b.new(), b.new(), b.new(), b.new()
    f = L.vx_swa_attn_prefill_noalloc
    assert f(q, k, v, o, 1, 65537, 1, None, 0, ctypes.byref(c), None) == E_SHAPE
    assert "scratch" in L.vx_last_error().decode()
    assert f(q, k, v, o, 2, 40000, 1, None, 0, ctypes.byref(c), None) == E_SHAPE
    assert f(q, k, v, o, 1, 8, 2, None, 0, None, None) == E_NULL
    assert f(q, k, v, o, 1, 8, 2, None, 0, ctypes.byref(cfg(window=0)), None) == E_RANGE
    z = ctypes.c_void_p(0)
    assert f(z, z, z, z, 0, 8, 2, None, 0, ctypes.byref(c), None) == OK
    assert b.untouched()


def test_prefill_empty_is_ok_without_launch(L):
    c = cfg()
    z = ctypes.c_void_p(0)
    assert L.vx_swa_attn_prefill(z, z, z, z, 0, 10, 4, 0, 1, z, 0, 0, ctypes.byref(c), z) == OK
    assert L.vx_swa_attn_prefill(z, z, z, z, 3, 0, 4, 0, 1, z, 0, 0, ctypes.byref(c), z) == OK
    assert L.vx_last_error().decode() == ""


def prefill_varlen(L, b, c, S=2, max_T=8, H=2, rope_applied=1, table=None, tp0=0, tlen=0,
                   seed=False, total=10, **ov):
    a = dict(q=b.new(), k=b.new(), v=b.new(), o=b.new(), cu=b.new())
    if seed:
        a.update(rk=b.new(), rv=b.new(), pos=b.new())
    a.update(ov)
    return L.vx_swa_attn_prefill_varlen(a["q"], a["k"], a["v"], a["o"], a["cu"], S, total, max_T, H,
                                        rope_applied, table, tp0, tlen, a.get("rk"), a.get("rv"),
                                        a.get("pos"), None if c is None else ctypes.byref(c), None)


def test_prefill_varlen_argument_errors(L):
    b = Bufs()
    c = cfg()
    assert prefill_varlen(L, b, None) == E_NULL
    assert prefill_varlen(L, b, cfg(io_dtype=vx.VX_F32, out_dtype=vx.VX_F32)) == E_DTYPE
    assert prefill_varlen(L, b, c, S=-1) == E_SHAPE
    assert prefill_varlen(L, b, c, max_T=-2) == E_SHAPE
    assert prefill_varlen(L, b, c, H=0) == E_SHAPE
    assert prefill_varlen(L, b, c, total=-1) == E_SHAPE
    assert prefill_varlen(L, b, c, total=17) == E_SHAPE  # more than S*max_T
    assert prefill_varlen(L, b, c, cu=ctypes.c_void_p(0)) == E_NULL
    assert prefill_varlen(L, b, c, q=ctypes.c_void_p(0)) == E_NULL
    assert prefill_varlen(L, b, c, cu=ctypes.c_void_p(b.new().value + 2)) == E_ALIGN
    q = b.new()
    assert prefill_varlen(L, b, c, q=q, o=q) == E_RANGE
    # seeding needs both rings and pos
    assert prefill_varlen(L, b, c, seed=True, pos=ctypes.c_void_p(0)) == E_NULL
    assert prefill_varlen(L, b, c, seed=True, rv=ctypes.c_void_p(0)) == E_NULL
    r = b.new()
    assert prefill_varlen(L, b, c, seed=True, rk=r, rv=r) == E_RANGE
    assert prefill_varlen(L, b, c, seed=True, pos=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    assert prefill_varlen(L, b, c, seed=True, max_T=0, total=0) == E_SHAPE
    # the table must start at position 0 and cover max_T positions
    t = b.new()
    assert prefill_varlen(L, b, c, rope_applied=0, table=t, tp0=0, tlen=7) == E_RANGE
    assert prefill_varlen(L, b, c, rope_applied=0, table=t, tp0=1, tlen=100) == E_RANGE
    assert b.untouched()


def test_prefill_varlen_empty_is_ok_without_launch(L):
    c = cfg()
    z = ctypes.c_void_p(0)
    assert L.vx_swa_attn_prefill_varlen(z, z, z, z, z, 0, 0, 8, 4, 1, z, 0, 0, z, z, z,
                                        ctypes.byref(c), z) == OK
    assert L.vx_swa_attn_prefill_varlen(z, z, z, z, z, 3, 0, 0, 4, 1, z, 0, 0, z, z, z,
                                        ctypes.byref(c), z) == OK


def stream_step(L, b, c, S=2, n=4, H=2, **ov):
    a = dict(q=b.new(), k=b.new(), v=b.new(), rk=b.new(), rv=b.new(), pos=b.new(), o=b.new())
    a.update(ov)
    return L.vx_swa_attn_stream_step(a["q"], a["k"], a["v"], a["rk"], a["rv"], a["pos"], a["o"],
                                     S, n, H, 0, None if c is None else ctypes.byref(c), None)


def test_stream_step_argument_errors(L):
    b = Bufs()
    c = cfg(window=16)
    assert stream_step(L, b, None) == E_NULL
    assert stream_step(L, b, c, n=0) == E_RANGE
    assert stream_step(L, b, c, n=17) == E_RANGE  # n > W
    assert stream_step(L, b, cfg(window=750), n=65) == E_RANGE  # above the per-step cap
    assert stream_step(L, b, c, S=-1) == E_SHAPE
    assert stream_step(L, b, c, H=0) == E_SHAPE
    assert stream_step(L, b, c, pos=ctypes.c_void_p(0)) == E_NULL
    assert stream_step(L, b, c, rk=ctypes.c_void_p(0)) == E_NULL
    assert stream_step(L, b, c, pos=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    assert stream_step(L, b, c, q=ctypes.c_void_p(b.new().value + 8)) == E_ALIGN
    rk = b.new()
    assert stream_step(L, b, c, rk=rk, o=rk) == E_RANGE
    assert stream_step(L, b, cfg(head_dim=128)) == E_SHAPE
    assert b.untouched()
    z = ctypes.c_void_p(0)
    assert L.vx_swa_attn_stream_step(z, z, z, z, z, z, z, 0, 4, 2, 0, ctypes.byref(c), z) == OK


def test_ring_append_argument_errors(L):
    b = Bufs()
    c = cfg(window=16)

    def call(S=2, n=4, H=2, **ov):
        a = dict(rk=b.new(), rv=b.new(), k=b.new(), v=b.new(), pos=b.new())
        a.update(ov)
        return L.vx_kv_ring_append(a["rk"], a["rv"], a["k"], a["v"], a["pos"], S, n, H, 0,
                                   ctypes.byref(c), None)
    assert call(n=0) == E_RANGE
    assert call(n=17) == E_RANGE
    assert call(pos=ctypes.c_void_p(0)) == E_NULL
    assert call(k=ctypes.c_void_p(b.new().value + 2)) == E_ALIGN
    r = b.new()
    assert call(rk=r, rv=r) == E_RANGE
    assert call(S=-2) == E_SHAPE
    assert b.untouched()


def test_stream_step_append_errors(L):
    b = Bufs()
    c = cfg(window=750)

    def call(S=2, n=4, H=2, **ov):
        a = dict(q=b.new(), k=b.new(), v=b.new(), rk=b.new(), rv=b.new(), pin=b.new(),
                 pout=b.new(), o=b.new())
        a.update(ov)
        return L.vx_swa_attn_stream_step_append(a["q"], a["k"], a["v"], a["rk"], a["rv"], a["pin"],
                                                a["pout"], a["o"], S, n, H, 0, ctypes.byref(c), None)
    assert call(n=17) == E_RANGE  # above the fused cap
    assert call(n=0) == E_RANGE
    p = b.new()
    assert call(pin=p, pout=p) == E_RANGE  # pos_in and pos_out must differ
    assert call(pout=ctypes.c_void_p(0)) == E_NULL
    assert call(pout=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    r = b.new()
    assert call(rk=r, o=r) == E_RANGE
    assert b.untouched()


def test_rope_qk_and_table_errors(L):
    b = Bufs()
    c = cfg()
    z = ctypes.c_void_p(0)
    assert L.vx_rope_qk(z, z, 1, 4, 2, 0, ctypes.byref(c), z) == E_NULL
    q = b.new()
    assert L.vx_rope_qk(q, q, 1, 4, 2, 0, ctypes.byref(c), z) == E_RANGE
    assert L.vx_rope_qk(q, z, 1, 4, 2, ctypes.c_void_p(q.value + 4), ctypes.byref(c), z) == E_ALIGN
    assert L.vx_rope_qk(ctypes.c_void_p(q.value + 4), z, 1, 4, 2, 0, ctypes.byref(c), z) == E_ALIGN
    assert L.vx_rope_qk(q, z, 1, 4, -2, 0, ctypes.byref(c), z) == E_SHAPE
    assert L.vx_rope_table(z, 0, 10, ctypes.byref(c), z) == E_NULL
    assert L.vx_rope_table(q, -1, 10, ctypes.byref(c), z) == E_RANGE
    assert L.vx_rope_table(q, 0, -1, ctypes.byref(c), z) == E_SHAPE
    assert L.vx_rope_table(ctypes.c_void_p(q.value + 4), 0, 3, ctypes.byref(c), z) == E_ALIGN
    assert L.vx_rope_table(q, 0, 3, ctypes.byref(cfg(rope_theta=-1.0)), z) == E_RANGE
    assert L.vx_rope_table(z, 0, 0, ctypes.byref(c), z) == OK
    assert b.untouched()


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        vx.prefill(x, x, x)
    with pytest.raises(ValueError):
        vx.rope_qk(x, None)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(vx, "_lib", None)
    monkeypatch.setattr(vx, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        vx.lib()


# ---------------------------------------------------------------------------
# grouped-query entry points (head_dim 128)
# ---------------------------------------------------------------------------

def gqa_cfg(**kw):
    c = vx._Cfg()
    vx.lib().vx_default_gqa_cfg(ctypes.byref(c))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_default_gqa_cfg(L):
    c = gqa_cfg()
    assert (c.head_dim, c.window, c.rope_theta, c.softmax_scale) == (128, 8192, 1e6, 0.0)
    assert (c.io_dtype, c.out_dtype, c.flags) == (vx.VX_BF16, vx.VX_BF16, 0)


def test_gqa_prefill_argument_errors(L):
    b = Bufs()
    z = ctypes.c_void_p(0)
    c64 = gqa_cfg(window=64)

    def call(B=1, T=8, Hq=4, Hkv=1, pos0=0, rope_applied=1, c=c64, tlen=0, **ov):
        a = dict(q=b.new(), k=b.new(), v=b.new(), o=b.new(), table=z, rk=z, rv=z, pos=z, kr=z)
        a.update(ov)
        return L.vx_gqa_attn_prefill(a["q"], a["k"], a["v"], a["o"], B, T, Hq, Hkv, pos0,
                                     rope_applied, a["table"], 0, tlen, a["rk"], a["rv"], a["pos"],
                                     a["kr"], ctypes.byref(c), None)
    assert call(c=gqa_cfg(head_dim=64)) == E_SHAPE
    assert call(c=gqa_cfg(io_dtype=vx.VX_F32, out_dtype=vx.VX_F32)) == E_DTYPE
    assert call(c=gqa_cfg(out_dtype=5)) == E_DTYPE
    assert call(c=gqa_cfg(flags=1)) == E_RANGE
    assert call(c=gqa_cfg(window=0)) == E_RANGE
    assert call(c=gqa_cfg(softmax_scale=-1.0)) == E_RANGE
    assert call(Hq=6, Hkv=4) == E_SHAPE     # not a multiple
    assert call(Hq=12, Hkv=1) == E_SHAPE    # group of 12 not supported
    assert call(Hkv=0) == E_SHAPE
    assert call(B=-1) == E_SHAPE
    assert call(pos0=-1) == E_RANGE
    assert call(q=z) == E_NULL
    assert call(o=ctypes.c_void_p(b.new().value + 8)) == E_ALIGN
    r = b.new()
    assert call(q=r, o=r) == E_RANGE
    assert call(rope_applied=0) == E_NULL           # no table
    assert call(rope_applied=0, table=b.new(), tlen=4) == E_RANGE  # covers 4 of 8 positions
    assert call(rk=b.new()) == E_NULL                # seeding needs both rings and pos
    assert call(rk=b.new(), rv=b.new(), pos=b.new(), pos0=2) == E_RANGE
    assert call(rk=b.new(), rv=b.new(), pos=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    assert call(kr=b.new()) == E_RANGE                               # k_rot with rope_applied
    t8 = b.new()
    assert call(rope_applied=0, table=t8, tlen=8, kr=ctypes.c_void_p(b.new().value + 2)) == E_ALIGN
    r = b.new()
    assert call(rope_applied=0, table=t8, tlen=8, kr=r, k=r) == E_RANGE   # k_rot overlaps k
    r = b.new()
    assert call(rope_applied=0, table=t8, tlen=8, kr=r, o=r) == E_RANGE
    assert call(B=0) == OK and call(T=0) == OK
    assert L.vx_last_error().decode() == ""
    assert b.untouched()


def test_gqa_decode_argument_errors(L):
    b = Bufs()
    z = ctypes.c_void_p(0)
    c64 = gqa_cfg(window=64)

    def call(S=2, n=1, Hq=4, Hkv=1, c=c64, **ov):
        a = dict(q=b.new(), k=b.new(), v=b.new(), rk=b.new(), rv=b.new(), pin=b.new(),
                 pout=b.new(), o=b.new())
        a.update(ov)
        return L.vx_gqa_attn_decode(a["q"], a["k"], a["v"], a["rk"], a["rv"], a["pin"], a["pout"],
                                    a["o"], S, n, Hq, Hkv, 0, ctypes.byref(c), None)
    assert call(c=gqa_cfg(head_dim=64)) == E_SHAPE
    assert call(c=gqa_cfg(io_dtype=vx.VX_F32, out_dtype=vx.VX_F32)) == E_DTYPE
    assert call(n=0) == E_RANGE
    assert call(n=65) == E_RANGE                 # more than the window
    assert call(n=5) == E_RANGE                  # 5 tokens x 4 heads > 16 columns
    assert call(Hq=16, Hkv=1, n=2) == E_RANGE    # 32 columns
    assert call(Hq=6, Hkv=4) == E_SHAPE
    assert call(S=-1) == E_SHAPE
    p = b.new()
    assert call(pin=p, pout=p) == E_RANGE
    assert call(pout=z) == E_NULL
    assert call(pin=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    assert call(q=ctypes.c_void_p(b.new().value + 2)) == E_ALIGN
    r = b.new()
    assert call(rk=r, o=r) == E_RANGE
    r = b.new()
    assert call(rk=r, rv=r) == E_RANGE
    r = b.new()
    assert call(rv=r, k=r) == E_RANGE            # ring overlaps the new keys
    assert call(S=0) == OK
    assert b.untouched()


def test_rope_table_head_dims(L):
    b = Bufs()
    q = b.new()
    assert L.vx_rope_table(q, 0, 3, ctypes.byref(cfg(head_dim=96)), None) == E_SHAPE
    assert L.vx_rope_table(q, -1, 3, ctypes.byref(gqa_cfg()), None) == E_RANGE
    assert L.vx_rope_table(ctypes.c_void_p(0), 0, 0, ctypes.byref(gqa_cfg()), None) == OK
    assert b.untouched()


# ---------------------------------------------------------------------------
# projections around the encoder's attention
# ---------------------------------------------------------------------------

def test_linear_argument_errors(L):
    b = Bufs()
    z = ctypes.c_void_p(0)

    def call(M=4, N=64, K=128, od=vx.VX_BF16, **ov):
        a = dict(x=b.new(), w=b.new(), bias=z, y=b.new())
        a.update(ov)
        return L.vx_linear(a["x"], a["w"], a["bias"], a["y"], M, N, K, od, None)
    assert call(K=100) == E_SHAPE       # K not a multiple of 128
    assert call(N=48) == E_SHAPE        # N not a multiple of 32
    assert call(N=0) == E_SHAPE
    assert call(M=-1) == E_SHAPE
    assert call(od=7) == E_DTYPE
    assert call(x=z) == E_NULL
    assert call(w=ctypes.c_void_p(b.new().value + 2)) == E_ALIGN
    assert call(bias=ctypes.c_void_p(b.new().value + 2)) == E_ALIGN
    r = b.new()
    assert call(x=r, y=r) == E_RANGE
    assert call(M=0) == OK
    assert b.untouched()


def test_enc_qkv_rope_and_attn_step_errors(L):
    b = Bufs()
    z = ctypes.c_void_p(0)
    c = cfg()

    def qkv(S=2, n=4, H=2, dm=128, cc=c, **ov):
        a = dict(x=b.new(), w=b.new(), bq=z, bv=z, pos=b.new(), q=b.new(), k=b.new(), v=b.new())
        a.update(ov)
        return L.vx_enc_qkv_rope(a["x"], a["w"], a["bq"], a["bv"], a["pos"], S, n, H, dm, a["q"],
                                 a["k"], a["v"], ctypes.byref(cc), None)
    assert qkv(dm=96) == E_SHAPE
    assert qkv(H=1) == E_SHAPE             # H*64 = 64 is not a multiple of 128
    assert qkv(H=0) == E_SHAPE
    assert qkv(n=0) == E_SHAPE
    assert qkv(cc=cfg(io_dtype=vx.VX_F32, out_dtype=vx.VX_F32)) == E_DTYPE
    assert qkv(pos=z) == E_NULL
    assert qkv(pos=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    r = b.new()
    assert qkv(q=r, k=r) == E_RANGE
    r = b.new()
    assert qkv(x=r, v=r) == E_RANGE
    assert qkv(S=0) == OK

    def step(S=2, n=4, H=2, dm=128, cc=c, **ov):
        a = dict(x=b.new(), wqkv=b.new(), bq=z, bv=z, wo=b.new(), bo=z, rk=b.new(), rv=b.new(),
                 pin=b.new(), pout=b.new(), q=b.new(), k=b.new(), v=b.new(), o=b.new(), y=b.new())
        a.update(ov)
        return L.vx_enc_attn_step(a["x"], a["wqkv"], a["bq"], a["bv"], a["wo"], a["bo"], a["rk"],
                                  a["rv"], a["pin"], a["pout"], a["q"], a["k"], a["v"], a["o"],
                                  a["y"], S, n, H, dm, ctypes.byref(cc), None)
    assert step(n=17) == E_RANGE           # above the fused step's 16 frames
    assert step(H=1) == E_SHAPE            # H*64 = 64 is not a multiple of 128
    assert step(dm=200) == E_SHAPE
    p = b.new()
    assert step(pin=p, pout=p) == E_RANGE
    r = b.new()
    assert step(o=r, y=r) == E_RANGE
    r = b.new()
    assert step(q=r, rk=r) == E_RANGE
    assert step(y=z) == E_NULL
    assert step(cc=cfg(flags=1)) == E_RANGE
    assert step(S=0) == OK
    assert b.untouched()


# ---------------------------------------------------------------------------
# the streaming encoder step
# ---------------------------------------------------------------------------

def test_rmsnorm_argument_errors(L):
    b = Bufs()
    z = ctypes.c_void_p(0)

    def call(M=4, dim=128, eps=1e-5, **ov):
        a = dict(x=b.new(), g=b.new(), y=b.new())
        a.update(ov)
        return L.vx_rmsnorm(a["x"], a["g"], a["y"], M, dim, eps, None)
    assert call(dim=12) == E_SHAPE
    assert call(dim=0) == E_SHAPE
    assert call(M=-1) == E_SHAPE
    assert call(eps=-1.0) == E_RANGE
    assert call(eps=float("nan")) == E_RANGE
    assert call(g=z) == E_NULL
    assert call(y=ctypes.c_void_p(b.new().value + 2)) == E_ALIGN
    r = b.new()
    assert call(x=r, y=r) == E_RANGE
    assert call(M=0) == OK
    assert b.untouched()


def _stem_w(b, **ov):
    z = ctypes.c_void_p(0)
    a = dict(w1=b.new(), b1=z, w2=b.new(), b2=z)
    a.update(ov)
    return vx._StemW(*[a[k] for k in vx.STEM_KEYS])


def test_enc_stem_step_argument_errors(L):
    b = Bufs(1 << 18)
    z = ctypes.c_void_p(0)

    def call(S=2, n=2, nm=128, dm=128, w=None, **ov):
        a = dict(mel=b.new(), c1=b.new(), x=b.new())
        a.update(ov)
        w = _stem_w(b) if w is None else w
        return L.vx_enc_stem_step(a["mel"], a["c1"], None if w is False else ctypes.byref(w),
                                  a["x"], S, n, nm, dm, None)
    assert call(nm=100) == E_SHAPE         # 3*n_mels not a multiple of 128
    assert call(dm=200) == E_SHAPE
    assert call(n=0) == E_SHAPE
    assert call(S=-1) == E_SHAPE
    assert call(w=False) == E_NULL
    assert call(w=_stem_w(b, w2=z)) == E_NULL
    assert call(x=z) == E_NULL
    assert call(w=_stem_w(b, b1=ctypes.c_void_p(b.new().value + 2))) == E_ALIGN
    r = b.new()
    assert call(mel=r, c1=r) == E_RANGE
    r = b.new()
    assert call(x=r, w=_stem_w(b, w2=r)) == E_RANGE
    assert call(S=0) == OK
    assert b.untouched()


def _layer_w(b, **ov):
    z = ctypes.c_void_p(0)
    a = {k: (z if k.startswith("b_") else b.new()) for k in vx.LAYER_KEYS}
    a.update(ov)
    return vx._LayerW(*[a[k] for k in vx.LAYER_KEYS])


def _work(b, **ov):
    a = {k: b.new() for k in vx.WORK_KEYS}
    a.update(ov)
    return vx._Work(*[a[k] for k in vx.WORK_KEYS])


def test_enc_layer_step_argument_errors(L):
    b = Bufs(1 << 18)
    z = ctypes.c_void_p(0)
    c = cfg(window=8)

    def call(S=1, n=4, H=2, dm=128, ffn=128, eps=1e-5, cc=c, w=None, wk=None, **ov):
        a = dict(x=b.new(), rk=b.new(), rv=b.new(), pin=b.new(), pout=b.new())
        a.update(ov)
        w = _layer_w(b) if w is None else w
        wk = _work(b) if wk is None else wk
        return L.vx_enc_layer_step(a["x"], None if w is False else ctypes.byref(w), a["rk"],
                                   a["rv"], a["pin"], a["pout"],
                                   None if wk is False else ctypes.byref(wk), S, n, H, dm, ffn,
                                   eps, ctypes.byref(cc), None)
    assert call(n=17, cc=cfg(window=32)) == E_RANGE   # above the fused step's 16 frames
    assert call(n=9) == E_RANGE                        # n > W
    assert call(ffn=100) == E_SHAPE
    assert call(ffn=0) == E_SHAPE
    assert call(H=1) == E_SHAPE                        # H*64 = 64 is not a multiple of 128
    assert call(dm=200) == E_SHAPE
    assert call(eps=-1.0) == E_RANGE
    assert call(eps=float("inf")) == E_RANGE
    assert call(cc=cfg(window=8, flags=1)) == E_RANGE
    assert call(cc=cfg(window=8, io_dtype=vx.VX_F32, out_dtype=vx.VX_F32)) == E_DTYPE
    assert call(w=False) == E_NULL
    assert call(w=_layer_w(b, w_up=z)) == E_NULL
    assert call(w=_layer_w(b, g_ffn=z)) == E_NULL
    assert call(wk=False) == E_NULL
    assert call(wk=_work(b, u=z)) == E_NULL
    assert call(wk=_work(b, o=ctypes.c_void_p(b.new().value + 2))) == E_ALIGN
    assert call(w=_layer_w(b, b_down=ctypes.c_void_p(b.new().value + 4))) == E_ALIGN
    assert call(pin=ctypes.c_void_p(b.new().value + 4)) == E_ALIGN
    p = b.new()
    assert call(pin=p, pout=p) == E_RANGE
    r = b.new()
    assert call(rk=r, rv=r) == E_RANGE
    r = b.new()
    assert call(x=r, wk=_work(b, h=r)) == E_RANGE
    r = b.new()
    assert call(x=r, w=_layer_w(b, w_down=r)) == E_RANGE
    r = b.new()
    assert call(wk=_work(b, q=r, k=r)) == E_RANGE
    assert call(S=0) == OK
    assert b.untouched()


def test_enc_step_argument_errors(L):
    b = Bufs(1 << 18)
    z = ctypes.c_void_p(0)
    c = cfg(window=8)

    def call(S=1, n=2, nm=128, H=2, dm=128, ffn=128, nl=2, layers=None, stem=None, **ov):
        a = dict(mel=b.new(), c1=b.new(), x=b.new(), rk=b.new(), rv=b.new(), pin=b.new(),
                 pout=b.new())
        a.update(ov)
        if layers is None:
            layers = [_layer_w(b) for _ in range(max(nl, 1))]
        arr = (vx._LayerW * len(layers))(*layers) if layers is not False else None
        stem = _stem_w(b) if stem is None else stem
        wk = _work(b)
        return L.vx_enc_step(a["mel"], a["c1"], ctypes.byref(stem), arr, nl, a["rk"], a["rv"],
                             a["pin"], a["pout"], a["x"], ctypes.byref(wk), S, n, nm, H, dm, ffn,
                             1e-5, ctypes.byref(c), None)
    assert call(nl=0) == E_SHAPE
    assert call(nl=5000) == E_SHAPE
    assert call(layers=False) == E_NULL
    assert call(layers=[_layer_w(b), _layer_w(b, w_qkv=z)]) == E_NULL
    assert call(nm=64) == E_SHAPE
    assert call(stem=_stem_w(b, w1=z)) == E_NULL
    r = b.new()
    assert call(mel=r, x=r) == E_RANGE
    r = b.new()
    assert call(c1=r, layers=[_layer_w(b, w_o=r), _layer_w(b)]) == E_RANGE
    assert call(S=0) == OK
    assert b.untouched()
