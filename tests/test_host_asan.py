"""The library's host code under AddressSanitizer (CPU, no GPU needed).

The library is rebuilt with its host side instrumented
(build.build_host_asan) and loaded, with the sanitizer runtime preloaded, in
a Python process that does not import torch. It then runs every host entry
point on inputs that stop at a host check: argument errors, envelope limits,
extreme sizes for the workspace formulas, the predicates and the status text.
Any out-of-bounds access or use after free on the host aborts that process.
No call reaches a device.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "sparse_embedding_weight_amd"))
import build  # noqa: E402  (the package's build script)

SCRIPT = r'''
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
def sig(name, args, res=i32):
    f = getattr(lib, name); f.argtypes = args; f.restype = res; return f
pos_bits = sig("ewg_position_bits", [i64])
can = sig("can_accumulate_embedding_wgrad", [i64, i64, i64, i32, i32, i32])
wsb = sig("accumulate_embedding_wgrad_workspace_bytes", [i64, i64], sz)
ACC = [vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, i32, vp, sz, vp]
acc = sig("accumulate_embedding_wgrad", ACC)
acc_t = sig("accumulate_embedding_wgrad_timed", ACC + [vp])
no_alloc = sig("accumulate_embedding_wgrad_no_alloc", ACC[:11] + [vp])
can_s = sig("can_accumulate_embedding_wgrad_vocab_shard", [i64, i64, i64, i64, i32, i32, i32])
shard = sig("accumulate_embedding_wgrad_vocab_shard",
            [vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, i32, vp, sz, vp])
sort = sig("accumulate_embedding_wgrad_sort_tokens", [vp, i64, i64, i32] + [vp] * 6 + [vp, sz, vp])
can_m = sig("can_accumulate_embedding_wgrad_many_tokens", [i64, i64, i64, i32, i32, i32])
wsb_m = sig("accumulate_embedding_wgrad_many_tokens_workspace_bytes", [i64, i64], sz)
many = sig("accumulate_embedding_wgrad_many_tokens", ACC)
many_t = sig("accumulate_embedding_wgrad_many_tokens_timed", ACC + [vp])
status = sig("ewg_status_string", [i32], ctypes.c_char_p)
I32, I64, BF16, F32 = 0, 1, 2, 3
OK, UNSUPPORTED, INVALID, WS_SMALL = 0, 1, 2, 3

for n in (-1, 0, 1, 2, 3072, 3073, 4096, 4097, 8192, 8193, 1 << 40):
    pos_bits(n)
for n in (0, 3072, 3073, 8192, 8193, -5):
    for h in (0, 1, 7168, 1 << 40):
        for v in (0, 1, 129280, 1 << 31, -1):
            can(n, h, v, I32, BF16, F32)
            wsb(n, h)
            can_m(n, h, v, I64, F32, BF16)
            wsb_m(n, h)
for n in (8193, 131072, 131073, 1 << 40):
    for h in (1, 7168, 1 << 20, 1 << 40, -1):
        wsb_m(n, h)
        can_m(n, h, 129280, I32, BF16, F32)
assert can(8192, 7168, 129280, I32, BF16, F32) == 1 and can(3072, 7168, 100, I32, BF16, F32) == 0
assert can(8192, 7168, 100, 7, BF16, F32) == 0 and can(8192, 7168, 100, I32, I32, F32) == 0

def call(f, **kw):
    a = dict(ids=8, grad=16, main_grad=32, n=4096, h=64, v=100, gs=64, ms=64,
             i=I32, g=BF16, m=F32, ws=256 * 1024, wsb=1 << 30, stream=None)
    a.update(kw)
    return f(a["ids"], a["grad"], a["main_grad"], a["n"], a["h"], a["v"], a["gs"], a["ms"],
             a["i"], a["g"], a["m"], a["ws"], a["wsb"], a["stream"])

for f in (acc, many):
    assert call(f, i=7) == INVALID and call(f, g=-1) == INVALID and call(f, m=99) == INVALID
    for ptr in ("ids", "grad", "main_grad", "ws"):
        assert call(f, **{ptr: None}) == INVALID
    assert call(f, gs=63) == INVALID and call(f, ms=10) == INVALID
    assert call(f, ws=256 * 1024 + 8) == INVALID
    assert call(f, n=-1) == UNSUPPORTED and call(f, h=0) == UNSUPPORTED
assert call(acc, n=3072) == UNSUPPORTED and call(acc, n=8193) == UNSUPPORTED
assert call(acc, v=1 << 20, n=8192) == UNSUPPORTED
assert call(acc, wsb=wsb(4096, 64) - 1) == WS_SMALL
assert call(many, n=131073) == UNSUPPORTED and call(many, v=(1 << 18) + 1) == UNSUPPORTED
assert call(many, n=20000, wsb=wsb_m(20000, 64) - 1) == WS_SMALL
ev = (ctypes.c_void_p * 4)()
assert acc_t(8, 16, 32, 4096, 64, 100, 64, 64, I32, BF16, F32, 256 * 1024, 1 << 30, None, None) == INVALID
assert acc_t(8, 16, 32, 100, 64, 100, 64, 64, I32, BF16, F32, 256 * 1024, 1 << 30, None, ev) == UNSUPPORTED
assert many_t(8, 16, 32, 20000, 64, 100, 64, 64, I32, BF16, F32, 256 * 1024, 1 << 40, None, None) == INVALID
assert no_alloc(8, 8, 8, 3072, 128, 512, 128, 128, I32, BF16, F32, None) == UNSUPPORTED
assert no_alloc(None, 8, 8, 8192, 128, 512, 128, 128, I32, BF16, F32, None) == INVALID
assert no_alloc(8, 8, 8, 8192, 128, 512, 127, 128, I32, BF16, F32, None) == INVALID
assert can_s(8192, 7168, 0, (1 << 18) - 1, I32, BF16, F32) == 1
assert can_s(8192, 7168, -1, 100, I32, BF16, F32) == 0 and can_s(8192, 7168, 0, 1 << 18, I32, BF16, F32) == 0
def sh(**kw):
    a = dict(ids=8, grad=16, main_grad=32, n=4096, h=64, start=1000, rows=100, gs=64, ms=64,
             i=I32, g=BF16, m=F32, ws=256 * 1024, wsb=1 << 30)
    a.update(kw)
    return shard(a["ids"], a["grad"], a["main_grad"], a["n"], a["h"], a["start"], a["rows"],
                 a["gs"], a["ms"], a["i"], a["g"], a["m"], a["ws"], a["wsb"], None)
assert sh(start=-5) == UNSUPPORTED and sh(rows=0) == UNSUPPORTED and sh(i=9) == INVALID
assert sh(ids=None) == INVALID and sh(gs=10) == INVALID and sh(ws=256 * 1024 + 4) == INVALID
assert sh(wsb=wsb(4096, 64) - 1) == WS_SMALL
assert sort(8, 4096, 100, 5, *([8] * 6), 256 * 1024, 1 << 30, None) == INVALID
assert sort(8, 100, 100, 0, *([8] * 6), 256 * 1024, 1 << 30, None) == UNSUPPORTED
assert sort(8, 4096, 100, 0, *([8] * 5), None, 256 * 1024, 1 << 30, None) == INVALID
assert sort(8, 4096, 100, 0, *([8] * 6), 256 * 1024, 100, None) == WS_SMALL
for code in range(-20, 21):
    assert len(status(code)) > 0
print("host checks ok")
'''


@pytest.fixture(scope="module")
def asan_library():
    runtime = build.asan_runtime()
    if not runtime:
        pytest.skip("the compiler's shared AddressSanitizer runtime is not installed")
    return build.build_host_asan(), runtime


def test_host_entry_points_under_address_sanitizer(asan_library):
    library, runtime = asan_library
    # the host code is instrumented: it calls the sanitizer's access checks
    syms = subprocess.run(["nm", "-D", "--undefined-only", library], capture_output=True,
                          text=True, check=True).stdout
    assert "__asan_report_load" in syms and "__asan_report_store" in syms
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    r = subprocess.run([sys.executable, "-c", SCRIPT, library], capture_output=True, text=True,
                       env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host checks ok" in r.stdout
