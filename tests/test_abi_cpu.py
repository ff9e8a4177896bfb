"""The C ABI on the CPU: the library loads, exports what pa.h declares, and
rejects every invalid argument before any GPU work (no compute calls)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
LIB = os.path.join(ROOT, "paged_kv_cache_decode_amd", "libpa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_exports_match_header():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    pa_exported = sorted(s for s in exported if s.startswith("pa_"))
    assert pa_exported == declared_functions()


def test_header_compiles_as_c_and_cpp(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "pa.h"\nint main(void){pa_tensor t; (void)t; return 0;}\n')
    for comp in (["gcc", "-std=c99"], ["g++", "-x", "c++", "-std=c++17"]):
        subprocess.run([*comp, "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c",
                        str(src), "-o", str(tmp_path / "t.o")], check=True)


# ---------------------------------------------------------------------------
# Validation through the real library with fake (never dereferenced) pointers
# ---------------------------------------------------------------------------

from paged_kv_cache_decode_amd import binding as B  # noqa: E402

FAKE = 0x10000
GAP = 1 << 40  # fake device addresses far enough apart never to overlap


def T(shape, dtype, data=FAKE, stride=None):
    d = B.PaTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    st = stride or [0] * len(shape)
    if stride is None:
        acc = 1
        for i in range(len(shape) - 1, -1, -1):
            st[i] = acc
            acc *= shape[i]
    for i, s in enumerate(shape):
        d.shape[i] = s
        d.stride[i] = st[i]
    return d


def decode_args(S=4, H=32, Hkv=8, d=128, NB=100, Bs=16, MB=8, dt=B.PA_BF16, out_dt=B.PA_F32):
    return dict(q=T([S, H, d], dt, GAP), k=T([NB, Bs, Hkv, d], dt, 2 * GAP),
                v=T([NB, Bs, Hkv, d], dt, 3 * GAP), bt=T([S, MB], B.PA_I32, 4 * GAP),
                cl=T([S], B.PA_I32, 5 * GAP), out=T([S, H, d], out_dt, 6 * GAP))


def call_decode(a, scale=0.1):
    L = B.lib()
    r = ctypes.byref
    return L.pa_decode(r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["cl"]),
                       ctypes.c_float(scale), r(a["out"]), None)


def plan(a):
    info = B.PaDecodePlanInfo()
    r = ctypes.byref
    st = B.lib().pa_decode_plan(r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["cl"]),
                                r(a["out"]), r(info))
    return st, info


def test_status_strings():
    L = B.lib()
    for s in range(-8, 1):
        assert L.pa_status_string(s).decode().startswith(B.STATUS[s])


@pytest.mark.parametrize("mutate,status", [
    (lambda a: a.update(q=None), -1),
    (lambda a: setattr(a["k"], "data", None), -1),
    (lambda a: setattr(a["bt"], "dtype", B.PA_F32), -2),
    (lambda a: setattr(a["out"], "dtype", B.PA_F16), -2),
    (lambda a: setattr(a["q"], "dtype", B.PA_I32), -2),
    (lambda a: setattr(a["cl"], "ndim", 2), -3),
    (lambda a: a["q"].shape.__setitem__(1, 30), -3),
    (lambda a: a["v"].shape.__setitem__(2, 4), -3),
    (lambda a: a["k"].stride.__setitem__(0, 99999), -4),
    (lambda a: setattr(a["q"], "data", GAP + 2), -4),
    (lambda a: a["q"].stride.__setitem__(2, 2), -4),
    (lambda a: a.update(decode_args(d=96)), -5),
    (lambda a: a.update(decode_args(Bs=8)), -5),
    (lambda a: a.update(decode_args(Hkv=2)), -5),  # G = 16
    (lambda a: a.update(decode_args(H=24, Hkv=8)), -5),
    (lambda a: setattr(a["out"], "data", 2 * GAP + 4096), -8),
])
def test_decode_rejects(mutate, status):
    a = decode_args()
    mutate(a)
    if a["q"] is None:
        L = B.lib()
        r = ctypes.byref
        st = L.pa_decode(None, r(a["k"]), r(a["v"]), r(a["bt"]), r(a["cl"]), ctypes.c_float(1),
                         r(a["out"]), None)
    else:
        st = call_decode(a)
    assert st == status, B.lib().pa_last_error()
    assert B.lib().pa_last_error().decode()


def test_decode_rejects_nan_scale():
    assert call_decode(decode_args(), scale=float("nan")) == -8


def test_decode_plan_math(monkeypatch):
    monkeypatch.delenv("PA_DECODE_WORKERS", raising=False)
    st, info = plan(decode_args(S=64, MB=256))
    assert st == 0
    W = info.workers
    assert W > 0 and info.waves_per_group == 4 and info.block_threads == 256
    assert tuple(info.grid) == (-(-W // 32) * 8, 1, 1)  # groups, a multiple of 8
    G, d, S, Hkv = 4, 128, 64, 8
    slots = W + S * Hkv
    counters = -(-S * Hkv * 4 // 256) * 256  # per-unit counters, padded to 256 bytes
    assert info.workspace_bytes == counters + slots * G * d * 4 + slots * G * 4
    # A long-context shape: 4 x 100,000 keys (6,250 blocks of 16); 64-bit sizes.
    st, info = plan(decode_args(S=4, MB=6250, NB=31250))
    assert st == 0


def test_worker_override(monkeypatch):
    monkeypatch.setenv("PA_DECODE_WORKERS", "7")
    st, info = plan(decode_args(S=2, MB=64))
    assert st == 0 and info.workers == 7 and tuple(info.grid) == (8, 1, 1)
    monkeypatch.setenv("PA_DECODE_WORKERS", "0")
    assert plan(decode_args())[0] == -8
    monkeypatch.setenv("PA_DECODE_WORKERS", "x")
    assert plan(decode_args())[0] == -8


def test_forced_alloc_failure(monkeypatch):
    """The workspace-allocation failure path, forced from the host."""
    monkeypatch.setenv("PA_TEST_FAIL_ALLOC", "1")
    monkeypatch.setenv("PA_DECODE_WORKERS", "64")
    a = decode_args(S=2, MB=64)
    assert call_decode(a) == -6
    assert "PA_TEST_FAIL_ALLOC" in B.lib().pa_last_error().decode()


def prefill_args(S=2, T_=100, H=8, Hkv=2, d=128, NB=20, Bs=16, MB=8, dt=B.PA_BF16):
    return dict(q=T([T_, H, d], dt, GAP), k=T([NB, Bs, Hkv, d], dt, 2 * GAP),
                v=T([NB, Bs, Hkv, d], dt, 3 * GAP), bt=T([S, MB], B.PA_I32, 4 * GAP),
                cl=T([S], B.PA_I32, 5 * GAP), qsl=T([S + 1], B.PA_I32, 6 * GAP),
                out=T([T_, H, d], B.PA_F32, 7 * GAP))


def call_prefill(a, maxq=64, causal=1, scale=0.1):
    r = ctypes.byref
    return B.lib().pa_prefill(r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["cl"]),
                              r(a["qsl"]), maxq, ctypes.c_float(scale), causal, r(a["out"]), None)


@pytest.mark.parametrize("mutate,kw,status", [
    (lambda a: a["qsl"].shape.__setitem__(0, 2), {}, -3),
    (lambda a: None, {"causal": 2}, -8),
    (lambda a: None, {"maxq": -1}, -8),
    (lambda a: (setattr(a["q"], "dtype", B.PA_F32), setattr(a["k"], "dtype", B.PA_F32),
                setattr(a["v"], "dtype", B.PA_F32)), {}, -5),
    (lambda a: a.update(prefill_args(d=64)), {}, -5),
    (lambda a: setattr(a["qsl"], "dtype", B.PA_F32), {}, -2),
])
def test_prefill_rejects(mutate, kw, status):
    a = prefill_args()
    mutate(a)
    assert call_prefill(a, **kw) == status, B.lib().pa_last_error()


def test_write_kv_rejects():
    r = ctypes.byref
    kn = T([10, 8, 128], B.PA_BF16, GAP)
    vn = T([10, 8, 128], B.PA_BF16, 2 * GAP)
    sm = T([9], B.PA_I32, 3 * GAP)
    kp = T([4, 16, 8, 128], B.PA_BF16, 4 * GAP)
    vp = T([4, 16, 8, 128], B.PA_BF16, 5 * GAP)
    assert B.lib().pa_write_kv(r(kn), r(vn), r(sm), r(kp), r(vp), None) == -3
    sm = T([10], B.PA_I32, 3 * GAP)
    kp2 = T([4, 16, 8, 128], B.PA_F16, 4 * GAP)
    assert B.lib().pa_write_kv(r(kn), r(vn), r(sm), r(kp2), r(vp), None) == -2


def head_major(t, NB=100, Bs=16, Hkv=8, d=128):
    """The same logical [NB, B, Hkv, d] pool with head-major blocks: strides
    of a contiguous [NB, Hkv, B, d] buffer."""
    for i, s in enumerate([Bs * Hkv * d, d, Bs * d, 1]):
        t.stride[i] = s
    return t


def test_pool_layouts():
    """Both pool layouts plan; other strides, or K and V in different
    layouts, are rejected before any GPU work."""
    a = decode_args()
    head_major(a["k"]), head_major(a["v"])
    assert plan(a)[0] == 0
    b = decode_args()
    head_major(b["k"])  # K head-major, V token-major
    assert call_decode(b) == -4
    assert "same layout" in B.lib().pa_last_error().decode()
    c = decode_args()
    for t in (c["k"], c["v"]):
        head_major(t)
        t.stride[1], t.stride[2] = 2 * 128, 16 * 128  # rows of a head not adjacent
    assert call_decode(c) == -4


def test_decode_lse_and_merge_reject():
    """pa_decode_lse checks its lse output, pa_merge_states its parts, before
    any GPU work."""
    L = B.lib()
    r = ctypes.byref
    a = decode_args(S=4, H=32)
    bad = [(T([4, 32], B.PA_F16, 7 * GAP), -2),            # not f32
           (T([4, 31], B.PA_F32, 7 * GAP), -3),            # wrong shape
           (T([4, 32], B.PA_F32, 7 * GAP, [1, 4]), -4),    # last dim not contiguous
           (T([4, 32], B.PA_F32, 6 * GAP), -8)]            # aliases out
    for lse, status in bad:
        st = L.pa_decode_lse(r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["cl"]),
                             ctypes.c_float(0.1), r(a["out"]), r(lse), None)
        assert st == status, L.pa_last_error()
    assert L.pa_decode_lse(r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["cl"]),
                           ctypes.c_float(0.1), r(a["out"]), None, None) == -1
    P, S, H, d = 3, 4, 8, 128
    po, pl = T([P, S, H, d], B.PA_F32, GAP), T([P, S, H], B.PA_F32, 2 * GAP)
    out = T([S, H, d], B.PA_BF16, 3 * GAP)
    cases = [(T([P, S, H, d], B.PA_F16, GAP), pl, out, -2),
             (po, T([P, S, H + 1], B.PA_F32, 2 * GAP), out, -3),
             (po, pl, T([S, H, 64], B.PA_F32, 3 * GAP), -3),
             (T([P, S, H, 96], B.PA_F32, GAP), pl, T([S, H, 96], B.PA_F32, 3 * GAP), -5),
             (T([0, S, H, d], B.PA_F32, GAP), T([0, S, H], B.PA_F32, 2 * GAP), out, -3),
             (po, pl, T([S, H, d], B.PA_F32, GAP + 64), -8)]
    for po_, pl_, out_, status in cases:
        st = L.pa_merge_states(r(po_), r(pl_), r(out_), None, None)
        assert st == status, L.pa_last_error()


def test_decode_noalloc_rejects_what_its_fixed_workspace_cannot_hold(monkeypatch):
    """pa_decode_noalloc validates like pa_decode, then refuses calls whose
    counters or partial results exceed its fixed per-GPU array -- before any
    device work (fake pointers here)."""
    L = B.lib()
    r = ctypes.byref

    def call(a):
        return L.pa_decode_noalloc(r(a["q"]), r(a["k"]), r(a["v"]), r(a["bt"]), r(a["cl"]),
                                   ctypes.c_float(0.1), r(a["out"]), None)

    a = decode_args()
    a["bt"].dtype = B.PA_F32
    assert call(a) == -2  # the same validation as pa_decode
    assert call(decode_args(S=9000, H=8, Hkv=8)) == -6  # 72,000 (sequence, KV head) pairs
    assert "fixed workspace" in L.pa_last_error().decode()
    monkeypatch.setenv("PA_DECODE_WORKERS", "100000")  # 100,032 partial slots of 2,064 bytes
    assert call(decode_args()) == -6


def test_measurement_aids_reject_bad_arguments():
    """pa_clock_probe and pa_profiler_samples check their arguments before
    any device work; the profiler reads need no GPU."""
    L = B.lib()
    assert L.pa_clock_probe(1000, None, None) == -1
    assert L.pa_clock_probe(0, ctypes.c_void_p(FAKE), None) == -8
    assert L.pa_clock_probe(100000001, ctypes.c_void_p(FAKE), None) == -8
    assert L.pa_clock_probe(1000, ctypes.c_void_p(FAKE + 4), None) == -4
    assert L.pa_profiler_samples(b"decode_partitions", None, 4) == -1
    buf = (ctypes.c_float * 4)()
    assert L.pa_profiler_samples(b"decode_partitions", buf, -1) == -8
    assert L.pa_profiler_samples(b"no_such_kernel", buf, 4) == 0
    assert B.profiler_samples("no_such_kernel") == []
