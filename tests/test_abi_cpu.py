"""The C-ABI library on the host (no GPU needed): it loads, exports every
function the header declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp4.h")

moe = pytest.importorskip("block_scaled_fp4_group_amd")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "extern")))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_fp4_grouped_gemm", "moe_combine", "fp4_transcode_mx_to_nv"):
        assert n in names


def test_every_declared_function_is_exported():
    lib = ctypes.CDLL(moe.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(moe.EXPORTS) == set(names)


def test_every_kernel_launch_stub_is_defined():
    """A kernel template whose host-side instantiation the compiler drops leaves
    its launch stub undefined; the library then fails to load on use."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    undef = subprocess.run(["nm", "-u", moe.LIB_PATH], capture_output=True, text=True, check=True).stdout
    stubs = [l.split()[-1] for l in undef.splitlines() if "__device_stub__" in l]
    assert not stubs, stubs[:4]


def _err(status, expect):
    assert status == expect, (status, moe.lib.moe_last_error())
    assert moe.lib.moe_last_error()


FAKE = ctypes.c_void_p(0x10000)     # an aligned non-null address; never dereferenced on error paths


def test_route_rejects_bad_params():
    for p in [moe.RouteParams(257, 8, 4, 8, 2.827, 1), moe.RouteParams(256, 7, 4, 8, 2.827, 1),
              moe.RouteParams(256, 8, 9, 8, 2.827, 1), moe.RouteParams(256, 8, 4, 17, 2.827, 1),
              moe.RouteParams(32, 8, 1, 5, 2.827, 1), moe.RouteParams(8, 8, 4, 2, 1.0, 1)]:
        _err(moe.lib.moe_route(FAKE, None, 4, ctypes.byref(p), FAKE, FAKE, None), moe.MOE_ERR_INVALID)
    p = moe.RouteParams(256, 8, 4, 8, 2.827, 1)
    _err(moe.lib.moe_route(None, None, 4, ctypes.byref(p), FAKE, FAKE, None), moe.MOE_ERR_INVALID)
    assert moe.lib.moe_route(None, None, 0, ctypes.byref(p), None, None, None) == moe.MOE_OK   # T == 0 no-op
    _err(moe.lib.moe_route(FAKE, None, 4, None, FAKE, FAKE, None), moe.MOE_ERR_INVALID)


def test_permute_workspace_and_limits():
    assert moe.lib.moe_permute_workspace_bytes(16384, 8, 128) >= 64 * 128 * 4
    _err(moe.lib.moe_permute(FAKE, 4096, 8, 256, FAKE, FAKE, FAKE, FAKE, 16, None), moe.MOE_ERR_WORKSPACE)
    _err(moe.lib.moe_permute(FAKE, 4, 8, 2000, FAKE, FAKE, FAKE, None, 0, None), moe.MOE_ERR_INVALID)
    _err(moe.lib.moe_permute(FAKE, 4, 8, 256, None, FAKE, FAKE, None, 0, None), moe.MOE_ERR_INVALID)


def test_route_permute_rejects_bad_arguments():
    def call(p, T=4, logits=FAKE, counter=FAKE, offsets=FAKE):
        return moe.lib.moe_route_permute(logits, None, T, None if p is None else ctypes.byref(p), FAKE, FAKE,
                                         offsets, FAKE, FAKE, counter, None, 0, None)
    good = moe.RouteParams(256, 8, 4, 8, 2.827, 1)
    for p in [moe.RouteParams(257, 8, 4, 8, 2.827, 1), moe.RouteParams(256, 7, 4, 8, 2.827, 1),
              moe.RouteParams(256, 8, 4, 17, 2.827, 1), None]:
        _err(call(p), moe.MOE_ERR_INVALID)
    _err(call(good, counter=None), moe.MOE_ERR_INVALID)
    _err(call(good, counter=ctypes.c_void_p(0x10002)), moe.MOE_ERR_INVALID)    # not 4-byte aligned
    _err(call(good, logits=None), moe.MOE_ERR_INVALID)
    _err(call(good, offsets=None), moe.MOE_ERR_INVALID)
    _err(call(good, T=-1), moe.MOE_ERR_INVALID)
    # above 2048 slots (two launches): pointers and the permutation workspace are checked before either launch
    _err(moe.lib.moe_route_permute(None, None, 4096, ctypes.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                                   None), moe.MOE_ERR_INVALID)
    _err(moe.lib.moe_route_permute(FAKE, None, 4096, ctypes.byref(good), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16,
                                   None), moe.MOE_ERR_WORKSPACE)


def _w(fmt=moe.MOE_FP4_MX, E=4, n=256, k=512, glob=None):
    return moe.Fp4Weights(fmt, E, n, k, 0x10000, 0x20000, glob)


def _gemm(act, w0, w1, epi=moe.MOE_EPI_SWIGLU, rows=8, out=None, algo=0):
    out = out or moe.Out(0x30000, None, None, 1.0)
    return moe.lib.moe_fp4_grouped_gemm(ctypes.byref(act), ctypes.byref(w0), None if w1 is None else ctypes.byref(w1),
                                        epi, FAKE, rows, ctypes.byref(out), algo, None)


def test_gemm_rejects_bad_arguments():
    act = moe.Act(moe.MOE_ACT_BF16, 0x40000, None, 1.0, None, 1, 8)
    _err(_gemm(act, _w(k=160), _w(k=160)), moe.MOE_ERR_UNSUPPORTED)          # k % 128
    _err(_gemm(act, _w(), _w(n=128)), moe.MOE_ERR_INVALID)                     # w0 / w1 differ
    _err(_gemm(act, _w(), None), moe.MOE_ERR_INVALID)                          # SwiGLU needs w1
    _err(_gemm(act, _w(fmt=moe.MOE_FP4_NV), _w(fmt=moe.MOE_FP4_NV)), moe.MOE_ERR_INVALID)   # NV without global
    bad = moe.Act(moe.MOE_ACT_NVFP4, 0x40000, 0x50000, 3.0, None, 1, 8)
    _err(_gemm(bad, _w(), _w()), moe.MOE_ERR_INVALID)                          # non power-of-two input scale
    unal = moe.Act(moe.MOE_ACT_BF16, 0x40008, None, 1.0, None, 1, 8)
    _err(_gemm(unal, _w(), _w()), moe.MOE_ERR_INVALID)                         # misaligned activations
    _err(_gemm(act, _w(), _w(), out=moe.Out(None, None, None, 1.0)), moe.MOE_ERR_INVALID)   # no output
    _err(_gemm(act, _w(), _w(), algo=7), moe.MOE_ERR_INVALID)
    assert _gemm(act, _w(), _w(), rows=0) == moe.MOE_OK                        # zero rows: no-op


def test_combine_transcode_quant_reject():
    _err(moe.lib.moe_combine(FAKE, FAKE, FAKE, None, 4, 8, 12, FAKE, None), moe.MOE_ERR_INVALID)   # h % 8
    _err(moe.lib.moe_combine(None, FAKE, FAKE, None, 4, 8, 16, FAKE, None), moe.MOE_ERR_INVALID)
    cnt = ctypes.c_void_p(0x60000)
    _err(moe.lib.fp4_transcode_mx_to_nv(FAKE, FAKE, 2, 16, 48, FAKE, FAKE, cnt, None), moe.MOE_ERR_INVALID)
    _err(moe.lib.fp4_transcode_mx_to_nv(FAKE, FAKE, 2, 8, 64, FAKE, FAKE, cnt, None), moe.MOE_ERR_INVALID)
    _err(moe.lib.fp4_transcode_mx_to_nv(FAKE, FAKE, 2, 16, 64, FAKE, FAKE, None, None), moe.MOE_ERR_INVALID)
    _err(moe.lib.moe_quantize_nvfp4(FAKE, 4, 48, 1.0, FAKE, FAKE, None, None), moe.MOE_ERR_INVALID)
    _err(moe.lib.moe_quantize_nvfp4(FAKE, 4, 64, 0.3, FAKE, FAKE, None, None), moe.MOE_ERR_INVALID)
    assert moe.lib.moe_quantize_nvfp4(None, 0, 64, 1.0, None, None, None, None) == moe.MOE_OK


def test_status_strings():
    for s in range(5):
        assert moe.lib.moe_status_string(s)


def test_tile_weights_rejects_bad_arguments():
    t = moe.lib.moe_fp4_tile_weights
    A, B, C, D = (ctypes.c_void_p(0x100000 * i) for i in (1, 2, 3, 4))
    _err(t(moe.MOE_FP4_MX, 2, 250, 512, A, B, C, D, None), moe.MOE_ERR_INVALID)     # n % 16
    _err(t(moe.MOE_FP4_MX, 2, 256, 640, A, B, C, D, None), moe.MOE_ERR_INVALID)     # k % 512
    _err(t(7, 2, 256, 512, A, B, C, D, None), moe.MOE_ERR_INVALID)                  # format
    _err(t(moe.MOE_FP4_MX, 2, 256, 512, A, B, None, D, None), moe.MOE_ERR_INVALID)  # NULL
    _err(t(moe.MOE_FP4_MX, 2, 256, 512, A, B, A, D, None), moe.MOE_ERR_INVALID)     # in place
    # codes [2, 256, 256] = 128 KiB from 0x100000: an output starting inside them overlaps
    _err(t(moe.MOE_FP4_MX, 2, 256, 512, A, B, ctypes.c_void_p(0x100000 + 0x10000), D, None), moe.MOE_ERR_INVALID)
    assert t(moe.MOE_FP4_MX, 0, 256, 512, None, None, None, None, None) == moe.MOE_OK   # no experts: no-op


def test_gemm_checks_the_tiled_layout():
    act = moe.Act(moe.MOE_ACT_BF16, 0x40000, None, 1.0, None, 1, 8)
    w = moe.Fp4Weights(moe.MOE_FP4_MX, 4, 256, 640, 0x10000, 0x20000, None, moe.MOE_FP4_TILED)
    _err(_gemm(act, w, w), moe.MOE_ERR_INVALID)                                  # tiled needs k % 512
    w0 = moe.Fp4Weights(moe.MOE_FP4_MX, 4, 256, 512, 0x10000, 0x20000, None, moe.MOE_FP4_TILED)
    w1 = moe.Fp4Weights(moe.MOE_FP4_MX, 4, 256, 512, 0x10000, 0x20000, None, 0)
    _err(_gemm(act, w0, w1), moe.MOE_ERR_INVALID)                                # w0 / w1 layouts differ
    _err(_gemm(act, w0, w0, algo=3), moe.MOE_ERR_INVALID)                        # bad algo (no kernel 3)
    _err(_gemm(act, w0, w0, algo=4), moe.MOE_ERR_INVALID)


def test_route_permute_noalloc_rejects_before_touching_the_gpu():
    """Bad parameters, NULL pointers and batches beyond the static scratch are
    refused on the host (no HIP call is made on these paths)."""
    p = moe.RouteParams(256, 8, 4, 8, 2.827, 1)
    bad = moe.RouteParams(256, 7, 4, 8, 2.827, 1)
    f = moe.lib.moe_route_permute_noalloc
    _err(f(FAKE, None, 4, ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None), moe.MOE_ERR_INVALID)
    _err(f(FAKE, None, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, None), moe.MOE_ERR_INVALID)
    _err(f(None, None, 4, ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None), moe.MOE_ERR_INVALID)
    _err(f(FAKE, None, 4, ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None), moe.MOE_ERR_INVALID)
    too_many = (1 << 27) // (256 * 8) + 1
    _err(f(FAKE, None, too_many, ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None), moe.MOE_ERR_UNSUPPORTED)


def test_compact_format_checks():
    """Compact (MXC) weights: base scales required, k % 512, weight-streaming
    kernel only; the converter checks sizes, pointers and alignment."""
    act = moe.Act(moe.MOE_ACT_BF16, 0x40000, None, 1.0, None, 1, 8)
    G = ctypes.c_void_p(0x70000)
    wc = moe.Fp4Weights(moe.MOE_FP4_MXC, 4, 256, 512, 0x10000, 0x20000, G)
    _err(_gemm(act, _w(fmt=moe.MOE_FP4_MXC), _w(fmt=moe.MOE_FP4_MXC)), moe.MOE_ERR_INVALID)   # no base
    w640 = moe.Fp4Weights(moe.MOE_FP4_MXC, 4, 256, 640, 0x10000, 0x20000, G)
    _err(_gemm(act, w640, w640), moe.MOE_ERR_UNSUPPORTED)                        # k % 512
    _err(_gemm(act, wc, wc, algo=moe.MOE_ALGO_PREFILL), moe.MOE_ERR_UNSUPPORTED)
    mx8 = moe.Act(moe.MOE_ACT_MXFP8, 0x40000, 0x50000, 1.0, None, 1, 8)
    _err(_gemm(mx8, wc, wc), moe.MOE_ERR_UNSUPPORTED)                            # block-scaled MFMA modes
    sq = moe.Out(0x30000, None, None, 1.0, None, 0, 0x60000)
    _err(_gemm(act, wc, None, epi=moe.MOE_EPI_NONE, out=sq), moe.MOE_ERR_UNSUPPORTED)   # row_sumsq
    flagged = moe.Fp4Weights(moe.MOE_FP4_MXC, 4, 256, 512, 0x10000, 0x20000, G, moe.MOE_FP4_SCALES_POW2)
    _err(_gemm(act, flagged, flagged), moe.MOE_ERR_INVALID)                      # NV-only flags
    assert _gemm(act, wc, wc, rows=0) == moe.MOE_OK
    c = moe.lib.moe_fp4_compact_mx
    cnt = ctypes.c_void_p(0x60000)
    _err(c(FAKE, FAKE, 2, 256, 640, FAKE, FAKE, cnt, None), moe.MOE_ERR_INVALID)     # k % 512
    _err(c(FAKE, FAKE, 2, 250, 512, FAKE, FAKE, cnt, None), moe.MOE_ERR_INVALID)     # n % 16
    _err(c(FAKE, FAKE, 2, 256, 512, FAKE, FAKE, None, None), moe.MOE_ERR_INVALID)    # counters
    _err(c(FAKE, None, 2, 256, 512, FAKE, FAKE, cnt, None), moe.MOE_ERR_INVALID)     # NULL
    _err(c(ctypes.c_void_p(0x10008), FAKE, 2, 256, 512, FAKE, FAKE, cnt, None), moe.MOE_ERR_INVALID)
    _err(moe.lib.moe_fp4_tile_weights(moe.MOE_FP4_MXC, 2, 256, 640, FAKE, FAKE, FAKE, FAKE, None),
         moe.MOE_ERR_INVALID)


def test_header_is_plain_c():
    """include/moe_fp4.h compiles as C99 in a C translation unit (no C++ or
    torch types cross the boundary) and links against the library."""
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    hip_inc = "/opt/rocm/include"
    if gcc is None or not os.path.isdir(hip_inc):
        pytest.skip("needs gcc and the HIP headers")
    src = ("#include \"moe_fp4.h\"\n"
           "int main(void) {\n"
           "  moe_fp4_weights w = {MOE_FP4_MXC, 1, 16, 512, 0, 0, 0, 0};\n"
           "  moe_route_params p = {256, 8, 4, 8, 2.827f, 1};\n"
           "  (void)w; (void)p;\n"
           "  return moe_status_string(MOE_OK) ? 0 : 1;\n"
           "}\n")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "use.c")
        with open(c, "w") as f:
            f.write(src)
        out = os.path.join(d, "use")
        r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I",
                            os.path.join(ROOT, "include"), "-I", hip_inc, c, "-o", out, moe.LIB_PATH,
                            "-Wl,-rpath," + os.path.dirname(moe.LIB_PATH), "-Wl,--allow-shlib-undefined"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
