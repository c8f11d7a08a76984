"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/pkv.h declares, and its host-side validation rejects bad arguments
(and accepts empty work) before any HIP call is made."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

import paged_quantized_kv_amd as pkv  # noqa: E402

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EALIGN = 0, -1, -2, -3
A = 1 << 20  # a 16-byte aligned fake device address; never dereferenced


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:PKV_API\s+)?(?:int64_t|int|const char \*)\s*(pkv_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for s in ("pkv_gather_indexer_k_fp8", "pkv_store_indexer_k_fp8", "pkv_store_kv_fp4",
              "pkv_gather_indexer_k_dequant", "pkv_gather_kv_fp4_dequant",
              "pkv_fp8_mqa_logits", "pkv_paged_attention_decode", "pkv_last_error",
              "pkv_abi_version"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pkv.library_path())
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)$", out, re.M))
    for s in declared_symbols():
        assert s in exported, s
        assert getattr(lib, s) is not None
    assert pkv.abi_version() == 6
    # nothing else of the library is exported (the compiler's own
    # per-translation-unit ids aside)
    others = [name for name in re.findall(r"^\S*\s*\S+ (\S+)$", out, re.M)
              if not name.startswith(("pkv_", "__hip_cuid_"))]
    assert others == [], others


def lib():
    return pkv._lib


def last_error():
    return lib().pkv_last_error().decode()


def gather(**kw):
    a = dict(kv_cache=A, k_fp8=A, k_scale=A, block_table=A, cu=A, R=2, maxb=4, T=57, nb=8,
             stride=64 * 132, B=64, D=128)
    a.update(kw)
    return lib().pkv_gather_indexer_k_fp8(a["kv_cache"], a["k_fp8"], a["k_scale"],
                                          a["block_table"], a["cu"], a["R"], a["maxb"], a["T"],
                                          a["nb"], a["stride"], a["B"], a["D"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=100), PKV_EUNSUPPORTED, "multiple of 16"),
    (dict(stride=64 * 132 - 16), PKV_EUNSUPPORTED, "smaller than the page"),
    (dict(stride=64 * 132 + 8), PKV_EALIGN, "multiple of 16"),
    (dict(R=-1), PKV_EINVAL, "num_reqs"),
    (dict(T=-5), PKV_EINVAL, "num_tokens"),
    (dict(nb=0), PKV_EINVAL, "num_blocks"),
    (dict(B=0), PKV_EINVAL, "block_size"),
    (dict(maxb=-1), PKV_EINVAL, "max_blocks_per_req"),
    (dict(k_fp8=0), PKV_EINVAL, "null"),
    (dict(kv_cache=A + 4), PKV_EALIGN, "16-byte"),
    (dict(k_scale=A + 2), PKV_EALIGN, "4-byte"),
    (dict(R=70000, maxb=40000), PKV_EUNSUPPORTED, "2^31"),
    (dict(R=1, maxb=(1 << 22) + 1), PKV_EUNSUPPORTED, "max_blocks_per_req must be <="),
])
def test_gather_validation(kw, code, msg):
    assert gather(**kw) == code
    assert msg in last_error()


@pytest.mark.parametrize("kw", [dict(R=0), dict(T=0), dict(maxb=0),
                                dict(R=0, kv_cache=0, k_fp8=0, k_scale=0)])
def test_gather_empty_work_is_ok_without_launch(kw):
    assert gather(**kw) == PKV_OK
    assert last_error() == ""


def store8(**kw):
    a = dict(k=A, ks=128, dt=0, slots=A, T=10, cache=A, nb=4, stride=64 * 132, B=64, D=128)
    a.update(kw)
    return lib().pkv_store_indexer_k_fp8(a["k"], a["ks"], a["dt"], a["slots"], a["T"],
                                         a["cache"], a["nb"], a["stride"], a["B"], a["D"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=1040, ks=1040, stride=64 * 1044), PKV_EUNSUPPORTED),
    (dict(D=24), PKV_EUNSUPPORTED),
    (dict(ks=100), PKV_EINVAL),
    (dict(ks=132), PKV_EALIGN),
    (dict(k=A + 8), PKV_EALIGN),
    (dict(slots=A + 4), PKV_EALIGN),
    (dict(cache=0), PKV_EINVAL),
    (dict(T=-1), PKV_EINVAL),
    (dict(dt=2), PKV_EINVAL),
    (dict(dt=-1), PKV_EINVAL),
])
def test_store_fp8_validation(kw, code):
    assert store8(**kw) == code


def test_store_fp8_empty_is_ok():
    assert store8(T=0, k=0, slots=0, cache=0) == PKV_OK


def store4(**kw):
    a = dict(key=A, kst=1024, val=A, vst=1024, dt=0, kc=A, vc=A + 9216, slots=A, T=8, H=8,
             D=128, B=16, nb=4, page=18432, layout=0, kscale=A, vscale=A)
    a.update(kw)
    return lib().pkv_store_kv_fp4(a["key"], a["kst"], a["val"], a["vst"], a["dt"], a["kc"],
                                  a["vc"], a["slots"], a["T"], a["H"], a["D"], a["B"], a["nb"],
                                  a["page"], a["layout"], a["kscale"], a["vscale"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=40, kst=320, vst=320), PKV_EUNSUPPORTED, "not a multiple of 16"),
    (dict(D=96, kst=768, vst=768), PKV_EUNSUPPORTED, "multiple of 64"),
    (dict(B=6), PKV_EUNSUPPORTED, "not a multiple of 4"),
    (dict(layout=2), PKV_EINVAL, "layout"),
    (dict(kst=1000), PKV_EINVAL, "row strides"),
    (dict(kst=1028), PKV_EALIGN, "multiples of 8"),
    (dict(page=9000), PKV_EUNSUPPORTED, "smaller than one side"),
    (dict(page=9220), PKV_EALIGN, "page_stride"),
    (dict(kscale=0), PKV_EINVAL, "null"),
    (dict(vc=A + 4), PKV_EALIGN, "8-byte"),
    (dict(H=0), PKV_EINVAL, "num_heads"),
    (dict(dt=3), PKV_EINVAL, "src_dtype"),
])
def test_store_fp4_validation(kw, code, msg):
    assert store4(**kw) == code
    assert msg in last_error()


def test_store_fp4_empty_is_ok():
    assert store4(T=0, key=0, val=0, kc=0, vc=0, slots=0, kscale=0, vscale=0) == PKV_OK


def gdq(**kw):
    a = dict(kv_cache=A, out=A, ost=128, dt=0, block_table=A, cu=A, R=2, maxb=4, T=57, nb=8,
             stride=64 * 132, B=64, D=128)
    a.update(kw)
    return lib().pkv_gather_indexer_k_dequant(a["kv_cache"], a["out"], a["ost"], a["dt"],
                                              a["block_table"], a["cu"], a["R"], a["maxb"],
                                              a["T"], a["nb"], a["stride"], a["B"], a["D"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=100, ost=104), PKV_EUNSUPPORTED, "multiple of 16"),
    (dict(stride=64 * 132 + 8), PKV_EALIGN, "multiple of 16"),
    (dict(dt=2), PKV_EINVAL, "out_dtype"),
    (dict(ost=120), PKV_EINVAL, "out_row_stride"),
    (dict(ost=132), PKV_EALIGN, "multiple of 8"),
    (dict(out=0), PKV_EINVAL, "null"),
    (dict(out=A + 8), PKV_EALIGN, "16-byte"),
    (dict(R=-1), PKV_EINVAL, "num_reqs"),
    (dict(R=70000, maxb=40000), PKV_EUNSUPPORTED, "2^31"),
])
def test_gather_dequant_validation(kw, code, msg):
    assert gdq(**kw) == code
    assert msg in last_error()


def test_gather_dequant_empty_is_ok():
    assert gdq(R=0, kv_cache=0, out=0, block_table=0, cu=0) == PKV_OK
    assert gdq(T=0, kv_cache=0, out=0, block_table=0, cu=0) == PKV_OK


def g4(**kw):
    a = dict(kc=A, vc=A + 9216, ko=A, kst=1024, vo=A, vst=1024, dt=0, block_table=A, cu=A,
             R=2, maxb=4, T=57, H=8, D=128, B=16, nb=8, page=18432, layout=0, kscale=A,
             vscale=A)
    a.update(kw)
    return lib().pkv_gather_kv_fp4_dequant(a["kc"], a["vc"], a["ko"], a["kst"], a["vo"],
                                           a["vst"], a["dt"], a["block_table"], a["cu"], a["R"],
                                           a["maxb"], a["T"], a["H"], a["D"], a["B"], a["nb"],
                                           a["page"], a["layout"], a["kscale"], a["vscale"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=96, kst=768, vst=768), PKV_EUNSUPPORTED, "multiple of 64"),
    (dict(B=6), PKV_EUNSUPPORTED, "not a multiple of 4"),
    (dict(layout=2), PKV_EINVAL, "layout"),
    (dict(dt=5), PKV_EINVAL, "out_dtype"),
    (dict(kst=1000), PKV_EINVAL, "row strides"),
    (dict(vst=1028), PKV_EALIGN, "multiples of 8"),
    (dict(page=9000), PKV_EUNSUPPORTED, "smaller than one side"),
    (dict(page=18440), PKV_EALIGN, "page_stride"),
    (dict(vc=A + 8), PKV_EALIGN, "16-byte"),
    (dict(vscale=0), PKV_EINVAL, "null"),
    (dict(H=0), PKV_EINVAL, "num_heads"),
    (dict(maxb=-2), PKV_EINVAL, "max_blocks_per_req"),
])
def test_gather_fp4_dequant_validation(kw, code, msg):
    assert g4(**kw) == code
    assert msg in last_error()


def test_gather_fp4_dequant_empty_is_ok():
    assert g4(T=0, kc=0, vc=0, ko=0, vo=0, block_table=0, cu=0, kscale=0, vscale=0) == PKV_OK


def lg(**kw):
    a = dict(q=A, qst=8192, k=A, kscale=A, w=A, ks=A, ke=A, out=A, rst=1000, rcols=1000, M=8,
             H=64, N=100, D=128)
    a.update(kw)
    return lib().pkv_fp8_mqa_logits(a["q"], a["qst"], a["k"], a["kscale"], a["w"], a["ks"],
                                    a["ke"], a["out"], a["rst"], a["rcols"], a["M"], a["H"],
                                    a["N"], a["D"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=64, qst=4096), PKV_EUNSUPPORTED, "head_dim must be 128"),
    (dict(H=24), PKV_EUNSUPPORTED, "num_heads"),
    (dict(H=128, qst=16384), PKV_EUNSUPPORTED, "num_heads"),
    (dict(qst=8000), PKV_EINVAL, "q_token_stride"),
    (dict(qst=8200), PKV_EALIGN, "multiple of 16"),
    (dict(rst=999), PKV_EINVAL, "row_stride"),
    (dict(M=-1), PKV_EINVAL, "num_q"),
    (dict(k=0), PKV_EINVAL, "null"),
    (dict(q=A + 8), PKV_EALIGN, "16-byte"),
    (dict(out=A + 2), PKV_EALIGN, "4-byte"),
])
def test_mqa_logits_validation(kw, code, msg):
    assert lg(**kw) == code
    assert msg in last_error()


def test_mqa_logits_empty_is_ok():
    assert lg(M=0, q=0, k=0, kscale=0, w=0, ks=0, ke=0, out=0) == PKV_OK
    assert lg(N=0, q=0, k=0, kscale=0, w=0, ks=0, ke=0, out=0) == PKV_OK


def pa(**kw):
    a = dict(out=A, es=A, ml=A, tmp=A, q=A, kc=A, vc=A, bt=A, cl=A, S=4, H=64, KVH=8, D=128,
             B=16, maxb=8, maxc=128, nb=64, scale=0.088, ksc=0.03, vsc=0.04, P=256)
    a.update(kw)
    return lib().pkv_paged_attention_decode(a["out"], a["es"], a["ml"], a["tmp"], a["q"], a["kc"],
                                            a["vc"], a["bt"], a["cl"], a["S"], a["H"], a["KVH"],
                                            a["D"], a["B"], a["maxb"], a["maxc"], a["nb"],
                                            a["scale"], a["ksc"], a["vsc"], a["P"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(S=-1), PKV_EINVAL, "num_seqs"),
    (dict(KVH=0), PKV_EINVAL, "num_kv_heads"),
    (dict(H=60), PKV_EINVAL, "not a multiple"),
    (dict(H=136, KVH=8), PKV_EUNSUPPORTED, "at most 16"),
    (dict(D=64), PKV_EUNSUPPORTED, "head_size must be 128"),
    (dict(B=8), PKV_EUNSUPPORTED, "multiple of 16"),
    (dict(B=0), PKV_EUNSUPPORTED, "multiple of 16"),
    (dict(P=32), PKV_EUNSUPPORTED, "partition_size"),
    (dict(P=4096), PKV_EUNSUPPORTED, "partition_size"),
    (dict(P=384), PKV_EUNSUPPORTED, "partition_size"),
    (dict(maxc=(1 << 30) + 1), PKV_EUNSUPPORTED, "max_context_len"),
    (dict(S=1 << 25, H=128, KVH=8), PKV_EUNSUPPORTED, "below 2^31"),
    (dict(maxb=-1), PKV_EINVAL, "max_blocks_per_seq"),
    (dict(maxc=-1), PKV_EINVAL, "max_context_len"),
    (dict(nb=0), PKV_EINVAL, "num_blocks"),
    (dict(scale=float("inf")), PKV_EINVAL, "finite"),
    (dict(vsc=float("nan")), PKV_EINVAL, "finite"),
    (dict(tmp=0), PKV_EINVAL, "null"),
    (dict(out=0), PKV_EINVAL, "null"),
    (dict(kc=A + 8), PKV_EALIGN, "16-byte"),
    (dict(tmp=A + 4), PKV_EALIGN, "16-byte"),
    (dict(es=A + 2), PKV_EALIGN, "4-byte"),
    (dict(bt=A + 1), PKV_EALIGN, "4-byte"),
])
def test_paged_attention_validation(kw, code, msg):
    assert pa(**kw) == code
    assert msg in last_error()


def test_paged_attention_empty_is_ok():
    assert pa(S=0, out=0, es=0, ml=0, tmp=0, q=0, kc=0, vc=0, bt=0, cl=0) == PKV_OK


def pan(**kw):
    a = dict(out=A, q=A, kc=A, vc=A, bt=A, cl=A, S=4, H=64, KVH=8, D=128, B=16, maxb=8,
             maxc=128, nb=64, scale=0.088, ksc=0.03, vsc=0.04, P=256)
    a.update(kw)
    return lib().pkv_paged_attention_decode_noalloc(a["out"], a["q"], a["kc"], a["vc"], a["bt"],
                                                    a["cl"], a["S"], a["H"], a["KVH"], a["D"],
                                                    a["B"], a["maxb"], a["maxc"], a["nb"],
                                                    a["scale"], a["ksc"], a["vsc"], a["P"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(S=-1), PKV_EINVAL, "num_seqs"),
    (dict(H=60), PKV_EINVAL, "not a multiple"),
    (dict(P=384), PKV_EUNSUPPORTED, "partition_size"),
    (dict(out=0), PKV_EINVAL, "null"),
    (dict(kc=A + 8), PKV_EALIGN, "16-byte"),
    # 4096 x 64 heads x 64 partitions: 2 x 4 MiB + 2 GiB of workspace, over the 32 MiB
    (dict(S=4096, maxb=4096, maxc=65536, P=1024), PKV_EUNSUPPORTED, "built-in scratch"),
    # just over: n = 1009 * 64 gives 2 * align256(4 n) + 512 n = 33579520 > 2^25
    # (1008 sequences, 33546240 bytes, would fit)
    (dict(S=1009, H=64, KVH=8, maxc=256, P=256), PKV_EUNSUPPORTED, "built-in scratch"),
])
def test_paged_attention_noalloc_validation(kw, code, msg):
    """Every check runs on the host before any HIP call, so none of these
    reaches the device."""
    assert pan(**kw) == code
    assert msg in last_error()


def test_paged_attention_noalloc_empty_is_ok():
    assert pan(S=0, out=0, q=0, kc=0, vc=0, bt=0, cl=0) == PKV_OK


def test_diag_validation():
    assert lib().pkv_diag_encode_e4m3(A, A, 15, None) == PKV_EINVAL
    assert lib().pkv_diag_encode_e2m1(A + 4, A, 16, None) == PKV_EALIGN
    assert lib().pkv_diag_encode_e4m3(0, 0, 0, None) == PKV_OK


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):
        pkv.pkv_gather_indexer_k_fp8(x, x, x, x, x, block_size=64)


def test_last_error_is_per_thread():
    """pkv_last_error is the calling thread's own message: threads that fail
    differently (or succeed) at the same time each read back their own."""
    import threading
    cases = [(dict(D=100), PKV_EUNSUPPORTED, "multiple of 16"),
             (dict(R=-1), PKV_EINVAL, "num_reqs"),
             (dict(T=0), PKV_OK, "")]
    bad = []
    start = threading.Barrier(len(cases))

    def worker(kw, code, msg):
        start.wait()
        for _ in range(2000):
            rc = gather(**kw)
            err = last_error()
            if rc != code or (msg not in err if msg else err != ""):
                bad.append((kw, rc, err))
                return

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]


def test_plain_c_client_builds_and_links(tmp_path):
    """pkv.h compiles as strict C99 (gcc -pedantic -Werror) and a C program
    linked against libpkv.so gets the documented status codes and messages
    (host checks only: no GPU is touched)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "pkv_c_client"
    libdir = os.path.dirname(pkv.library_path())
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_client", "pkv_c_client.c"),
                        "-o", str(exe), os.path.join(libdir, "libpkv.so"),
                        "-Wl,-rpath," + libdir], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c client ok" in r.stdout, (r.returncode, r.stderr[-2000:])


def build_hip_client(tmp_path):
    """Builds tests/c_client/pkv_hip_client.cpp (host code only) with g++
    against the HIP runtime and libpkv.so; returns the executable's path."""
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("g++ or the HIP headers not available")
    exe = tmp_path / "pkv_hip_client"
    libdir = os.path.dirname(pkv.library_path())
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_client", "pkv_hip_client.cpp"),
                        "-o", str(exe), os.path.join(libdir, "libpkv.so"),
                        "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath," + libdir + ":/opt/rocm/lib"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_hip_client_builds(tmp_path):
    """The C++ client that drives libpkv with raw HIP buffers and its own
    stream compiles warning-free against pkv.h (it runs in the GPU tests)."""
    assert build_hip_client(tmp_path).exists()
