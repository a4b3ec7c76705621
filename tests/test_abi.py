"""libzpq's C ABI without a GPU: the library loads, exports every function
declared in include/zpq.h, and rejects invalid arguments on the host before
anything is launched (none of these calls reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

import block_quantized_communication_amd as zpq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zpq.h")

OK, NULL, SIZE, BLOCK, ALIGN, DTYPE, MODE, LAUNCH, ARG, ALIAS = range(10)
P = 1 << 20        # fake, 16-byte aligned "device" addresses: never dereferenced
NUL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:zpq_status|const char\*|int32_t)\s+(zpq_\w+)\s*\(", text, flags=re.M)


def vp(x):
    return ctypes.c_void_p(x)


def test_exports_match_header():
    names = declared_functions()
    assert sorted(names) == sorted(zpq.EXPORTS)
    L = zpq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert zpq.abi_version() == 1
    text = open(HEADER).read()
    assert "#define ZPQ_ABI_VERSION 1" in text
    for s in range(10):
        assert zpq.lib().zpq_status_str(s).decode() not in ("", "unknown status")
    assert zpq.lib().zpq_status_str(99).decode() == "unknown status"


def q8(x=P, dt=1, n=1024, block=256, codes=P + (1 << 16), scales=P + (1 << 18)):
    return zpq.lib().zpq_quant_i8(vp(x), dt, n, block, vp(codes), vp(scales), NUL)


def test_quant_i8_validation():
    assert q8(block=100) == BLOCK
    assert q8(block=16) == BLOCK
    assert q8(n=1000) == SIZE
    assert q8(n=-256) == SIZE
    assert q8(dt=3) == DTYPE
    assert q8(x=0) == NULL
    assert q8(scales=0) == NULL
    assert q8(x=P + 8) == ALIGN
    assert q8(codes=P + 4) == ALIGN
    assert q8(codes=P + 1024) == ALIAS          # codes inside x's 2 KB
    assert q8(scales=P + (1 << 16) + 512) == ALIAS
    assert q8(n=0, x=0, codes=0, scales=0) == OK   # empty: nothing to do
    assert q8(n=(1 << 40) + 256) == SIZE             # beyond the element limit


def dq8(codes=P, scales=P + (1 << 16), n=1024, block=256, y=P + (1 << 18), dt=1):
    return zpq.lib().zpq_dequant_i8(vp(codes), vp(scales), n, block, vp(y), dt, NUL)


def test_dequant_i8_validation():
    assert dq8(block=48) == BLOCK
    assert dq8(n=1280 + 1) == SIZE
    assert dq8(dt=7) == DTYPE
    assert dq8(y=0) == NULL
    assert dq8(scales=P + (1 << 16) + 4) == ALIGN
    assert dq8(y=P + 512) == ALIAS
    assert dq8(n=0, codes=0, scales=0, y=0) == OK
    assert dq8(n=(1 << 40) + 256) == SIZE


def qt8(x=P, dt=2, n=1024, codes=P + (1 << 16), scale=P + (1 << 18)):
    return zpq.lib().zpq_quant_i8_tensor(vp(x), dt, n, vp(codes), vp(scale), NUL)


def test_quant_i8_tensor_validation():
    assert qt8(n=1000) == SIZE
    assert qt8(n=-16) == SIZE
    assert qt8(n=(1 << 40) + 16) == SIZE
    assert qt8(dt=5) == DTYPE
    assert qt8(scale=0) == NULL
    assert qt8(x=0) == NULL
    assert qt8(codes=0) == NULL
    assert qt8(x=P + 4) == ALIGN
    assert qt8(scale=P + (1 << 18) + 4) == ALIGN
    assert qt8(codes=P + 256) == ALIAS           # codes inside x's 2 KB
    assert qt8(scale=P + (1 << 16) + 64) == ALIAS


def rq4(g=P, dt=2, n=8 * 4 * 128 * 3, L=8, N=4, block=128, codes=P + (1 << 18),
        scales=P + (1 << 19)):
    return zpq.lib().zpq_qgz_reorder_quant_i4(vp(g), dt, n, L, N, block, vp(codes), vp(scales),
                                              NUL)


def test_qgz_reorder_quant_validation():
    assert rq4(block=127) == BLOCK
    assert rq4(L=0) == ARG
    assert rq4(N=-1) == ARG
    assert rq4(n=8 * 4 * 128 * 3 + 128) == SIZE    # whole blocks but not whole slices
    assert rq4(dt=-1) == DTYPE
    assert rq4(g=0) == NULL
    assert rq4(codes=P + (1 << 18) + 8) == ALIGN
    assert rq4(codes=P + 4096) == ALIAS
    assert rq4(n=0, g=0, codes=0, scales=0) == OK
    assert rq4(n=(1 << 40) + 8 * 4 * 128) == SIZE


def dr4(ic=P, isc=P + (1 << 18), K=8, c=4096, block=128, oc=P + (1 << 19),
        os_=P + (1 << 19) + (1 << 16), ov=0, odt=0, div=1.0):
    return zpq.lib().zpq_qgz_dequant_reduce_requant_i4(vp(ic), vp(isc), K, c, block, vp(oc),
                                                       vp(os_), vp(ov), odt,
                                                       ctypes.c_float(div), NUL)


def test_dequant_reduce_validation():
    assert dr4(block=96) == BLOCK
    assert dr4(K=0) == ARG
    assert dr4(c=4096 + 64) == SIZE
    assert dr4(c=1 << 32) == SIZE                    # per-lane offsets are 32-bit
    # exactly one output mode
    assert dr4(ov=P + (1 << 20)) == MODE              # both
    assert dr4(oc=0, os_=0) == MODE                   # neither
    assert dr4(os_=0) == MODE                         # half of I4
    fl = dict(oc=0, os_=0, ov=P + (1 << 20))
    assert dr4(odt=3, **fl) == DTYPE
    assert dr4(div=0.0, **fl) == ARG
    assert dr4(div=-2.0, **fl) == ARG
    assert dr4(div=float("inf"), **fl) == ARG
    assert dr4(div=float("nan"), **fl) == ARG
    assert dr4(ic=0) == NULL
    assert dr4(isc=P + (1 << 18) + 4) == ALIGN
    assert dr4(oc=P + 512) == ALIAS                   # inside the received codes
    assert dr4(ov=P + (1 << 18), oc=0, os_=0) == ALIAS
    assert dr4(c=0, ic=0, isc=0) == OK


def test_binding_refuses_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1024, dtype=torch.float16)         # a CPU tensor
    with pytest.raises(ValueError):
        zpq.quant_i8(x, 256, out=(torch.zeros(1024, dtype=torch.int8),
                                  torch.zeros(4, dtype=torch.float32)))


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without the built HIP library every entry point raises."""
    monkeypatch.setattr(zpq, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libzpq.so"))
    monkeypatch.setattr(zpq, "_lib", None)
    with pytest.raises(ImportError):
        zpq.lib()
    with pytest.raises(ImportError):
        zpq.abi_version()


def test_bench_measures_one_gpu_only():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_modes_end_after_their_own_output():
    """Each alternative mode of bench.py (a study, --per-config, --patterns,
    ...) prints its one JSON line and returns: none falls through into the
    throughput benchmark, whose line would follow its own."""
    import ast
    with open(os.path.join(ROOT, "bench.py")) as f:
        tree = ast.parse(f.read())
    main = next(n for n in tree.body if isinstance(n, ast.FunctionDef) and n.name == "main")
    studies = set()
    for node in main.body:
        if not isinstance(node, ast.If) or node.orelse:
            continue
        test = ast.unparse(node.test)
        if not test.startswith("args."):
            continue
        m = re.fullmatch(r"args\.study == '([a-z-]+)'", test)
        if m:
            studies.add(m.group(1))
        if re.fullmatch(r"args\.(study == '[a-z-]+'|per_config|patterns|valu_rates)", test):
            assert isinstance(node.body[-1], ast.Return), test
    choices = next(k for k in ast.walk(tree) if isinstance(k, ast.keyword) and k.arg == "choices")
    assert studies == {c.value for c in choices.value.elts}


def test_binding_refuses_host_tensors():
    """The binding passes raw pointers: tensors not on a GPU are refused in
    Python, before the library sees them."""
    import torch
    x = torch.zeros(1024, dtype=torch.float16)
    with pytest.raises(ValueError):
        zpq.quant_i8(x, 256)
    with pytest.raises(ValueError):
        zpq.quant_i8_tensor(x)
    with pytest.raises(ValueError):
        zpq.qgz_reorder_quant_i4(x, 2, 2, 64)
    with pytest.raises(ValueError):
        zpq.dequant_i8(torch.zeros(1024, dtype=torch.int8), torch.zeros(4), 256)
    with pytest.raises(ValueError):
        zpq.qgz_dequant_reduce_requant_i4(torch.zeros(1024, dtype=torch.uint8),
                                           torch.zeros(16), 2, 1024, 128)


def test_receive_launch_names_the_shapes_libzpq_picks():
    """bench.py's receive-shapes study names the kernel each launch uses; on
    256 CUs the fused workload's 48-source average takes 8 elements per lane
    and 4 sources in flight (3-wave workgroups when built with them), the
    hop 1 of 8 x 2^25 takes 32 per lane and 2 in flight, and overrides
    apply."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    assert bench.receive_launch([], 48, 2752512, 64, 1, 256) == (
        8, 4, 256, "k_dequant_reduceILi64ELi8ELi1ELi4E")
    assert bench.receive_launch(["-DZPQ_REDUCE_WG3=1"], 48, 2752512, 64, 1, 256)[2] == 192
    assert bench.receive_launch(["-DZPQ_REDUCE_WG3=1"], 8, 1 << 25, 128, 0, 256)[2] == 256
    assert bench.receive_launch([], 8, 1 << 25, 128, 0, 256) == (
        32, 2, 256, "k_dequant_reduceILi128ELi32ELin1ELi2E")
    assert bench.receive_launch([], 16, 1 << 24, 128, 2, 256) == (
        16, 2, 256, "k_dequant_reduceILi128ELi16ELi2ELi2E")
    assert bench.receive_launch(["-DZPQ_REDUCE_NARROW_WAVES=0"], 48, 2752512, 64, 1, 256)[:2] == (16, 2)
    assert bench.receive_launch(["-DZPQ_REDUCE_EPL_I4=16", "-DZPQ_REDUCE_PF_I4=4"],
                                8, 1 << 25, 128, 0, 256)[:2] == (16, 4)


def test_variant_build_reads_the_compiler_resource_report():
    """build --variants keeps the compiler's register and occupancy report of
    every receive kernel (kernel-resource-usage remarks), and only those."""
    from block_quantized_communication_amd import build as hip_build
    text = "\n".join([
        "zpq.hip:938:1: remark: Function Name: _ZN12_GLOBAL__N_116k_dequant_reduceILi64ELi32ELin1ELi2EEEvPKhPKf [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:938:1: remark:     TotalSGPRs: 92 [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:938:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:938:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:938:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:938:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:938:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:436:1: remark: Function Name: _ZN12_GLOBAL__N_110k_quant_i8ILi1ELi256ELi8ELi2EEEvPKvlPaPfj [-Rpass-analysis=kernel-resource-usage]",
        "zpq.hip:436:1: remark:     VGPRs: 38 [-Rpass-analysis=kernel-resource-usage]",
    ])
    r = hip_build._resources(text)
    assert list(r) == ["_ZN12_GLOBAL__N_116k_dequant_reduceILi64ELi32ELin1ELi2EEEvPKhPKf"]
    assert r[next(iter(r))] == {"sgprs": 92, "vgprs": 64, "agprs": 0, "scratch_bytes_per_lane": 0,
                                "waves_per_simd": 8, "lds_bytes": 0}
    assert all(v for v in hip_build.RECEIVE_VARIANTS.values() if v) and \
        hip_build.RECEIVE_VARIANTS["default"] == []
    # the qgZ store-policy variants: their own kernels' report, names apart
    # from the receive variants, each overriding only the code-store policy
    assert list(hip_build._resources(text, "k_quant_i8")) == [
        "_ZN12_GLOBAL__N_110k_quant_i8ILi1ELi256ELi8ELi2EEEvPKvlPaPfj"]
    assert not set(hip_build.QGZ_STORE_VARIANTS) & set(hip_build.RECEIVE_VARIANTS)
    assert not set(hip_build.TIMELINE_VARIANTS) & (set(hip_build.RECEIVE_VARIANTS) |
                                                   set(hip_build.QGZ_STORE_VARIANTS))
    assert all("-DZPQ_TIMELINE=1" in v for v in hip_build.TIMELINE_VARIANTS.values())
    assert all(len(v) == 1 and v[0].startswith("-DZPQ_CPOL_QGZ=")
               for v in hip_build.QGZ_STORE_VARIANTS.values())
