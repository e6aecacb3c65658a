"""The C ABI library (no GPU needed): it loads, exports every function include/fp8q.h
declares, and rejects invalid arguments on the host before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char)\s*\*?\s*(\w+)\s*\(", src, flags=re.M)


def test_header_declares_the_boundary():
    names = set(_declared())
    assert {"fp8_act_quant", "fp8_weight_quant", "fp8_weight_dequant", "fp8_block_gemm",
            "fp8_block_gemm_workspace_bytes", "fp8q_strerror", "fp8q_version"} <= names


def test_library_exports_every_declared_symbol():
    from fp8_act_quant_amd import _lib
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(_declared()) <= exported
    assert set(_lib.SIGNATURES) == set(_declared())


def test_binding_has_no_cpu_fallback():
    import fp8_act_quant_amd as fq
    src = open(os.path.join(ROOT, "fp8_act_quant_amd", "__init__.py")).read()
    assert "oracle" not in src
    assert fq.lib._name.endswith("libfp8q.so")


@pytest.fixture(scope="module")
def lib():
    from fp8_act_quant_amd import _lib
    return _lib.lib


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def test_strerror_and_version(lib):
    from fp8_act_quant_amd import _lib
    for code in range(0, 7):
        assert lib.fp8q_strerror(code)
    assert lib.fp8q_strerror(99) == b"unknown status"
    assert lib.fp8q_version() >> 16 == 1
    assert _lib.strerror(_lib.FP8Q_ERR_ALIGN).startswith("pointer alignment")


def test_act_quant_validation(lib):
    from fp8_act_quant_amd import _lib as L
    assert lib.fp8_act_quant(FAKE, FAKE, FAKE, 4, 100, None) == L.FP8Q_ERR_SHAPE
    assert lib.fp8_act_quant(FAKE, FAKE, FAKE, -1, 128, None) == L.FP8Q_ERR_SHAPE
    assert lib.fp8_act_quant(FAKE, FAKE, FAKE, 4, -128, None) == L.FP8Q_ERR_SHAPE
    assert lib.fp8_act_quant(None, FAKE, FAKE, 4, 128, None) == L.FP8Q_ERR_NULL
    assert lib.fp8_act_quant(FAKE, None, FAKE, 4, 128, None) == L.FP8Q_ERR_NULL
    assert lib.fp8_act_quant(FAKE, FAKE, None, 4, 128, None) == L.FP8Q_ERR_NULL
    assert lib.fp8_act_quant(FAKE + 8, FAKE, FAKE, 4, 128, None) == L.FP8Q_ERR_ALIGN
    assert lib.fp8_act_quant(FAKE, FAKE + 4, FAKE, 4, 128, None) == L.FP8Q_ERR_ALIGN
    assert lib.fp8_act_quant(FAKE, FAKE, FAKE + 2, 4, 128, None) == L.FP8Q_ERR_ALIGN
    # empty calls are valid no-ops, even with NULL pointers
    assert lib.fp8_act_quant(None, None, None, 0, 128, None) == L.FP8Q_OK
    assert lib.fp8_act_quant(None, None, None, 5, 0, None) == L.FP8Q_OK
    # sizes beyond the kernels' addressing are rejected
    assert lib.fp8_act_quant(FAKE, FAKE, FAKE, 1 << 40, 1 << 20, None) == L.FP8Q_ERR_SHAPE


def test_act_quant_kmajor_validation(lib):
    """The K-block-major variant validates like fp8_act_quant, and also rejects grids of
    2^29 or more scales (their byte offsets would not fit the GEMM's 32-bit addressing)."""
    from fp8_act_quant_amd import _lib as L
    f = lib.fp8_act_quant_kmajor
    assert f(FAKE, FAKE, FAKE, 4, 100, None) == L.FP8Q_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, -1, 128, None) == L.FP8Q_ERR_SHAPE
    assert f(None, FAKE, FAKE, 4, 128, None) == L.FP8Q_ERR_NULL
    assert f(FAKE, FAKE, None, 4, 128, None) == L.FP8Q_ERR_NULL
    assert f(FAKE, FAKE + 4, FAKE, 4, 128, None) == L.FP8Q_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE + 2, 4, 128, None) == L.FP8Q_ERR_ALIGN
    assert f(None, None, None, 0, 128, None) == L.FP8Q_OK
    assert f(FAKE, FAKE, FAKE, 1 << 23, 64 * 128, None) == L.FP8Q_ERR_SHAPE      # exactly 2^29 scales
    assert f(FAKE, FAKE, FAKE, 1 << 29, 128, None) == L.FP8Q_ERR_SHAPE


def test_weight_quant_and_dequant_validation(lib):
    from fp8_act_quant_amd import _lib as L
    for fn in (lib.fp8_weight_quant,):
        assert fn(FAKE, FAKE, FAKE, 4, 130, None) == L.FP8Q_ERR_SHAPE
        assert fn(None, FAKE, FAKE, 4, 128, None) == L.FP8Q_ERR_NULL
        assert fn(FAKE, FAKE + 1, FAKE, 4, 128, None) == L.FP8Q_ERR_ALIGN
        assert fn(None, None, None, 0, 256, None) == L.FP8Q_OK
        assert fn(FAKE, FAKE, FAKE, 128 * 65536, 128, None) == L.FP8Q_ERR_SHAPE
        # a grid dimension counts at most 2^32 - 1 work-items (one 256-thread workgroup per
        # 128-column block)
        assert fn(FAKE, FAKE, FAKE, 1, 1 << 31, None) == L.FP8Q_ERR_SHAPE
    assert lib.fp8_weight_dequant(FAKE, FAKE, FAKE, 4, 64, None) == L.FP8Q_ERR_SHAPE
    assert lib.fp8_weight_dequant(FAKE, None, FAKE, 4, 128, None) == L.FP8Q_ERR_NULL
    assert lib.fp8_weight_dequant(FAKE, FAKE, FAKE + 2, 4, 128, None) == L.FP8Q_ERR_ALIGN
    assert lib.fp8_weight_dequant(FAKE, FAKE + 1, FAKE, 4, 128, None) == L.FP8Q_ERR_ALIGN
    assert lib.fp8_weight_dequant(None, None, None, 3, 0, None) == L.FP8Q_OK


def test_block_gemm_validation(lib):
    from fp8_act_quant_amd import _lib as L
    g = lib.fp8_block_gemm
    ok = dict(aq=FAKE, sa=FAKE, wq=FAKE, sw=FAKE, y=FAKE, dt=L.FP8Q_OUT_BF16, M=4, N=4, K=128)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return g(a["aq"], a["sa"], a["wq"], a["sw"], a["y"], a["dt"], a["M"], a["N"], a["K"],
                 a.get("ws"), a.get("wsb", 0), None)

    assert call(dt=7) == L.FP8Q_ERR_DTYPE
    assert call(K=96) == L.FP8Q_ERR_SHAPE
    assert call(M=-2) == L.FP8Q_ERR_SHAPE
    assert call(N=-2) == L.FP8Q_ERR_SHAPE
    assert call(y=None) == L.FP8Q_ERR_NULL
    assert call(aq=None) == L.FP8Q_ERR_NULL
    assert call(sw=None) == L.FP8Q_ERR_NULL
    assert call(aq=FAKE + 8) == L.FP8Q_ERR_ALIGN
    assert call(y=FAKE + 4) == L.FP8Q_ERR_ALIGN
    assert call(sa=FAKE + 1) == L.FP8Q_ERR_ALIGN
    assert call(ws=FAKE + 8, wsb=4096) == L.FP8Q_ERR_ALIGN
    assert call(M=0, aq=None, sa=None, wq=None, sw=None, y=None) == L.FP8Q_OK
    assert call(N=0, aq=None, sa=None, wq=None, sw=None, y=None) == L.FP8Q_OK
    assert call(M=1 << 30, N=1 << 30) == L.FP8Q_ERR_SHAPE
    # K below 2^24: a 256-row tile's byte range (256 K) must be stated in 32 bits
    assert call(K=1 << 24) == L.FP8Q_ERR_SHAPE
    # row and column counts up to 2^36 (tile counts stay within 32-bit ints), even where
    # M * N and M * K are within the element limit
    assert call(M=(1 << 38) + 128, N=128, K=128) == L.FP8Q_ERR_SHAPE
    assert call(M=128, N=(1 << 36) + 1, K=128) == L.FP8Q_ERR_SHAPE
    assert lib.fp8_block_gemm_workspace_bytes(4, 4, 1 << 24, L.FP8Q_OUT_BF16) == 0
    assert lib.fp8_block_gemm_workspace_bytes(4096, 576, 7168, L.FP8Q_OUT_BF16) >= 0
    assert lib.fp8_block_gemm_workspace_bytes(4, 4, 100, L.FP8Q_OUT_BF16) == 0
    assert lib.fp8_block_gemm_workspace_bytes(4, 4, 128, 9) == 0
    # the K-block-major scale flag: its own size limit; unknown flag bits are rejected; the
    # workspace does not depend on the scale layout
    km = L.FP8Q_OUT_BF16 | L.FP8Q_SA_KMAJOR
    assert call(dt=km, M=1 << 23, K=64 * 128) == L.FP8Q_ERR_SHAPE
    assert call(dt=km | L.FP8Q_GEMM_EXACT_SLICES, M=1 << 23, K=64 * 128) == L.FP8Q_ERR_SHAPE
    assert call(dt=L.FP8Q_OUT_BF16 | 0x2000) == L.FP8Q_ERR_DTYPE
    assert call(dt=km, sa=FAKE + 2) == L.FP8Q_ERR_ALIGN
    assert call(dt=km, M=0, aq=None, sa=None, wq=None, sw=None, y=None) == L.FP8Q_OK
    for shape in ((4096, 576, 7168), (128, 7168, 7168), (4096, 1536, 7168)):
        assert (lib.fp8_block_gemm_workspace_bytes(*shape, km) ==
                lib.fp8_block_gemm_workspace_bytes(*shape, L.FP8Q_OUT_BF16))


def test_bf16_gemm_validation(lib):
    """fp8_bf16_gemm rejects bad arguments before touching the device (so this runs without
    one): output dtype, K not a multiple of 64 or at/above 2^23, negative sizes, null and
    misaligned pointers; an empty output is a no-op."""
    from fp8_act_quant_amd import _lib as L
    g = lib.fp8_bf16_gemm
    ok = dict(x=FAKE, w=FAKE, b=None, y=FAKE, dt=L.FP8Q_OUT_F32, M=4, N=4, K=64)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return g(a["x"], a["w"], a["b"], a["y"], a["dt"], a["M"], a["N"], a["K"], None)

    assert call(dt=7) == L.FP8Q_ERR_DTYPE
    assert call(K=96) == L.FP8Q_ERR_SHAPE
    assert call(K=1 << 23) == L.FP8Q_ERR_SHAPE
    assert call(M=(1 << 38) + 64, N=64, K=64) == L.FP8Q_ERR_SHAPE
    assert call(M=-1) == L.FP8Q_ERR_SHAPE
    assert call(N=-1) == L.FP8Q_ERR_SHAPE
    assert call(y=None) == L.FP8Q_ERR_NULL
    assert call(x=None) == L.FP8Q_ERR_NULL
    assert call(w=None) == L.FP8Q_ERR_NULL
    assert call(x=FAKE + 2) == L.FP8Q_ERR_ALIGN
    assert call(w=FAKE + 8) == L.FP8Q_ERR_ALIGN
    assert call(y=FAKE + 2) == L.FP8Q_ERR_ALIGN
    assert call(b=FAKE + 2) == L.FP8Q_ERR_ALIGN
    assert call(M=0, x=None, w=None, y=None) == L.FP8Q_OK
    assert call(N=0, x=None, w=None, y=None) == L.FP8Q_OK


def test_gemm_split_plans_of_the_workloads(lib):
    """The split-K plans the GEMM's planner makes for the large workloads, through the
    host-only workspace query: only the kv down-projection (96 tiles of 128x192 for 256 CUs)
    splits K, in 2 ranges (32 KiB of arrival words + 2 x 96 fp32 partial tiles of 128x192);
    fp32 output (exact slices) never splits. The no-allocation entry point refuses, before any
    launch, a shape whose plan needs more than its static scratch."""
    from fp8_act_quant_amd import _lib as L
    ws = lib.fp8_block_gemm_workspace_bytes
    assert ws(4096, 576, 7168, L.FP8Q_OUT_BF16) == 32768 + 2 * 96 * 128 * 192 * 4
    for shape in ((4096, 1536, 7168), (8192, 32768, 512), (16384, 7168, 7168), (64, 256, 256)):
        assert ws(*shape, L.FP8Q_OUT_BF16) == 0, shape
        assert ws(*shape, L.FP8Q_OUT_F32) == 0, shape
    assert ws(4096, 576, 7168, L.FP8Q_OUT_F32) == 0
    assert ws(4096, 576, 7168, L.FP8Q_OUT_BF16) <= L.FP8Q_NOALLOC_SCRATCH_BYTES
    M, N, K = 4096, 18432, 16384
    assert ws(M, N, K, L.FP8Q_OUT_BF16) > L.FP8Q_NOALLOC_SCRATCH_BYTES
    st = lib.fp8_block_gemm_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, L.FP8Q_OUT_BF16, M, N, K, None)
    assert st == L.FP8Q_ERR_WORKSPACE


def test_gemm_plans_of_the_workloads(lib):
    """fp8q_gemm_plan reports the planner's choice for a shape (host only), the same one
    fp8_block_gemm_workspace_bytes sizes: the configurations and split counts of the large
    workloads in their default modes; a forced configuration that the contraction mode does
    not implement leaves the default; bad arguments are rejected without writing the outputs."""
    from fp8_act_quant_amd import _lib as L
    names = []
    while (n := lib.fp8q_gemm_config_name(len(names))) is not None:
        names.append(n.decode())

    def plan(M, N, K, dt):
        c, s = ctypes.c_int(-7), ctypes.c_int(-7)
        assert lib.fp8q_gemm_plan(M, N, K, dt, ctypes.byref(c), ctypes.byref(s)) == L.FP8Q_OK
        return names[c.value], s.value

    bf16, f32 = L.FP8Q_OUT_BF16, L.FP8Q_OUT_F32
    assert plan(4096, 1536, 7168, bf16) == ("128x192w8", 1)
    assert plan(4096, 1536, 7168, bf16 | L.FP8Q_SA_KMAJOR) == ("128x192w8", 1)
    assert plan(4096, 576, 7168, bf16) == ("128x192w8", 2)
    assert plan(4096, 576, 7168, f32) == ("128x128", 1)
    assert plan(8192, 32768, 512, bf16) == ("256x256w8", 1)
    assert plan(16384, 7168, 7168, f32) == ("256x256w8", 1)
    assert plan(16384, 7168, 7168, f32 | L.FP8Q_GEMM_FP8_PRODUCTS) == ("256x256w8", 1)
    try:
        assert lib.fp8q_gemm_force_config(names.index("256x256w8"), 0) == L.FP8Q_OK
        assert plan(4096, 1536, 7168, bf16)[0] == "256x256w8"      # (split count: the planner's)
        assert plan(4096, 1536, 7168, f32) == ("256x256w8", 1)
        assert lib.fp8q_gemm_force_config(names.index("256x192w8"), 0) == L.FP8Q_OK
        assert plan(4096, 1536, 7168, f32) == ("128x128", 1)      # no exact-slice 256x192: the default
        assert lib.fp8q_gemm_force_config(names.index("256x256w8"), 1) == L.FP8Q_OK
        assert plan(4096, 1536, 7168, bf16) == ("256x256w8", 1)
    finally:
        lib.fp8q_gemm_force_config(-1, 0)
    c, s = ctypes.c_int(-7), ctypes.c_int(-7)
    for args, err in (((0, 8, 128, bf16), L.FP8Q_ERR_SHAPE), ((8, 8, 100, bf16), L.FP8Q_ERR_SHAPE),
                      ((8, 8, 128, 3), L.FP8Q_ERR_DTYPE)):
        assert lib.fp8q_gemm_plan(*args, ctypes.byref(c), ctypes.byref(s)) == err, args
    assert lib.fp8q_gemm_plan(8, 8, 128, bf16, None, ctypes.byref(s)) == L.FP8Q_ERR_NULL
    assert (c.value, s.value) == (-7, -7)


def test_python_binding_rejects_cpu_tensors_and_bad_shapes():
    import torch

    import fp8_act_quant_amd as fq
    with pytest.raises(ValueError):
        fq.act_quant(torch.zeros(4, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fq.weight_quant(torch.zeros(4, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fq.act_quant(torch.zeros(4, 128, dtype=torch.bfloat16), block_size=64)


def test_grouped_and_training_validation(lib):
    """The grouped GEMM and the backward entry points reject bad arguments on the host
    (no device is touched: every call below fails validation or is an empty no-op)."""
    from fp8_act_quant_amd import _lib as L
    g = lib.fp8_grouped_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 4, 8, 128, None) == L.FP8Q_ERR_SHAPE       # no experts
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1025, 4, 8, 128, None) == L.FP8Q_ERR_SHAPE    # too many
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 4, 8, 100, None) == L.FP8Q_ERR_SHAPE       # K % 128
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 2, 4, 8, 128, None) == L.FP8Q_ERR_NULL        # offsets
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, 0, 2, 4, 8, 128, None) == L.FP8Q_ERR_ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5, 2, 4, 8, 128, None) == L.FP8Q_ERR_DTYPE
    assert g(None, None, None, None, None, None, 0, 2, 0, 8, 128, None) == L.FP8Q_OK              # no rows
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 | L.FP8Q_SA_KMAJOR, 2, 4, 8, 128, None) == L.FP8Q_ERR_DTYPE
    t = lib.fp8_act_quant_t
    assert t(FAKE, FAKE, FAKE, 4, 12, None) == L.FP8Q_ERR_SHAPE                                    # C % 8
    assert t(FAKE, FAKE, FAKE, -1, 16, None) == L.FP8Q_ERR_SHAPE
    assert t(FAKE + 2, FAKE, FAKE, 4, 16, None) == L.FP8Q_ERR_ALIGN
    assert t(FAKE, FAKE, None, 4, 16, None) == L.FP8Q_ERR_NULL
    assert t(None, None, None, 0, 16, None) == L.FP8Q_OK
    wt = lib.fp8_weight_transpose
    assert wt(FAKE, FAKE, FAKE, FAKE, 16, 100, None) == L.FP8Q_ERR_SHAPE
    assert wt(FAKE, FAKE, FAKE + 8, FAKE, 16, 128, None) == L.FP8Q_ERR_ALIGN
    assert wt(FAKE, None, FAKE, FAKE, 16, 128, None) == L.FP8Q_ERR_NULL
    assert wt(FAKE, FAKE, FAKE, FAKE, 64, 1 << 30, None) == L.FP8Q_ERR_SHAPE                    # grid x
    assert t(FAKE, FAKE, FAKE, 1 << 31, 8, None) == L.FP8Q_ERR_SHAPE                             # grid x
    r = lib.fp8_rowwise_gemm
    assert r(FAKE, FAKE, FAKE, FAKE, FAKE, 9, 4, 4, 128, None, 0, None) == L.FP8Q_ERR_DTYPE
    assert r(FAKE, FAKE, FAKE, FAKE, FAKE, 1 | L.FP8Q_SA_KMAJOR, 4, 4, 128, None, 0, None) == L.FP8Q_ERR_DTYPE
    assert r(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 4, 100, None, 0, None) == L.FP8Q_ERR_SHAPE
    assert r(FAKE, FAKE, FAKE, FAKE, None, 0, 4, 4, 128, None, 0, None) == L.FP8Q_ERR_NULL
    assert r(FAKE, FAKE, FAKE + 8, FAKE, FAKE, 0, 4, 4, 128, None, 0, None) == L.FP8Q_ERR_ALIGN
    assert r(None, None, None, None, None, 0, 0, 4, 128, None, 0, None) == L.FP8Q_OK
    assert lib.fp8_rowwise_gemm_workspace_bytes(4, 4, 100, 0) == 0
    assert lib.fp8_rowwise_gemm_workspace_bytes(1, 1, 4096, 1) > 0      # a split-K plan for a tiny output


def test_python_training_binding_rejects_cpu_tensors():
    import torch
    import fp8_act_quant_amd as fq
    x = torch.zeros((4, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fq.act_quant_t(x)                                  # not a GPU tensor
    q = torch.zeros((4, 128), dtype=torch.float8_e4m3fn)
    s = torch.zeros((1, 1), dtype=torch.float32)
    with pytest.raises(ValueError):
        fq.weight_transpose(q, s)
    with pytest.raises(ValueError):
        fq.fp8_gemm_rowwise(q, s, q, s)
    with pytest.raises(ValueError):
        fq.fp8_grouped_gemm(q, s, q.view(1, 4, 128), s.view(1, 1, 1), torch.zeros(2, dtype=torch.int64))
