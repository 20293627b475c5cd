"""The GPU library's arithmetic contract, checked without a device: build
flags, kernel sources and the compiled gfx950 code (see contract.py), each
with planted mistakes in copies that the checks must catch (the pages'
source-level contract test with planted regressions, ADR-1444 "float_vif_hip
runs the arithmetic of the CUDA twin ...", Consequences)."""
import os
import shutil

import pytest

import contract
from contract import CSRC


@pytest.fixture(scope="module")
def flags():
    from vif_image_fidelity_amd import build
    return list(build.FLAGS)


@pytest.fixture(scope="module")
def isa(flags):
    inc = os.path.join(contract.ROOT, "include")
    return {n: contract.compile_isa(os.path.join(CSRC, n), flags, [inc])
            for n in contract.ISA_SOURCES}


def test_build_flags(flags):
    assert contract.flag_violations(flags) == []


def test_kernel_sources():
    assert contract.source_violations(contract.read_kernel_sources()) == []


def test_compiled_kernels(isa):
    names = []
    for n, asm in isa.items():
        assert contract.isa_violations(asm) == [], n
        names += list(contract.kernel_ops(asm))
    # every kernel of both features was seen
    assert any("scale_kernelILi8ELi4Eh" in k for k in names)
    assert any("scale_kernelILi1ELi0Ef" in k for k in names)
    assert any("decimate_pow2_kernel" in k for k in names)
    assert any("decimate_kernelI" in k for k in names)
    assert any("ssim_kernel" in k for k in names)
    assert any("scale_sums_kernel" in k for k in names)
    # every scale carries its row sums from tile to tile (no row-sum kernel)
    assert not any("4vifk13rowsum_kernel" in k for k in names)


# ----------------------------------------------------------- planted mistakes

@pytest.mark.parametrize("flag_edit", [
    ("-ffp-contract=off", "-ffp-contract=fast"),
    ("-fno-fast-math", "-ffast-math"),
    ("-fhip-fp32-correctly-rounded-divide-sqrt", "-O3"),
    ("-fno-gpu-flush-denormals-to-zero", "-fgpu-flush-denormals-to-zero"),
    ("-packed-fp32-ops", "+packed-fp32-ops"),
])
def test_flag_mutants_caught(flags, flag_edit):
    old, new = flag_edit
    mutated = [new if f == old else f for f in flags]
    assert mutated != flags
    assert contract.flag_violations(mutated)


SOURCE_MUTANTS = [
    ("vif_kernels.hip", "a[i] = k == 0 ? t * val : a[i] + t * val;",
     "a[i] = k == 0 ? t * val : __builtin_fmaf(t, val, a[i]);"),
    ("vif_device_math.h", "  return static_cast<float>(e) + q;",
     "  return log2f(x);"),
    ("vif_kernels.hip", "  const int x0 = tx * kTileW;",
     "  const int x0 = tx * kTileW;\n"
     "  atomicAdd(io.rows, 1.0f);"),
    ("vif_kernels.hip", "  float acc = 0.0f;\n  if (tx > 0)",
     "  float acc = 0.0f;\n  __hip_atomic_fetch_add(io.rows, 1.0f, "
     "__ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n  if (tx > 0)"),
    ("vif_noalloc.hip", "    carry[i] = 0ull;",
     "    __hip_atomic_exchange(carry + i, 0ull, __ATOMIC_RELAXED, "
     "__HIP_MEMORY_SCOPE_AGENT);"),
    ("fssim_kernels.hip", "#include <hip/hip_runtime.h>",
     "#include <hip/hip_runtime.h>\n#include <cuda_runtime.h>"),
    ("fssim_kernels.hip", "      s = s + wtap(sa, k) * v[i + k];",
     "      s = fmaf(wtap(sa, k), v[i + k], s);"),
    ("vif_device_math.h", "__device__ __forceinline__ float log2_poly",
     "#ifdef __HIP_PLATFORM_AMD__\n#endif\n"
     "__device__ __forceinline__ float log2_poly"),
    # the written-out fp64 division loses its remainder correction, or
    # gains a fused step, or a fused step moves outside it
    ("vif_device_math.h", "  return __builtin_fma(rem, r, q);",
     "  return q;"),
    ("vif_device_math.h", "  const double q = a * r;",
     "  const double q = __builtin_fma(a, r, 0.0);"),
    ("vif_device_math.h", "  const float q = p * t;",
     "  const float q = __builtin_fmaf(p, t, 0.0f);"),
    # the same for the written-out fp32 division
    ("vif_device_math.h", "  return __builtin_fmaf(rem, r, q);",
     "  return q;"),
    ("vif_device_math.h", "  float q = a * r;",
     "  float q = __builtin_fmaf(a, r, 0.0f);"),
    ("vif_device_math.h", "  const float gs = g * s12;",
     "  const float gs = __builtin_fmaf(g, s12, 0.0f);"),
]


@pytest.mark.parametrize("fname,old,new", SOURCE_MUTANTS)
def test_source_mutants_caught(fname, old, new):
    srcs = contract.read_kernel_sources()
    assert srcs[fname].count(old) == 1, (fname, old)
    srcs[fname] = srcs[fname].replace(old, new)
    assert contract.source_violations(srcs)


def test_isa_catches_contraction(flags, tmp_path):
    """The kernels built with -ffp-contract=fast: the compiler fuses the
    filter's multiplies and adds, and the machine-code check sees fused
    multiply-adds beyond the division expansions."""
    for n in os.listdir(CSRC):
        if n.endswith((".hip", ".h")):
            shutil.copy(os.path.join(CSRC, n), tmp_path / n)
    fast = [("-ffp-contract=fast" if f == "-ffp-contract=off" else f)
            for f in flags]
    asm = contract.compile_isa(str(tmp_path / "vif_kernels.hip"), fast,
                               [os.path.join(contract.ROOT, "include")])
    v = contract.isa_violations(asm)
    assert any("fp32 fused multiply-adds" in s for s in v), v


def test_isa_catches_planted_instructions():
    """Listings with a packed-fp32 add, a scalar store, an atomic and
    scratch memory in an otherwise clean kernel."""
    clean = ("_Zk:\n\tv_mul_f32_e32 v1, v2, v3\n\tv_add_f32_e32 v1, v1, v4\n"
             "\ts_endpgm\n")
    assert contract.isa_violations(clean) == []
    for line in ("\tv_pk_add_f32 v[0:1], v[2:3], v[4:5]\n",
                 "\ts_store_dword s1, s[2:3], 0x0\n",
                 "\tglobal_atomic_add_f32 v1, v2, s[0:1]\n",
                 "\tscratch_store_dword off, v1, off\n",
                 "\tv_fma_f32 v1, v2, v3, v4\n",
                 "\tv_rcp_f32_e32 v1, v2\n",
                 "\tv_log_f32_e32 v1, v2\n"):
        bad = clean.replace("\ts_endpgm", line + "\ts_endpgm")
        assert contract.isa_violations(bad), line
