"""Source, flag and machine-code contract of the GPU library (CPU only).

The kernels reproduce the CPU definition bit for bit only if every fp32
multiply and add stays a separate IEEE rounding and every division is
correctly rounded.  The pages describe the same discipline for the HIP twin:
plain operators under -ffp-contract=off, correctly rounded division, and a
source-level contract test with planted regressions that runs without a
device (ADR-1444 "float_vif_hip runs the arithmetic of the CUDA twin ...",
Context and Consequences).  This module checks three layers:

  flags    the library's compiler flags fix contraction off, IEEE division,
           denormals and no fast-math, with packed fp32 disabled;
  sources  the kernel sources call no fused multiply-add (except those of
           the fp64 and fp32 divisions written out in div_in_range and
           div_in_range_f32, each checked to be exactly the division's
           sequence), no library or hardware log/exp, no atomic
           read-modify-write (an atomic add would merge sums in arrival
           order; atomic loads and stores that only hand a value from one
           block to the next are allowed), and include no CUDA or Triton;
  ISA      the compiled gfx950 code of every kernel: each fp32 fused
           multiply-add belongs to a correctly rounded division (one
           v_rcp_f32 each: five in the compiler's expansion, which ends in
           v_div_fixup_f32, six in the written-out one), each fp64 one to an
           fp64 division
           (one v_rcp_f64 each: five fused multiply-adds and a v_div_fmas in
           the compiler's expansion, which ends in v_div_fixup_f64, six in
           the written-out one), and there are no packed-fp32, float mad,
           hardware log/exp, atomic, scalar-memory-store or scratch
           instructions.

Each check returns a list of violation strings (empty when the contract
holds); the tests plant mistakes in copies to show each check fires.
"""
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vif_image_fidelity_amd", "csrc")

# Device code: every file whose functions run on the GPU.
KERNEL_SOURCES = ("vif_kernels.hip", "vif_device_math.h", "vif_selftest.hip",
                  "vif_noalloc.hip", "fssim_kernels.hip")
# Compiled for the ISA check (the others are included by these).
ISA_SOURCES = ("vif_kernels.hip", "vif_noalloc.hip", "fssim_kernels.hip")

REQUIRED_FLAGS = ("--offload-arch=gfx950", "-ffp-contract=off",
                  "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
                  "-fno-gpu-flush-denormals-to-zero")
FORBIDDEN_FLAGS = ("-ffast-math", "-ffp-contract=fast", "-ffp-contract=on",
                   "-funsafe-math-optimizations", "-ffinite-math-only",
                   "-fgpu-flush-denormals-to-zero", "-fno-honor-nans",
                   "-fno-honor-infinities", "-fapprox-func")


def flag_violations(flags):
    v = []
    for f in REQUIRED_FLAGS:
        if f not in flags:
            v.append("flag missing: %s" % f)
    for f in FORBIDDEN_FLAGS:
        if f in flags:
            v.append("forbidden flag: %s" % f)
    seq = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if not any(flags[i:i + 4] == seq for i in range(len(flags))):
        v.append("packed fp32 not disabled")
    return v


_SOURCE_RULES = (
    (r"\b(?:__builtin_)?fmaf?\s*\(|\b__fmaf?_r\w*\s*\(|\b__fmaf\s*\(",
     "explicit fused multiply-add"),
    (r"\b(?:log2f?|logf?|log10f?|__log2f|__logf|exp2f?|expf?|__expf|"
     r"__builtin_amdgcn_(?:log|exp)\w*|__builtin_(?:log|exp)\w*)\s*\(",
     "library or hardware log/exp in device code"),
    (r"\batomic(?!_load\b|_store\b)\w*\s*\(|"
     r"\b__hip_atomic_(?!load\b|store\b)\w*|\b__atomic_\w+",
     "atomic read-modify-write"),
    (r"#\s*include\s*[<\"](?:cuda|cublas|cub/|thrust/)", "CUDA include"),
    (r"\btriton\b", "Triton"),
    (r"__HIP_PLATFORM_|__CUDA_ARCH__|__NVCC__", "dual-platform code path"),
)


def _strip_comments(text):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.sub(r"//[^\n]*", "", text)


# The places the sources may fuse: the fp64 and fp32 divisions written out
# step by step, the same steps as the compiler's expansions.  fp64: a
# reciprocal, two Newton-Raphson refinements of two fused multiply-adds
# each, the product, the remainder and the corrected quotient.  fp32: a
# reciprocal, one refinement, the product, and two rounds of remainder and
# correction.
_DIV_HELPERS = (
    ("div_in_range", re.compile(
        r"double div_in_range\(double a, double d\) \{(?P<body>.*?)\n\}",
        re.S), [
        "double r = __builtin_amdgcn_rcp(d);",
        "double e = __builtin_fma(-d, r, 1.0);",
        "r = __builtin_fma(r, e, r);",
        "e = __builtin_fma(-d, r, 1.0);",
        "r = __builtin_fma(r, e, r);",
        "const double q = a * r;",
        "const double rem = __builtin_fma(-d, q, a);",
        "return __builtin_fma(rem, r, q);",
    ]),
    ("div_in_range_f32", re.compile(
        r"float div_in_range_f32\(float a, float d\) \{(?P<body>.*?)\n\}",
        re.S), [
        "float r = __builtin_amdgcn_rcpf(d);",
        "const float e = __builtin_fmaf(-d, r, 1.0f);",
        "r = __builtin_fmaf(e, r, r);",
        "float q = a * r;",
        "float rem = __builtin_fmaf(-d, q, a);",
        "q = __builtin_fmaf(rem, r, q);",
        "rem = __builtin_fmaf(-d, q, a);",
        "return __builtin_fmaf(rem, r, q);",
    ]),
)


def _take_div_helper(name, code, v):
    """Checks the written-out divisions, then removes their bodies from
    the code the other rules scan."""
    for helper, pattern, steps in _DIV_HELPERS:
        m = pattern.search(code)
        if m is None:
            continue
        body = [ln.strip() for ln in m.group("body").splitlines()
                if ln.strip()]
        if body != steps:
            v.append("%s: %s is not the division's steps" % (name, helper))
        code = code[:m.start("body")] + code[m.end("body"):]
    return code


def source_violations(sources):
    """sources: {file name: text} of device code."""
    v = []
    for name, text in sources.items():
        code = _take_div_helper(name, _strip_comments(text), v)
        for pat, what in _SOURCE_RULES:
            for m in re.finditer(pat, code):
                v.append("%s: %s (%s)" % (name, what, m.group(0).strip()))
    return v


def read_kernel_sources():
    return {n: open(os.path.join(CSRC, n)).read() for n in KERNEL_SOURCES}


def compile_isa(src_path, flags, include_dirs=()):
    """gfx950 assembly of one source file (device code only)."""
    out = src_path + ".contract.s"
    cmd = (["hipcc"] + [f for f in flags if f not in ("-fPIC", "-shared")] +
           ["--cuda-device-only", "-S", "-o", out, src_path])
    for d in include_dirs:
        cmd += ["-I", d]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed: %s" % r.stderr[-2000:])
    try:
        return open(out).read()
    finally:
        os.remove(out)


def kernel_ops(asm):
    """{kernel symbol: [mnemonic, ...]} of every kernel in an assembly
    listing (from its label to its s_endpgm), with the kernel's private
    segment (scratch) size."""
    out, cur, body = {}, None, []
    for ln in asm.splitlines():
        m = re.match(r"^(_Z\S+):(\s|$)", ln)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is None:
            continue
        m = re.match(r"^\s+([a-z_][a-z0-9_]*)", ln)
        if m:
            body.append(m.group(1))
            if m.group(1) == "s_endpgm":
                out[cur] = body
                cur = None
    return out


def scratch_sizes(asm):
    return {m.group(1): int(m.group(2)) for m in re.finditer(
        r"\.amdhsa_kernel (\S+).*?\.amdhsa_private_segment_fixed_size (\d+)",
        asm, re.S)}


_ISA_FORBIDDEN = (
    (r"v_pk_\w+", "packed fp32/fp16 instruction"),
    (r"v_(?:mad|mac)_(?:f16|f32|f64|legacy)\w*|v_fma_mix\w*|v_dot\w*",
     "float mad/dot instruction"),
    (r"v_(?:log|exp)_\w+", "hardware log/exp"),
    (r"\w*atomic\w*", "atomic instruction"),
    (r"s_(?:store|buffer_store|atomic|dcache_wb|scratch_store)\w*",
     "scalar memory store"),
    (r"scratch_\w+", "scratch memory access"),
)


def isa_violations(asm):
    v = []
    kernels = kernel_ops(asm)
    if not kernels:
        v.append("no kernel found in the assembly")
    for name, ops in kernels.items():
        def count(pat):
            return sum(1 for o in ops if re.fullmatch(pat, o))
        fma32 = count(r"v_fmac?_f32(?:_e32|_e64)?")
        fix32 = count(r"v_div_fixup_f32(?:_e64)?")
        rcp32 = count(r"v_rcp_f32(?:_e32|_e64)?")
        fma64 = count(r"v_fmac?_f64(?:_e32|_e64)?")
        fix64 = count(r"v_div_fixup_f64(?:_e64)?")
        rcp64 = count(r"v_rcp_f64(?:_e32|_e64)?")
        if fix32 > rcp32 or fma32 != 5 * fix32 + 6 * (rcp32 - fix32):
            v.append("%s: %d fp32 fused multiply-adds for %d divisions"
                     % (name, fma32, rcp32))
        if fix64 > rcp64 or fma64 != 5 * fix64 + 6 * (rcp64 - fix64):
            v.append("%s: %d fp64 fused multiply-adds for %d divisions"
                     % (name, fma64, rcp64))
        for pat, what in _ISA_FORBIDDEN:
            n = count(pat)
            if n:
                v.append("%s: %d x %s" % (name, n, what))
    for name, size in scratch_sizes(asm).items():
        if size:
            v.append("%s: %d bytes of scratch per lane" % (name, size))
    return v
