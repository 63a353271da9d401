"""CPU emulation build of libgau's kernel sources (test infrastructure only).

The library's .hip sources are compiled for the host with a shim
hip/hip_runtime.h (tests/emu/shim) that maps the HIP built-ins the kernels use
onto the emulation runtime (tests/emu/emu.cpp).  Only the LDS declarations are
rewritten (the host compiler has no __shared__); every other line of the
kernels compiles as written.  Two products, under tests/emu/_build:

  emu_bounds      AddressSanitizer build, FAST mode: every lane runs to
                  completion in turn; with every operand in an exact-size heap
                  buffer, any global or LDS access outside its buffer aborts
                  with the source line.
  libgau_emu.so   the C ABI of include/gau.h over the emulation (FULL mode:
                  lanes as fibers, block barriers, wave-wide MFMA and shuffles
                  with the hardware operand layouts, LDS DMA landing at issue
                  or only at the wait that requires it).

Nothing in the library uses this; it is how the CPU test suite checks the
kernels' addressing and synchronisation.
"""

import concurrent.futures
import hashlib
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
# The sources and the build folder can be redirected (EMU_CSRC, EMU_OUT) to
# check a modified copy of the kernels before it is adopted.
CSRC = os.environ.get("EMU_CSRC", os.path.join(ROOT, "chunked_linear_attention_amd", "csrc"))
OUT = os.environ.get("EMU_OUT", os.path.join(HERE, "_build"))
CXX = "/opt/rocm/llvm/bin/clang++"
UNITS = ["proj_gemm", "chunk_attn", "chunk_scan", "chunk_scores", "chunk_state", "chunk_scores_state", "out_gemm",
         "rope", "decode", "backward", "rms_norm", "gau_api"]
BOUNDS = os.path.join(OUT, "emu_bounds")
LIB = os.path.join(OUT, "libgau_emu.so")


def available():
    return os.path.exists(CXX)


def _inputs():
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    files += [os.path.join(ROOT, "include", "gau.h"), os.path.join(HERE, "emu.cpp"),
              os.path.join(HERE, "bounds_main.cpp"), os.path.join(HERE, "shim", "hip", "hip_runtime.h"),
              os.path.abspath(__file__)]
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _generate(gen):
    """Copy the kernel sources, rewriting the LDS declarations (and dropping
    AMDGPU occupancy attributes) only."""
    csrc = os.path.join(gen, "pkg", "csrc")
    os.makedirs(csrc, exist_ok=True)
    os.makedirs(os.path.join(gen, "include"), exist_ok=True)
    shutil.copy(os.path.join(ROOT, "include", "gau.h"), os.path.join(gen, "include", "gau.h"))
    for f in sorted(os.listdir(CSRC)):
        if not (f.endswith(".hip") or f.endswith(".h")):
            continue
        with open(os.path.join(CSRC, f)) as fh:
            s = fh.read()
        s = re.sub(r"extern __shared__ __align__\(16\) char lds\[\];", "char* lds = ::emu::lds_base();", s)
        s = re.sub(r"__shared__\s+(\w+)\s+(\w+)\[(\w+)\];",
                   r"\1* \2 = (\1*)::emu::static_shared(__LINE__, sizeof(\1) * (\3));", s)
        # AMDGPU occupancy attributes have no meaning on the host
        s = re.sub(r"__attribute__\(\(amdgpu_[a-z_]+\([^)]*\)\)\)", "", s)
        # inline assembly has no host meaning: refuse rather than miscompile
        if re.search(r"\b(__)?asm(__)?\s*(volatile\s*|__volatile__\s*)?\(", s):
            raise RuntimeError(f"{f}: inline assembly the emulation build does not rewrite")
        if "__shared__" in s:
            raise RuntimeError(f"{f}: LDS declaration the emulation build does not rewrite")
        with open(os.path.join(csrc, f), "w") as fh:
            fh.write(s)
    return csrc


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


def build(force=False):
    """Build both products (skipped when the inputs are unchanged)."""
    stamp = os.path.join(OUT, "stamp")
    key = _inputs()
    if not force and os.path.exists(stamp) and open(stamp).read() == key and os.path.exists(BOUNDS) \
            and os.path.exists(LIB):
        return
    if os.path.exists(OUT):
        shutil.rmtree(OUT)
    gen = os.path.join(OUT, "gen")
    csrc = _generate(gen)
    shim = os.path.join(HERE, "shim")
    common = [CXX, "-std=c++17", "-Wno-psabi", "-g", "-I" + shim, "-I" + os.path.join(gen, "include")]
    asan = common + ["-O1", "-fsanitize=address", "-fno-omit-frame-pointer"]
    full = common + ["-O2", "-fPIC"]
    jobs = []
    for u in UNITS:
        src = os.path.join(csrc, u + ".hip")
        jobs.append(asan + ["-x", "c++", "-c", src, "-o", os.path.join(OUT, "asan_" + u + ".o")])
        jobs.append(full + ["-x", "c++", "-c", src, "-o", os.path.join(OUT, "full_" + u + ".o")])
    jobs.append(asan + ["-c", os.path.join(HERE, "emu.cpp"), "-o", os.path.join(OUT, "asan_emu.o")])
    jobs.append(full + ["-c", os.path.join(HERE, "emu.cpp"), "-o", os.path.join(OUT, "full_emu.o")])
    jobs.append(asan + ["-I" + csrc, "-c", os.path.join(HERE, "bounds_main.cpp"),
                        "-o", os.path.join(OUT, "asan_bounds_main.o")])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(_run, jobs))
    objs = lambda p: sorted(os.path.join(OUT, f) for f in os.listdir(OUT) if f.startswith(p) and f.endswith(".o"))
    _run([CXX, "-fsanitize=address"] + objs("asan_") + ["-o", BOUNDS])
    _run([CXX, "-shared"] + objs("full_") + ["-o", LIB])
    with open(stamp, "w") as f:
        f.write(key)


if __name__ == "__main__":
    build(force="--force" in sys.argv)
    print(BOUNDS)
    print(LIB)
