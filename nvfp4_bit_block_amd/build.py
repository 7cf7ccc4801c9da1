"""Build libnvfp4.so (HIP kernels for gfx950 + the C ABI) in-tree.

Each source is compiled with hipcc for gfx950 only; the shared object is
linked against the HIP runtime that PyTorch ships, so that one process holds
one HIP runtime whichever of the two is loaded first.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
ARCH = "gfx950"

SOURCES = ["api.cpp", "quantize.hip", "dequantize.hip", "gemm.hip"]

HIPCC_FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-rdc",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source additions: the quantizers' matrix-core rotation keeps its
# accumulators in ordinary VGPRs (read by the vector ALU right after), not
# in the accumulation registers, which would cost a copy per value.
EXTRA_FLAGS = {"quantize.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _torch_lib_dir():
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        return None
    d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(src, []) + ["-I", INCLUDE, "-I", CSRC, "-c",
                                                              os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def _device_asm(src, verbose):
    """gfx950 assembly of one source, kept in _build/ for the build checks."""
    out = os.path.join(BUILD, os.path.basename(src) + ".s")
    cmd = [_hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(src, []) + ["-I", INCLUDE, "-I", CSRC,
                                                              "--cuda-device-only", "-S", os.path.join(CSRC, src),
                                                              "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(6, len(SOURCES) + 3)) as ex:
        # device assembly of the kernel sources (build checks; register counts
        # for the profile summaries)
        asm = [ex.submit(_device_asm, f, verbose) for f in ("quantize.hip", "gemm.hip", "dequantize.hip")]
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        for a in asm:
            a.result()
    tdir = _torch_lib_dir()
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    link = ["g++", "-shared", "-o", LIB + ".tmp"] + objs
    if tdir:
        link += [f"-L{tdir}", "-l:libamdhip64.so", f"-Wl,-rpath,{tdir}"]
    else:
        link += [f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"]
    link += ["-Wl,--no-undefined", "-Wl,-z,defs"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_test_lib(name: str, verbose: bool = False) -> str:
    """tests/_build/lib<name>.so from tests/<name>.hip: device checks of the
    library's arithmetic (test infrastructure; built with the library's own
    flags and headers, so that they run the kernels' code paths)."""
    tests = os.path.join(os.path.dirname(HERE), "tests")
    out_dir = os.path.join(tests, "_build")
    os.makedirs(out_dir, exist_ok=True)
    so = os.path.join(out_dir, f"lib{name}.so")
    obj = os.path.join(out_dir, f"{name}.o")
    cmd = [_hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(tests, f"{name}.hip"),
                                     "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}.hip:\n{r.stdout}\n{r.stderr}")
    tdir = _torch_lib_dir()
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    link = ["g++", "-shared", "-o", so + ".tmp", obj]
    if tdir:
        link += [f"-L{tdir}", "-l:libamdhip64.so", f"-Wl,-rpath,{tdir}"]
    else:
        link += [f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"]
    subprocess.run(link, check=True)
    os.replace(so + ".tmp", so)
    return so


TEST_LIBS = ("divcheck", "convcheck")


def build_test_libs(verbose: bool = False):
    with ThreadPoolExecutor(max_workers=len(TEST_LIBS)) as ex:
        return list(ex.map(lambda n: build_test_lib(n, verbose), TEST_LIBS))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
