"""Build libdca.so (HIP for gfx950 + the C ABI) in-tree with hipcc.

Every source under csrc/ is compiled to an object in parallel and linked into
dual_chunk_attention_amd/libdca.so.  Packed fp32 VALU ops are disabled on the device
(-packed-fp32-ops); hipcc's host pass warns that it does not know the feature, which is harmless.
The generated code of the sources in HAZARD_CHECKED is checked for the inline-asm MFMA hazards of
hazards.py; the build fails if one is found.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

try:
    from . import hazards
except ImportError:   # run as a script
    import hazards

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libdca.so")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
         "-Wno-unused-result", "-Wno-unused-command-line-argument"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# sources whose inline-asm MFMAs rely on hazards.asm_mfma_violations finding nothing
HAZARD_CHECKED = ["attn_fused.hip"]


def _compile(src, verbose):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = ["hipcc", "-c", "-x", "hip", src, "-o", obj] + FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        checks = [ex.submit(hazards.check_source, os.path.join(CSRC, f), FLAGS) for f in HAZARD_CHECKED]
        results = list(ex.map(lambda s: _compile(s, verbose), sources()))
        for f, c in zip(HAZARD_CHECKED, checks):
            n = c.result()   # raises on a violation
            if verbose:
                print(f"{f}: {n} inline-asm MFMA blocks free of VALU operand hazards", flush=True)
    for _, out in results:
        if out.strip() and verbose:
            print(out, flush=True)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
