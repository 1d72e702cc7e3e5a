"""Build the checked host library: ``csrc/sq_host.cpp`` with its bounds
asserts on (``-DSQ_HOSTCHECK``) and AddressSanitizer + UndefinedBehavior-
Sanitizer on the host code only, linked with ``stubs.cpp`` in place of the
kernel launchers.  Device code is built as usual (the one device array of
the host file); nothing here launches a kernel."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "quantized_recurrent_state_decode_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# host-only sanitizers: each -fsanitize applies to the host pass alone
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host",
            "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-DSQ_HOSTCHECK", "-I", INCLUDE, "-I", CSRC,
         "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def asan_runtime() -> str | None:
    """The clang ASan runtime to preload into the process that loads the library."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in (os.path.join(CSRC, "sq_host.cpp"), os.path.join(HERE, "stubs.cpp")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC] + FLAGS + HOST_SAN + ["-x", "hip", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        objs.append(obj)
    lib = os.path.join(out_dir, "libstepq_hostcheck.so")
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libasan"] + HOST_SAN + \
          ["-o", lib] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(os.path.join(ROOT, "_build", "hostcheck")))
