"""Build the library with its host code under AddressSanitizer and
UndefinedBehaviorSanitizer, linked with abi_hostsan_driver.cpp into
_build/hostsan/abi_hostsan.

Every sanitizer flag goes to the host pass only (-Xarch_host); the device
code is compiled as usual (the host objects register it) and is never
launched by the driver, which runs without a GPU.  Objects are rebuilt when
their source or a header is newer.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "dual_autoregressive_tts_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "hostsan")
BIN = os.path.join(OUT, "abi_hostsan")
DRIVER = os.path.join(HERE, "abi_hostsan_driver.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer", *SAN,
         "-I", os.path.join(ROOT, "include")]
DRIVER_FLAGS = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *SAN, "-D__HIP_PLATFORM_AMD__",
                "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr}")


def _stale(obj, deps):
    return not os.path.exists(obj) or any(os.path.getmtime(d) > os.path.getmtime(obj) for d in deps)


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    # objects built with other flags are stale too
    stamp = os.path.join(OUT, "flags")
    flags_text = repr((FLAGS, DRIVER_FLAGS))
    if not os.path.exists(stamp) or open(stamp).read() != flags_text:
        for o in glob.glob(os.path.join(OUT, "*.o")):
            os.remove(o)
        with open(stamp, "w") as f:
            f.write(flags_text)
    headers = glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "dualar.h")]
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        jobs.append((obj, [src] + headers, [HIPCC, *FLAGS, "-c", src, "-o", obj]))
    drv = os.path.join(OUT, "driver.o")
    jobs.append((drv, [DRIVER] + headers, [HIPCC, *DRIVER_FLAGS, "-x", "c++", "-c", DRIVER, "-o", drv]))
    todo = [cmd for obj, deps, cmd in jobs if _stale(obj, deps)]
    with ThreadPoolExecutor(max(1, min(8, len(todo)))) as ex:
        list(ex.map(_run, todo))
    objs = [obj for obj, _, _ in jobs]
    if todo or not os.path.exists(BIN):
        _run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-o", BIN])
    return BIN


if __name__ == "__main__":
    print(build())
