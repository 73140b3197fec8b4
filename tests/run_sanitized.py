"""Host-side sanitizer run: builds the fp64 oracle and the library's host
code (argument validation and launch set-up: gdn_api.hip, gdn_static.hip)
with AddressSanitizer and UndefinedBehaviorSanitizer into a temporary
directory, links the latter with the ordinary device objects, and runs the
CPU test suite (-m "not gpu") against the two builds with the sanitizer
runtime preloaded.  No GPU is used; device code is never instrumented.

    python tests/run_sanitized.py        (after python -m hybrid_linear_attention_decode_amd.build)
"""
import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "hybrid_linear_attention_decode_amd")
CSRC = os.path.join(PKG, "csrc")
LLVM = "/opt/rocm/llvm"
HIPCC = "/opt/rocm/bin/hipcc"
HOST_ONLY = ["gdn_api.hip", "gdn_static.hip"]


def run(cmd, **kw):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, **kw)


def main() -> int:
    rt = sorted(glob.glob(f"{LLVM}/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        print("no clang ASan runtime found", file=sys.stderr)
        return 2
    objs = {os.path.basename(p)[:-2]: p for p in glob.glob(os.path.join(PKG, "_build", "*.o"))}
    device = [objs[n] for n in ("gdn_decode", "gdn_prefill", "gdn_slots", "kda_prefill")
              if n in objs]
    if len(device) != 4:
        print("build the library first (python -m hybrid_linear_attention_decode_amd.build)",
              file=sys.stderr)
        return 2
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer"]
    host_san = [f for x in san for f in ("-Xarch_host", x)]
    with tempfile.TemporaryDirectory() as tmp:
        orc = os.path.join(tmp, "libgdn_oracle.so")
        run([f"{LLVM}/bin/clang", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
             "-ffp-contract=off", *san, os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", orc,
             "-lm"])
        host = []
        for src in HOST_ONLY:
            o = os.path.join(tmp, src[:-4] + ".o")
            run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                 "-ffp-contract=off", *host_san, f"-I{os.path.join(ROOT, 'include')}",
                 f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", o])
            host.append(o)
        lib = os.path.join(tmp, "libgdn.so")
        run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, *host, *device,
             "-o", lib])
        env = dict(os.environ, LD_PRELOAD=rt[-1], GDN_LIB_PATH=lib, GDN_ORACLE_LIB_PATH=orc,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                            "-p", "no:cacheprovider", os.path.join(ROOT, "tests")],
                           env=env, cwd=ROOT)
        return r.returncode


if __name__ == "__main__":
    sys.exit(main())
