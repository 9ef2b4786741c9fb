"""Host-sanitized build of libsffn.so for the CPU checks (never used on a GPU).

The entry points' host code (argument checks, workspace carving, dispatch: csrc/api.hip) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only; device code is unchanged and the kernel
objects of the normal build are linked as they are. The result, _build/san/libsffn_san.so, is loaded in place of
libsffn.so through SFFN_LIB_PATH, with the ASan runtime preloaded (see ``sanitizer_env``)."""
import os
import subprocess

from activation_sparse_ffn_predictor_amd import build as _b

SAN = os.path.join(_b.BUILD, "san")
OUT = os.path.join(SAN, "libsffn_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    return subprocess.run(["hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def sanitizer_env(base=None) -> dict:
    env = dict(os.environ if base is None else base)
    env["SFFN_LIB_PATH"] = OUT
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def build() -> str:
    os.makedirs(SAN, exist_ok=True)
    objs = []
    for src in _b.SOURCES:
        if src == "api.hip":
            obj = os.path.join(SAN, "api.o")
            cmd = ["hipcc", *_b.HIPFLAGS, *HOST_SAN, "-O1", "-g", "-I", os.path.join(_b.HERE, "..", "include"),
                   "-c", os.path.join(_b.SRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"sanitized compile of {src} failed:\n{r.stdout}{r.stderr}")
        else:
            obj = os.path.join(_b.BUILD, src.replace(".hip", ".o"))
            if not os.path.exists(obj):
                obj = _b._compile(src)
        objs.append(obj)
    # the sanitizer runtime is preloaded at run time, so the link needs no sanitizer flags
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", OUT, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}{r.stderr}")
    return OUT


if __name__ == "__main__":
    print(build())
