"""Builds tests/native/convrot_client (plain C99, gcc) against include/convrot.h, the in-tree
libconvrot.so and the HIP runtime's C API.  The binary finds both libraries through its
run path, so it runs from this folder on any machine with ROCm in /opt/rocm."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "rotation_w4a4_quantized_convrot_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCE = os.path.join(HERE, "convrot_client.c")
CLIENT = os.path.join(HERE, "convrot_client")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C ABI client")
    tmp = CLIENT + ".tmp"
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SOURCE,
           "-o", tmp, "-L", PKG, "-lconvrot", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../rotation_w4a4_quantized_convrot_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C ABI client failed:\n{r.stderr}")
    os.replace(tmp, CLIENT)
    if verbose:
        print(f"built {CLIENT}")
    return CLIENT


if __name__ == "__main__":
    build(verbose=True)
