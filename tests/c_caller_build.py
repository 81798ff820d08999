"""Builds tests/_build/c_caller from tests/c_caller.c with gcc: a plain C11
program linked against the in-tree libtreeverify.so and the HIP runtime,
found at run time through the binary's rpath. __graft_entry__.build() calls
this after building the library; the GPU test runs the binary."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(HERE, "c_caller.c")
BIN = os.path.join(HERE, "_build", "c_caller")
LIBDIR = os.path.join(ROOT, "tree_verify_attention_attn_amd")


def command(out=BIN):
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", out,
            "-L", LIBDIR, "-ltreeverify", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/../../tree_verify_attention_attn_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(force=False):
    if not force and os.path.exists(BIN) and os.path.getmtime(BIN) >= os.path.getmtime(SRC):
        return BIN
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    r = subprocess.run(command(), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {SRC}:\n{r.stdout}\n{r.stderr}")
    return BIN
