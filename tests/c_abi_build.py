"""Build tests/c_abi_example (a plain C caller of libpa, with the CPU oracle linked in): test
infrastructure, compiled in-tree by __graft_entry__.build() and, if missing, by its test."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_example.c")
ORACLE_SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")
PKG = os.path.join(ROOT, "paged_kv_cache_82_amd")
EXE = os.path.join(HERE, "c_abi_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = EXE) -> str:
    cmd = [os.environ.get("CC", "gcc"), "-std=c11", "-O2", "-Wall", "-fopenmp",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), SRC, ORACLE_SRC, "-o", out + ".tmp",
           "-L", PKG, "-lpa", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../paged_kv_cache_82_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {out} failed:\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
