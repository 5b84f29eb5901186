"""Build the plain C client of the C ABI (tests/c_client/attn_client) with gcc,
linked against the in-tree libattn.so (found at run time through an
$ORIGIN-relative rpath, so the tree can move)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CLIENT = os.path.join(HERE, "attn_client")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "attn_client.c"), "-o", CLIENT + ".tmp",
           "-L/opt/rocm/lib", "-lamdhip64", "-L", os.path.join(ROOT, "attention_qk_online_amd"),
           "-lattn", "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath,$ORIGIN/../../attention_qk_online_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C client failed:\n{r.stdout}\n{r.stderr}")
    os.replace(CLIENT + ".tmp", CLIENT)
    return CLIENT


if __name__ == "__main__":
    print(build(verbose=True))
