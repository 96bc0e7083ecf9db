"""Build and run one probe: python -m exact_attention_15_amd.probes {stream,units,lds} [--build-only]"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "probes")
PROBES = ("stream", "units", "lds")


def build(name: str) -> str:
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, name)
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, name + ".hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise SystemExit(f"hipcc failed for {name}:\n{r.stderr}")
    return exe


def main(argv):
    if not argv or argv[0] not in PROBES:
        print(__doc__, file=sys.stderr)
        return 2
    exe = build(argv[0])
    if "--build-only" in argv:
        print(exe)
        return 0
    return subprocess.run([exe]).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
