"""Builds libqmv.so (all HIP sources under csrc/) for gfx950 with hipcc.

    python -m quant_mat_vec_amd.build            # build
    python -m quant_mat_vec_amd.build --table    # build, print the kernel resource table

Objects go to quant_mat_vec_amd/_build/, the library next to this file.
Every compile also asks the compiler for its per-kernel resource report
(VGPRs, AGPRs, scratch, occupancy, LDS); the build writes it to
_build/kernel_resources.json, which the tests check.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmv.so")
RESOURCES = os.path.join(OBJ, "kernel_resources.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: no v_pk_*_f32 in any kernel.  amdgpu-mfma-vgpr-form:
# matrix-core results go straight to VGPRs (no accumulation-register copies).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wno-unused-command-line-argument",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
           "Occupancy [waves/SIMD]": "occupancy_waves_per_simd", "LDS Size [bytes/block]": "static_lds_bytes",
           "TotalSGPRs": "sgprs", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill"}


def parse_resources(text: str, source: str) -> list[dict]:
    """Kernels and their resources from the compiler's
    kernel-resource-usage remarks."""
    out, cur = [], None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"kernel": m.group(1), "source": os.path.basename(source)}
            out.append(cur)
            continue
        if cur is None:
            continue
        for key, name in _FIELDS.items():
            m = re.search(r"remark:\s+" + re.escape(key) + r": (\d+)", line)
            if m:
                cur[name] = int(m.group(1))
    return [k for k in out if k["kernel"].startswith("_ZN3qmv")]


def _compile(src: str):
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, parse_resources(r.stderr, src)


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source (always) and link libqmv.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        res = list(ex.map(_compile, srcs))
    objs = [o for o, _ in res]
    kernels = sorted((k for _, ks in res for k in ks), key=lambda k: (k["source"], k["kernel"]))
    with open(RESOURCES, "w") as f:
        json.dump(kernels, f, indent=1)
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


def demangled(names: list[str]) -> list[str]:
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
        return r.stdout.splitlines()
    except (OSError, subprocess.CalledProcessError):
        return names


def resource_table() -> str:
    """Markdown table of every kernel's resources from the last build."""
    with open(RESOURCES) as f:
        ks = json.load(f)
    names = demangled([k["kernel"] for k in ks])
    rows = ["| source | kernel | VGPRs | AGPRs | SGPRs | VGPR/SGPR spill | scratch B/lane | waves/SIMD | static LDS B |",
            "|---|---|---|---|---|---|---|---|---|"]
    for k, n in zip(ks, names):
        n = n.replace("qmv::", "").replace("(void const*, qmv::MmvqArgs, float*)", "")
        rows.append(f"| {k['source']} | `{n}` | {k.get('vgprs')} | {k.get('agprs')} | {k.get('sgprs')} | "
                    f"{k.get('vgpr_spill')}/{k.get('sgpr_spill')} | "
                    f"{k.get('scratch_bytes_per_lane')} | {k.get('occupancy_waves_per_simd')} | "
                    f"{k.get('static_lds_bytes')} |")
    return "\n".join(rows)


def resource_summary() -> str:
    """Markdown: per kernel template (by source file) the instantiation count
    and the range of each resource, then one row per instantiation (template
    arguments kept, parameter lists dropped)."""
    import collections
    import re
    with open(RESOURCES) as f:
        ks = json.load(f)
    names = [n.replace("qmv::", "").replace("(anonymous namespace)::", "").replace("void ", "")
             for n in demangled([k["kernel"] for k in ks])]
    short = [re.sub(r"\((?:[^()]|\([^()]*\))*\)$", "", n).strip() for n in names]
    fam = collections.defaultdict(list)
    for k, n in zip(ks, short):
        fam[(k["source"], re.split(r"[<(]", n)[0])].append(k)
    rows = ["| source | kernel template | instantiations | VGPRs | AGPRs max | spills max | scratch B/lane max | "
            "waves/SIMD min |", "|---|---|---|---|---|---|---|---|"]
    for (src, f), v in sorted(fam.items()):
        g = lambda key: [x.get(key) or 0 for x in v]  # noqa: E731
        rows.append(f"| {src} | `{f}` | {len(v)} | {min(g('vgprs'))}-{max(g('vgprs'))} | {max(g('agprs'))} | "
                    f"{max(g('vgpr_spill')) + max(g('sgpr_spill'))} | {max(g('scratch_bytes_per_lane'))} | "
                    f"{min(g('occupancy_waves_per_simd'))} |")
    rows += ["", "| source | kernel | VGPRs | AGPRs | SGPRs | spills V/S | scratch B/lane | waves/SIMD | LDS B |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k, n in sorted(zip(ks, short), key=lambda kn: (kn[0]["source"], kn[1])):
        rows.append(f"| {k['source']} | `{n}` | {k.get('vgprs')} | {k.get('agprs')} | {k.get('sgprs')} | "
                    f"{k.get('vgpr_spill')}/{k.get('sgpr_spill')} | {k.get('scratch_bytes_per_lane')} | "
                    f"{k.get('occupancy_waves_per_simd')} | {k.get('static_lds_bytes')} |")
    return "\n".join(rows)


if __name__ == "__main__":
    build()
    if "--table" in sys.argv[1:]:
        print(resource_table())
    if "--summary" in sys.argv[1:]:
        print(resource_summary())
