"""HBM traffic of the dominant kernel from rocprofv3 byte counters.

Two counter runs of ``bench.py --probe`` (which launches the MLP-in GEMM ten
times and then copies 1 GiB device-to-device three times):

    cd /tmp && export TMPDIR=/tmp
    timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o p -- python3 $REPO/bench.py --probe
    timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o p -- python3 $REPO/bench.py --probe

``python -m diffusion_transformer_image_mm_amd.traffic $OUT/pmc_fetch
$OUT/pmc_write`` then writes the summary that bench.py reads ($REPO is the
repository root, $OUT any output directory). Each counter (KiB per
dispatch) is scaled by expected/measured for the copy of known size, and the
result is tied to the SHA-256 of the kernel's sources
(k_gemm.hip and common.h): once they change, bench.py reports the traffic as
unknown (null).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the kernel's source and the header whose device helpers it inlines
KERNEL_SOURCES = [os.path.join(ROOT, "diffusion_transformer_image_mm_amd", "csrc", f) for f in ("k_gemm.hip", "common.h")]
SUMMARY = os.path.join(ROOT, "profiles", "gemm_mlp_in_flux_traffic.txt")
KERNEL_MATCH = "gemm_kernel4<2, 1>"          # fp16 weights, bias + GELU epilogue, four-wavefront kernel
COPY_MATCH = "__amd_rocclr_copyBuffer"
COPY_KIB = 1 << 20                            # the probe copies 1 GiB


def source_sha256() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _values(run_dir: str, match: str):
    path = glob.glob(os.path.join(run_dir, "*counter_collection.csv"))
    assert path, f"no counter csv under {run_dir}"
    return [float(r["Counter_Value"]) for r in csv.DictReader(open(path[0])) if match in r["Kernel_Name"]]


def summarize(fetch_dir: str, write_dir: str) -> str:
    gf, gw = _values(fetch_dir, KERNEL_MATCH), _values(write_dir, KERNEL_MATCH)
    cf, cw = _values(fetch_dir, COPY_MATCH), _values(write_dir, COPY_MATCH)
    f_fac = COPY_KIB / statistics.mean(cf)
    w_fac = COPY_KIB / statistics.mean(cw)
    fetch = statistics.mean(gf) * f_fac * 1024
    write = statistics.mean(gw) * w_fac * 1024
    lines = [
        "# HBM traffic of the MLP-in GEMM (gemm_kernel<F16, BIAS_GELU>, 4608x12288x3072, FLUX double block)",
        "# commands (from /tmp, TMPDIR=/tmp; $REPO = the repository root, $OUT = an output directory):",
        "#   timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o p"
        " -- python3 $REPO/bench.py --probe",
        "#   timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o p"
        " -- python3 $REPO/bench.py --probe",
        "#   python -m diffusion_transformer_image_mm_amd.traffic $OUT/pmc_fetch $OUT/pmc_write",
        f"# calibration: 1 GiB copy reads FETCH_SIZE {statistics.mean(cf):.0f} KiB -> factor {f_fac:.4f};"
        f" WRITE_SIZE {statistics.mean(cw):.0f} KiB -> factor {w_fac:.4f}",
        f"# gemm dispatches: {len(gf)} (FETCH_SIZE mean {statistics.mean(gf):.0f} KiB),"
        f" {len(gw)} (WRITE_SIZE mean {statistics.mean(gw):.0f} KiB)",
        f"kernel_source_sha256: {source_sha256()}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
    ]
    return "\n".join(lines) + "\n"


def load_traffic():
    """Traffic bytes per launch from the stored summary, or None when the
    summary is missing or was taken on a different kernel source."""
    try:
        kv = {}
        for line in open(SUMMARY):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != source_sha256():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


if __name__ == "__main__":
    text = summarize(sys.argv[1], sys.argv[2])
    os.makedirs(os.path.dirname(SUMMARY), exist_ok=True)
    with open(SUMMARY, "w") as f:
        f.write(text)
    sys.stdout.write(text)
