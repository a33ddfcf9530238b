"""Text summary of a rocprofv3 hardware-counter run of ``bench.py`` over the
FLUX double block's kernels (matrix-core busy cycles, engine cycles, LDS).

    cd /tmp && export TMPDIR=/tmp
    timeout -s KILL 150 rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT \\
        SQ_WAIT_INST_LDS SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES --output-format csv -d $OUT/pmc_block -o p \\
        -- python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu --no-step --no-klein
    python -m diffusion_transformer_image_mm_amd.counters $OUT/pmc_block/p_counter_collection.csv

($REPO is the repository root, $OUT any output directory.) Counter values
are per dispatch, summed over the chip: engine cycles per XCD are
GRBM_GUI_ACTIVE / 8 (MI355X: 8 XCDs), matrix-core busy cycles per SIMD are
SQ_VALU_MFMA_BUSY_CYCLES / 1024 (256 CUs x 4 SIMDs). The algorithmic
matrix-core cycles of a kernel are its FLOPs at 1024 FLOP per clock per
SIMD (dense bf16/fp16 MFMA; fp8 runs twice as many per clock).
"""
from __future__ import annotations

import csv
import statistics as st
import sys
from collections import defaultdict

SIMDS, XCDS = 1024, 8
L, H, M = 4608, 3072, 12288
# the FLUX double block's kernels with fp16-encoded weights, and their FLOPs
KERNELS = [
    ("mmdit::attention_kernel<128>", "attention (24 heads x 4608 x 128)", 4 * L * L * H, 1024),
    ("mmdit::attention_fp8_kernel<128>", "fp8 attention (24 heads x 4608 x 128)", 4 * L * L * H, 2048),
    ("mmdit::gemm_kernel4<2, 64>", "QKV GEMM + QK-norm + RoPE", 2 * L * 3 * H * H, 1024),
    ("mmdit::gemm_kernel4<2, 2>", "out-projection and MLP-out GEMMs", None, 1024),
    ("mmdit::gemm_kernel4<2, 1>", "MLP-in GEMM + GELU", 2 * L * M * H, 1024),
    ("mmdit::gemm_kernel4<3, 1>", "fp8 MLP-in GEMM + GELU", 2 * L * M * H, 2048),
    ("mmdit::ln_modulate_kernel<3, 4, false>", "LN + modulate", None, 1024),
    ("mmdit::gemv_kernel<2, 6>", "modulation GEMV (both streams)", None, 1024),
]


def summarize(path: str) -> str:
    vals = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = [f"{'kernel':40s} {'dispatches':>10s} {'cycles/XCD':>11s} {'MFMA busy/SIMD':>15s} "
           f"{'algorithmic':>12s} {'busy share':>10s} {'LDS conflicts':>13s} {'LDS wait':>8s}"]
    for name, label, flops, per_clk in KERNELS:
        v = vals.get(name)
        if not v:
            continue
        med = {c: st.median(x) for c, x in v.items()}
        n = len(next(iter(v.values())))
        cyc = med.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / SIMDS
        alg = f"{flops / per_clk / SIMDS:12,.0f}" if flops else f"{'':>12s}"
        share = f"{100 * busy / cyc:9.1f}%" if cyc else ""
        wait = med.get("SQ_WAIT_INST_LDS", 0.0) / max(med.get("SQ_WAVE_CYCLES", 1.0), 1.0)
        out.append(f"{name:40s} {n:10d} {cyc:11,.0f} {busy:15,.0f} {alg} {share:>10s} "
                   f"{med.get('SQ_LDS_BANK_CONFLICT', 0.0):13,.0f} {100 * wait:7.1f}%   {label}")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    sys.stdout.write(summarize(sys.argv[1]))
