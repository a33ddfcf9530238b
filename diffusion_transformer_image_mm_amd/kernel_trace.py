"""Text summary of a rocprofv3 kernel trace of ``bench.py --no-step``.

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof -o bench \\
        -- python3 $REPO/bench.py --steps 20 --no-cpu --no-step
    python -m diffusion_transformer_image_mm_amd.kernel_trace $OUT/prof/bench_kernel_trace.csv

($REPO is the repository root, $OUT any output directory.)

Durations are End - Start per dispatch. bench.py runs the block with bf16
weights, then with fp16-encoded weights, then 3 untimed + K timed
back-to-back launches of the MLP-in GEMM; the longest run of consecutive
launches of that kernel is taken as the timed one. A double block is the
eight launches from one fp16-weight modulation GEMV to the next.
"""
from __future__ import annotations

import csv
import statistics as st
import sys
from collections import defaultdict

DOMINANT = "mmdit::gemm_kernel4<2, 1>"   # fp16 weights, bias + GELU epilogue, four-wavefront kernel
FLOPS = 2 * 4608 * 12288 * 3072
# the double block's launches in order (the QKV epilogue also does QK-norm +
# RoPE + the attention layouts)
BLOCK_LABELS = ["modulation GEMV (both streams)", "LN1 + modulate", "QKV GEMM + QK-norm + RoPE", "attention",
                "out-projection GEMM + gated residual", "LN2 + modulate", "MLP-in GEMM + GELU",
                "MLP-out GEMM + gated residual"]
KERNELS_PER_BLOCK = len(BLOCK_LABELS)


def summarize(path: str) -> str:
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        r["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        r["short"] = r["Kernel_Name"].split("(")[0].replace("void ", "")
    out = []
    best, cur = [], []
    for r in rows:
        if r["short"] == DOMINANT:
            cur.append(r)
        else:
            best, cur = (cur if len(cur) > len(best) else best), []
    best = cur if len(cur) > len(best) else best
    d = [r["dur"] for r in best]
    timed = d[3:] if len(d) > 3 else d
    out.append(f"dominant kernel: {DOMINANT} = MLP-in GEMM 4608x12288x3072, fp16-encoded weights, bias+GELU epilogue")
    out.append(f"  back-to-back launches: {len(d)} (3 untimed + {len(timed)} timed in bench.py)")
    out.append(f"  timed launches: avg {st.mean(timed):.1f} us  median {st.median(timed):.1f} us"
               f"  min {min(timed):.1f}  max {max(timed):.1f}")
    out.append(f"  grid {best[0]['Grid_Size_X']} work-items x {best[0]['Workgroup_Size_X']},"
               f" VGPR {best[0]['VGPR_Count']}, LDS {best[0]['LDS_Block_Size']}")
    out.append(f"  -> {FLOPS / (st.mean(timed) * 1e-6) / 1e12:.1f} TFLOP/s")
    # one block = the launches from one fp16-weight modulation GEMV to the next
    starts = [i for i, r in enumerate(rows) if "gemv_kernel<2" in r["short"]]
    blocks = [rows[a:b] for a, b in zip(starts, starts[1:]) if b - a == KERNELS_PER_BLOCK]
    if blocks:
        names = [r["short"] for r in blocks[-1]]
        blocks = [b for b in blocks if [r["short"] for r in b] == names]
        out.append("")
        out.append(f"one FLUX double-block forward, fp16-encoded weights (median over {len(blocks)} blocks, us):")
        tot = 0.0
        for i in range(KERNELS_PER_BLOCK):
            dd = st.median([b[i]["dur"] for b in blocks])
            tot += dd
            out.append(f"  {BLOCK_LABELS[i]:37s} {names[i]:40s} {dd:8.1f}")
        spans = [(int(b[-1]["End_Timestamp"]) - int(b[0]["Start_Timestamp"])) / 1e3 for b in blocks]
        out.append(f"  sum of medians {tot:.1f} us; median first-start -> last-end {st.median(spans):.1f} us")
    agg = defaultdict(list)
    for r in rows:
        agg[r["short"]].append(r["dur"])
    total = sum(sum(v) for v in agg.values())
    out.append("")
    out.append("all kernels of the run (share of kernel time):")
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:12]:
        out.append(f"  {k[:60]:60s} calls {len(v):5d} avg {st.mean(v):8.1f} us  {100 * sum(v) / total:5.1f}%")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    sys.stdout.write(summarize(sys.argv[1]))
