"""CPU check of the kernel-trace summariser behind the committed block
profile: on a synthetic rocprofv3-style trace it must find the longest run of
back-to-back dominant-GEMM launches, time the last of them (after the 3
untimed ones), and take per-kernel medians over the blocks that share the
double block's 8-launch sequence."""
import csv
import re

from diffusion_transformer_image_mm_amd import kernel_trace as KT

BLOCK = ["void mmdit::gemv_kernel<2, 6>(float const*)", "void mmdit::ln_modulate_kernel<3, 4, false>(float const*)",
         "void mmdit::gemm_kernel4<2, 64>(mmdit::GemmArgs)", "void mmdit::attention_kernel<128>(unsigned short const*)",
         "void mmdit::gemm_kernel4<2, 2>(mmdit::GemmArgs)", "void mmdit::ln_modulate_kernel<3, 4, false>(float const*)",
         "void mmdit::gemm_kernel4<2, 1>(mmdit::GemmArgs)", "void mmdit::gemm_kernel4<2, 2>(mmdit::GemmArgs)"]


def _write(path, launches):
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X",
              "VGPR_Count", "LDS_Block_Size"]
    t = 1_000_000
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for name, us in launches:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + int(us * 1000),
                        "Grid_Size_X": 491520, "Workgroup_Size_X": 512, "VGPR_Count": 124, "LDS_Block_Size": 0})
            t += int(us * 1000) + 2000


def test_summary_of_synthetic_trace(tmp_path):
    launches = []
    for b in range(4):                       # 4 blocks: the kernel i of block b takes 10*(i+1) + b us
        launches += [(n, 10.0 * (i + 1) + b) for i, n in enumerate(BLOCK)]
    launches.append((BLOCK[0], 5.0))          # the next GEMV closes the fourth block
    launches.append(("void other_kernel()", 1.0))
    gemm = BLOCK[6]
    launches += [(gemm, 500.0)] * 3 + [(gemm, 300.0 + i) for i in range(20)]   # 3 untimed + 20 timed
    launches.append(("void other_kernel()", 1.0))
    launches += [(gemm, 1.0)] * 5            # a shorter run of the same kernel is not the timed one
    path = tmp_path / "t_kernel_trace.csv"
    _write(path, launches)
    text = KT.summarize(str(path))
    assert "back-to-back launches: 23 (3 untimed + 20 timed" in text
    mean = sum(300.0 + i for i in range(20)) / 20
    assert f"avg {mean:.1f} us" in text and "min 300.0" in text and "max 319.0" in text
    assert f"-> {KT.FLOPS / (mean * 1e-6) / 1e12:.1f} TFLOP/s" in text
    assert "median over 4 blocks" in text
    # medians over b = 0..3 of 10*(i+1) + b are 10*(i+1) + 1.5
    for i, n in enumerate(BLOCK):
        short = n.split("(")[0].replace("void ", "")
        assert re.search(re.escape(short) + r"\s+" + re.escape(f"{10.0 * (i + 1) + 1.5:.1f}"), text), short
    assert f"sum of medians {sum(10.0 * (i + 1) + 1.5 for i in range(8)):.1f} us" in text


def test_blocks_with_another_sequence_are_left_out(tmp_path):
    launches = []
    for b in range(3):
        seq = list(BLOCK)
        if b == 0:                            # a block whose 4th launch is another kernel
            seq[3] = "void mmdit::other_attention()"
        launches += [(n, 10.0) for n in seq]
    launches.append((BLOCK[0], 5.0))
    launches += [(BLOCK[6], 100.0)] * 4
    path = tmp_path / "t_kernel_trace.csv"
    _write(path, launches)
    text = KT.summarize(str(path))
    assert "median over 2 blocks" in text


def test_counter_summary_of_synthetic_run(tmp_path):
    """The hardware-counter summariser behind the committed counter profile:
    medians per kernel, engine cycles per XCD (/8), matrix-core busy cycles
    per SIMD (/1024) and the algorithmic cycles of the attention kernel."""
    from diffusion_transformer_image_mm_amd import counters as C
    path = tmp_path / "p_counter_collection.csv"
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    alg = 4 * 4608 * 4608 * 3072 / 1024          # attention FLOPs / (1024 FLOP/clk) over the chip's SIMDs
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for grbm in (8 * 500_000, 8 * 600_000, 8 * 550_000):
            name = "void mmdit::attention_kernel<128>(unsigned short const*)"
            w.writerow({"Kernel_Name": name, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": grbm})
            w.writerow({"Kernel_Name": name, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": alg})
            w.writerow({"Kernel_Name": name, "Counter_Name": "SQ_WAVE_CYCLES", "Counter_Value": 1000})
            w.writerow({"Kernel_Name": name, "Counter_Name": "SQ_WAIT_INST_LDS", "Counter_Value": 50})
    text = C.summarize(str(path))
    line = next(l for l in text.splitlines() if l.startswith("mmdit::attention_kernel<128>"))
    cells = line.split()
    assert cells[1] == "3"                                     # dispatches
    assert cells[2] == "550,000"                               # median GRBM / 8
    assert cells[3] == cells[4] == f"{alg / 1024:,.0f}"        # busy = algorithmic per SIMD
    assert cells[5] == f"{100 * (alg / 1024) / 550_000:.1f}%"
    assert cells[7] == "5.0%"
