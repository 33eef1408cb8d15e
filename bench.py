#!/usr/bin/env python3
"""Benchmark of the projection GEMM hot path on one MI355X.

A step is one pass of the whole dense projection path over one batch: the
forward, input-gradient and weight-gradient GEMMs of the 4096 -> 12288
projection at T = 16384 tokens (BF16 operands ~ N(0,1) / N(0,0.02), FP32
accumulation, BF16 outputs, deterministic plans), inputs resident in HBM.
``value`` is the step's TFLOP/s (3 x 2*T*N*K FLOP per step).

Also reported: each pass's microseconds, TFLOP/s and fraction of the BF16 MFMA
peak, warm (the timed steps) and under the cold-cache protocol (a 1 GiB fill
before every call, events around the call only, median of 15 groups of 20);
the skinny-N weight gradients (4096->64, 4096->128, 5120->48, 5120->64 at T =
1025, 4031, 16173, 16384, 65537, BF16 and FP32 out, planner plan and one and
two forced splits, cold-cache protocol) as GB/s of algorithmic HBM bytes
against the 8 TB/s peak; the roofline of the dominant kernel from HIP events
on the launch stream; and the FP64 oracle timed on the host cores on a
bounded sample.

Also timed (microseconds, eager and as a captured HIP graph): the 4096->1024
projection at T = 64, the FP32 router at T = 64 / 256 / 1024 (deterministic
and split-K modes), and the checkpointed FP32 step of 4096->1024 / 4096->512
at T = 16384, whole and per op.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz (dense)
PEAK_HBM_GBPS = 8000.0
T_BIG, N_BIG, K_BIG = 16384, 12288, 4096
SKINNY = [(4096, 64), (4096, 128), (5120, 48), (5120, 64)]
# token counts timed: all modes at 16384, the planner's plan also at 65537
SKINNY_T_ALL = [1025, 4031, 16173, 16384, 65537]
SKINNY_MODES = [(True, 0), (False, 1), (False, 2)]   # planner plan, one split, two splits
SKINNY_T = 16384
SKINNY_SOURCES = ["deterministic_bf16_projection_amd/csrc/skinny_wgrad.h",
                  "deterministic_bf16_projection_amd/csrc/skinny_direct.h",
                  "deterministic_bf16_projection_amd/csrc/skinny_lds.h",
                  "deterministic_bf16_projection_amd/csrc/gemm_kernel.h"]
KERNEL_SOURCES = ["deterministic_bf16_projection_amd/csrc/gemm_fast.h",
                  "deterministic_bf16_projection_amd/csrc/gemm_kernel.h",
                  "deterministic_bf16_projection_amd/csrc/device_common.h"]


def skinny_source_hash():
    return kernel_source_hash(SKINNY_SOURCES)


def kernel_source_hash(sources=None):
    """Hash of the kernel sources' code: comments and whitespace are left out,
    so that a comment edit does not mark the committed counters stale."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel_pass):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    PMC summary, if it was taken from the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, "gemm_%s_4096x12288_T16384_pmc.txt" % kernel_pass)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\S+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash():
        return None
    return float(b.group(1))


PROFILE_DIR = os.path.join(ROOT, "profiles")


def progress(msg):
    """A progress line on stderr (the JSON result line is the only stdout)."""
    print("bench: %s (%.0f s)" % (msg, time.time() - _T0), file=sys.stderr, flush=True)


_T0 = time.time()


def clock_under_load():
    """Engine clock (GHz) measured with rocm-smi under sustained load of the
    forward GEMM (committed summary), or None."""
    path = os.path.join(PROFILE_DIR, "gemm_fwd_4096x12288_T16384_clock_under_load.txt")
    if not os.path.exists(path):
        return None
    m = re.search(r"clock_ghz_under_load:\s*([0-9.]+)", open(path).read())
    return float(m.group(1)) if m else None


def read_mfma_busy(kernel_pass):
    """MFMA-busy fraction and engine clock of one pass's GEMM kernel from the
    committed rocprofv3 counter summary, if it was taken from the current
    kernel source; else None."""
    path = os.path.join(PROFILE_DIR, "gemm_4096x12288_T16384_mfma_busy.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\S+)", text)
    r = re.search(r"^%s: mfma_busy ([0-9.]+) clock_ghz ([0-9.]+)" % kernel_pass, text, re.M)
    # the clock comes from the forward kernel, the first of the counter run:
    # the later kernels' dispatch durations stretch under counter collection
    c = re.search(r"^fwd: mfma_busy [0-9.]+ clock_ghz ([0-9.]+)", text, re.M)
    if not m or not r or not c or m.group(1) != kernel_source_hash():
        return None
    return {"mfma_busy": float(r.group(1)), "clock_ghz": float(c.group(1)),
            "source": "rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE (profiles/); clock of the forward kernel"}


def read_step5_counters(N, op):
    """HBM bytes and MFMA busy of one checkpointed-step op (the first of its
    kind, 4096->N) from the committed rocprofv3 summary, if it was taken from
    the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, "checkpointed_step_T16384_f32_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\S+)", text)
    r = re.search(r"^4096->%d %s\s*: fetch ([0-9.e+]+) B, write ([0-9.e+]+) B \(([0-9.]+)x the algorithmic [^)]*\); "
                  r"mfma_busy ([0-9.]+)" % (N, op), text, re.M)
    if not m or not r or m.group(1) != kernel_source_hash():
        return None
    return {"hbm_bytes": float(r.group(1)) + float(r.group(2)), "x_algorithmic": float(r.group(3)),
            "mfma_busy": float(r.group(4)), "source": "rocprofv3 FETCH_SIZE / WRITE_SIZE / SQ_VALU_MFMA_BUSY_CYCLES "
            "(profiles/)"}


PASS_KERNEL_TAG = {  # template arguments (A K-major, B K-major) of each pass's GEMM kernel
    "fwd": "true, true", "dgrad": "true, false", "wgrad": "false, false"}
COPY_BYTES = 1 << 30


def calibration_kernels(torch, dev):
    """Kernels of known HBM bytes for scaling FETCH_SIZE / WRITE_SIZE: a 1 GiB
    device copy (reads and writes 1 GiB) and a sum over another 1 GiB buffer
    that no kernel has written since it was filled by a 2 GiB sweep (a pure
    read of 1 GiB)."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    other = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    sweep = torch.empty(2 * COPY_BYTES // 4, dtype=torch.float32, device=dev)
    sweep.fill_(0.0)  # evicts both buffers from L2 and the Infinity Cache
    dst = torch.empty_like(src)
    dst.copy_(src)
    total = other.sum()
    torch.cuda.synchronize()
    del src, other, sweep, dst, total


def profile_run():
    """One step of the three passes after the calibration kernels."""
    import numpy as np
    import torch
    import dpg_inputs
    import deterministic_bf16_projection_amd as dpg
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    calibration_kernels(torch, dev)
    x, w, dy = dpg_inputs.dense(T_BIG, N_BIG, K_BIG, seed_group=0)
    X, W, DY = to_dev(x), to_dev(w), to_dev(dy)
    Y = dpg.dpg_forward(X, W)
    DX = dpg.dpg_dgrad(DY, W)
    DW = dpg.dpg_wgrad(DY, X)
    torch.cuda.synchronize()
    print("profile run done", Y.shape, DX.shape, DW.shape)


def profile_skinny():
    """The skinny weight gradients once each (T=16384, FP32 out) under the
    planner's plan and with one and two forced splits, after the calibration
    kernels."""
    import numpy as np
    import torch
    import dpg_inputs
    import deterministic_bf16_projection_amd as dpg
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    calibration_kernels(torch, dev)
    for K, N in SKINNY:
        xs = to_dev(dpg_inputs.normal_bf16((SKINNY_T, K), 1.0, 0, 0))
        dys = to_dev(dpg_inputs.normal_bf16((SKINNY_T, N), 1.0, 0, 2))
        for det, split in SKINNY_MODES:
            out = dpg.dpg_wgrad(dys, xs, out_dtype=torch.float32, deterministic=det, split_k=split)
            torch.cuda.synchronize()
            print("skinny %d->%d det=%d split=%d done" % (K, N, det, split), tuple(out.shape), flush=True)


STEP5_N = (1024, 512)
STEP5_OPS = ("fwd", "fwd", "dgrad", "wgrad")


def profile_step5():
    """The checkpointed FP32-output step's four ops (forward twice, input and
    weight gradient; 4096->1024 and 4096->512 at T=16384, deterministic
    plans) once each after the calibration kernels."""
    import numpy as np
    import torch
    import dpg_inputs
    import deterministic_bf16_projection_amd as dpg
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    calibration_kernels(torch, dev)
    f32 = torch.float32
    for N in STEP5_N:
        x, w, dy = dpg_inputs.dense(T_BIG, N, K_BIG, seed_group=0)
        X, W, DY = to_dev(x), to_dev(w), to_dev(dy)
        for op in STEP5_OPS:
            if op == "fwd":
                dpg.dpg_forward(X, W, out_dtype=f32)
            elif op == "dgrad":
                dpg.dpg_dgrad(DY, W, out_dtype=f32)
            else:
                dpg.dpg_wgrad(DY, X, out_dtype=f32)
            torch.cuda.synchronize()
        print("step 4096->%d done" % N, flush=True)


def summarize_step5(fetch_csv, write_csv, busy_csv, command):
    """Writes profiles/checkpointed_step_T16384_f32_pmc.txt from three
    rocprofv3 --pmc runs of --profile-step5 (FETCH_SIZE; WRITE_SIZE;
    SQ_VALU_MFMA_BUSY_CYCLES + GRBM_GUI_ACTIVE): per op, its kernels (from the
    plan: the GEMM, plus the split reduction when the plan splits K), HBM bytes
    against the algorithmic ones, and the MFMA-busy fraction of its GEMM."""
    import csv
    import torch
    import deterministic_bf16_projection_amd as dpg

    def dispatches(path):
        d = {}
        for r in csv.DictReader(open(path)):
            e = d.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [d[k] for k in sorted(d)]

    fetch, write, busy = dispatches(fetch_csv), dispatches(write_csv), dispatches(busy_csv)
    f_scale, w_scale, cal = calibration_scales([(e["name"], e["FETCH_SIZE"]) for e in fetch],
                                               [(e["name"], e["WRITE_SIZE"]) for e in write])
    mine = lambda rows: [e for e in rows if "dpg::" in e["name"]]
    fetch, write, busy = mine(fetch), mine(write), mine(busy)
    pass_id = {"fwd": dpg.PASS_FORWARD, "dgrad": dpg.PASS_DGRAD, "wgrad": dpg.PASS_WGRAD}
    path = os.path.join(PROFILE_DIR, "checkpointed_step_T16384_f32_pmc.txt")
    i = 0
    with open(path, "w") as f:
        f.write("HBM traffic and MFMA busy of the checkpointed step's ops (4096->1024 and 4096->512, T=16384, FP32 "
                "out, deterministic plans), rocprofv3 PMC on MI355X\ncommands:\n  %s\n" % command.replace("\n", "\n  "))
        f.write("kernel_source_hash: %s\n" % kernel_source_hash())
        f.write(cal)
        f.write("mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 256 CUs x 4 SIMDs) of the GEMM kernel\n")
        for N in STEP5_N:
            for op in STEP5_OPS:
                plan = dpg.plan_describe(pass_id[op], T_BIG, N, K_BIG, torch.float32, True, 0)
                splits = int(re.search(r"splits=(\d+)", plan).group(1))
                n_k = 2 if splits > 1 else 1
                fb = sum(e["FETCH_SIZE"] for e in fetch[i:i + n_k]) * 1024.0 * f_scale
                wb = sum(e["WRITE_SIZE"] for e in write[i:i + n_k]) * 1024.0 * w_scale
                g = busy[i]
                mb = g["SQ_VALU_MFMA_BUSY_CYCLES"] / (g["GRBM_GUI_ACTIVE"] / 8.0 * 256 * 4)
                names = " + ".join(e["name"].replace("void dpg::", "").split("(")[0][:60] for e in fetch[i:i + n_k])
                i += n_k
                if op == "fwd":
                    alg = 2.0 * T_BIG * K_BIG + 2.0 * N * K_BIG + 4.0 * T_BIG * N
                elif op == "dgrad":
                    alg = 2.0 * T_BIG * N + 2.0 * N * K_BIG + 4.0 * T_BIG * K_BIG
                else:
                    alg = 2.0 * T_BIG * N + 2.0 * T_BIG * K_BIG + 4.0 * N * K_BIG
                f.write("4096->%d %-5s: fetch %.4g B, write %.4g B (%.2fx the algorithmic %.4g B); mfma_busy %.3f; "
                        "splits %d; kernels: %s\n" % (N, op, fb, wb, (fb + wb) / alg, alg, mb, splits, names))
    print("wrote", path)


def calibration_scales(fetch, write):
    """Scales that turn FETCH_SIZE / WRITE_SIZE (KB per dispatch) into bytes:
    the pure 1 GiB read (a sum) for the fetch counter, the 1 GiB copy for the
    write counter; fetch and write are lists of (kernel name, KB).  Also
    returns a line describing the calibration (the copy's fetch as a
    cross-check)."""
    def biggest(rows, pred):
        vals = [v for k, v in rows if pred(k.lower()) and "dpg" not in k]
        if not vals:
            raise SystemExit("no calibration kernel in the counter file")
        return max(vals)
    sum_f = biggest(fetch, lambda k: "reduce_kernel" in k)
    copy_f = biggest(fetch, lambda k: "copybuffer" in k)
    copy_w = biggest(write, lambda k: "copybuffer" in k)
    kb = COPY_BYTES / 1024.0
    f_scale, w_scale = kb / sum_f, kb / copy_w
    text = ("calibration: 1 GiB pure read (sum) FETCH_SIZE %.1f KB -> fetch x%.4f; 1 GiB copy WRITE_SIZE %.1f KB -> "
            "write x%.4f (the copy's FETCH_SIZE %.1f KB, i.e. x%.4f)\n" % (sum_f, f_scale, copy_w, w_scale, copy_f,
                                                                          kb / copy_f))
    return f_scale, w_scale, text


def summarize_skinny_pmc(fetch_csv, write_csv, command):
    """Writes profiles/skinny_wgrad_T16384_f32_pmc.txt from two rocprofv3 --pmc
    runs of --profile-skinny (FETCH_SIZE, WRITE_SIZE): HBM bytes of each skinny
    weight gradient (main kernel + split reduction) under the planner's plan
    and one and two forced splits, against its algorithmic bytes."""
    import csv

    def per_dispatch(path):
        d = {}
        for r in csv.DictReader(open(path)):
            e = d.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
            e[1] += float(r["Counter_Value"])
        return [tuple(d[k]) for k in sorted(d)]
    fetch, write = per_dispatch(fetch_csv), per_dispatch(write_csv)
    f_scale, w_scale, cal = calibration_scales(fetch, write)
    mine_f = [(k, v) for k, v in fetch if "dpg::" in k]
    mine_w = [(k, v) for k, v in write if "dpg::" in k]
    path = os.path.join(PROFILE_DIR, "skinny_wgrad_T16384_f32_pmc.txt")
    with open(path, "w") as f:
        f.write("HBM traffic of the skinny weight gradients (T=16384, FP32 out; planner plan, split_k=1, split_k=2), "
                "rocprofv3 PMC on MI355X\ncommands:\n  %s\n" % command.replace("\n", "\n  "))
        f.write("skinny_source_hash: %s\n" % skinny_source_hash())
        f.write(cal)
        i = 0
        for K, N in SKINNY:
            for det, split in SKINNY_MODES:
                tot_f = tot_w = 0.0
                names = []
                while i < len(mine_f):
                    k, v = mine_f[i]
                    if names and "reduce" not in k:
                        break
                    names.append(k.replace("void dpg::", "").split("(")[0])
                    tot_f += v * 1024.0 * f_scale
                    tot_w += mine_w[i][1] * 1024.0 * w_scale
                    i += 1
                    if "reduce" in k:
                        break
                alg = 2.0 * SKINNY_T * K + 2.0 * SKINNY_T * N + 4.0 * N * K
                f.write("%d->%d %s: fetch %.4g B, write %.4g B, total %.4g B; algorithmic %.4g B (ratio %.3f); "
                        "kernels: %s\n" % (K, N, "planner" if det else "split_k=%d" % split, tot_f, tot_w,
                                           tot_f + tot_w, alg, (tot_f + tot_w) / alg, " + ".join(names)))
    print("wrote", path)


def clock_load(seconds):
    """The forward GEMM of the benchmark shape in a loop for `seconds` (the
    engine clock is read meanwhile with rocm-smi)."""
    import torch
    import deterministic_bf16_projection_amd as dpg
    dev = torch.device("cuda:0")
    X = torch.randn(T_BIG, K_BIG, device=dev).bfloat16()
    W = (torch.randn(N_BIG, K_BIG, device=dev) * 0.02).bfloat16()
    Y = torch.empty(T_BIG, N_BIG, device=dev, dtype=torch.bfloat16)
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(20):
            dpg.dpg_forward(X, W, out=Y)
        torch.cuda.synchronize()
        n += 20
    us = (time.time() - t0) * 1e6 / n
    print("clock load: %d calls, %.1f us per call, %.1f TFLOP/s" % (n, us, 2.0 * T_BIG * N_BIG * K_BIG / us / 1e6))


def _read_counter_csv(path):
    import csv
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        out.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), r.get("Grid_Size")))
    return out


def summarize_pmc(fetch_csv, write_csv, command):
    """Writes profiles/gemm_<pass>_4096x12288_T16384_pmc.txt from two rocprofv3
    --pmc runs (FETCH_SIZE, WRITE_SIZE; kilobytes per dispatch)."""
    fetch = _read_counter_csv(fetch_csv)
    write = _read_counter_csv(write_csv)

    def pick(rows, pred):
        vals = [v for (k, c, v, g) in rows if pred(k)]
        return vals

    f_scale, w_scale, cal = calibration_scales([(k, v) for (k, c, v, g) in fetch], [(k, v) for (k, c, v, g) in write])
    for name, tag in PASS_KERNEL_TAG.items():
        pred = lambda k, tag=tag: "gemm_fast_kernel<256, 256" in k and (", %s," % tag) in k
        fk = pick(fetch, pred)
        wk = pick(write, pred)
        if not fk or not wk:
            continue
        fetch_b = fk[-1] * 1024.0 * f_scale
        write_b = wk[-1] * 1024.0 * w_scale
        alg = 2.0 * (T_BIG * K_BIG + N_BIG * K_BIG) if name == "fwd" else (
            2.0 * (T_BIG * N_BIG + N_BIG * K_BIG) if name == "dgrad" else 2.0 * (T_BIG * N_BIG + T_BIG * K_BIG))
        out_b = 2.0 * {"fwd": T_BIG * N_BIG, "dgrad": T_BIG * K_BIG, "wgrad": N_BIG * K_BIG}[name]
        path = os.path.join(PROFILE_DIR, "gemm_%s_4096x12288_T16384_pmc.txt" % name)
        with open(path, "w") as f:
            f.write("HBM traffic of the %s GEMM kernel (4096->12288, T=16384, BF16 out), rocprofv3 PMC on MI355X\n" % name)
            f.write("commands:\n  %s\n" % command.replace("\n", "\n  "))
            f.write("kernel_source_hash: %s\n" % kernel_source_hash())
            f.write(cal)
            f.write("FETCH_SIZE raw: %.1f KB   WRITE_SIZE raw: %.1f KB\n" % (fk[-1], wk[-1]))
            f.write("fetch_bytes_per_launch: %.4g\nwrite_bytes_per_launch: %.4g\n" % (fetch_b, write_b))
            f.write("hbm_bytes_per_launch: %.4g\n" % (fetch_b + write_b))
            f.write("algorithmic bytes (operands once + output): %.4g (ratio %.2f)\n"
                    % (alg + out_b, (fetch_b + write_b) / (alg + out_b)))
        print("wrote", path)


def summarize_counters(out_name, command, *csvs):
    """Writes profiles/<out_name> from rocprofv3 --pmc runs of --profile-run:
    every collected counter of each pass's 4096->12288 GEMM kernel (the last
    dispatch of it), and the average L2 read latency where
    TCP_TCC_READ_REQ_LATENCY and TCP_TCC_READ_REQ were collected."""
    import csv
    per = {}
    for path in csvs:
        disp = {}
        for r in csv.DictReader(open(path)):
            d = disp.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "dur_us": (int(r["End_Timestamp"]) -
                                                                                       int(r["Start_Timestamp"])) / 1e3})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for name, tag in PASS_KERNEL_TAG.items():
            ds = [d for d in disp.values() if "gemm_fast_kernel<256, 256" in d["name"] and (", %s, 0," % tag) in d["name"]]
            if ds:
                per.setdefault(name, {}).update({k: v for k, v in ds[-1].items() if k != "name"})
    path = os.path.join(PROFILE_DIR, out_name)
    with open(path, "w") as f:
        f.write("Memory-path counters of the 4096->12288 GEMM passes (T=16384, BF16 out), rocprofv3 PMC on MI355X\n")
        f.write("commands (one counter group per run):\n  %s\n" % command.replace("\n", "\n  "))
        f.write("kernel_source_hash: %s\n" % kernel_source_hash())
        for name, d in per.items():
            f.write("%s:" % name)
            for k in sorted(d):
                f.write(" %s=%.4g" % (k, d[k]))
            if d.get("TCP_TCC_READ_REQ_sum"):
                f.write("  avg_L2_read_latency_cycles=%.0f" % (d.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) /
                                                             d["TCP_TCC_READ_REQ_sum"]))
            if d.get("TCC_EA0_RDREQ_sum"):
                f.write("  dram_share_of_L2_misses=%.3f" % (d.get("TCC_EA0_RDREQ_DRAM_sum", 0.0) /
                                                          d["TCC_EA0_RDREQ_sum"]))
            f.write("\n")
    print("wrote", path)


def summarize_busy(counter_csv, command, xcds=8, cus=256):
    """Writes profiles/gemm_4096x12288_T16384_mfma_busy.txt from a rocprofv3
    --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE run: per pass, the engine
    clock (GRBM_GUI_ACTIVE counts every XCD, so cycles / XCDs / duration) and
    the fraction of SIMD cycles the MFMA pipes were busy
    (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x CUs x 4 SIMDs))."""
    import csv
    disp = {}
    for r in csv.DictReader(open(counter_csv)):
        d = disp.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "t0": int(r["Start_Timestamp"]),
                                               "t1": int(r["End_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    path = os.path.join(PROFILE_DIR, "gemm_4096x12288_T16384_mfma_busy.txt")
    with open(path, "w") as f:
        f.write("MFMA pipe utilisation of the 4096->12288 GEMM passes (T=16384, BF16 out), rocprofv3 PMC on MI355X\n")
        f.write("command:\n  %s\n" % command)
        f.write("kernel_source_hash: %s\n" % kernel_source_hash())
        f.write("clock = GRBM_GUI_ACTIVE / %d XCDs / duration; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                "(GRBM_GUI_ACTIVE / %d x %d CUs x 4 SIMDs)\n" % (xcds, xcds, cus))
        f.write("(under counter collection the second and third kernels' dispatch durations stretch beyond their "
                "busy cycles, so their clock figures are low; mfma_busy uses the busy cycles only)\n")
        for name, tag in PASS_KERNEL_TAG.items():
            ds = [d for d in disp.values() if "gemm_fast_kernel<256, 256" in d["name"] and (", %s, 0," % tag) in d["name"]]
            if not ds:
                continue
            d = ds[-1]
            dur_ns = d["t1"] - d["t0"]
            cyc = d["GRBM_GUI_ACTIVE"] / xcds
            busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * cus * 4)
            ghz = cyc / dur_ns
            flop = 2.0 * T_BIG * N_BIG * K_BIG
            f.write("%s: mfma_busy %.3f clock_ghz %.3f duration_us %.1f  (raw GRBM_GUI_ACTIVE %.4g, "
                    "SQ_VALU_MFMA_BUSY_CYCLES %.4g; %.0f TFLOP/s under the profiler = %.3f of the peak at that clock)\n"
                    % (name, busy, ghz, dur_ns / 1e3, d["GRBM_GUI_ACTIVE"], d["SQ_VALU_MFMA_BUSY_CYCLES"],
                       flop / dur_ns / 1e3, flop / dur_ns / 1e3 / (cus * 4096 * ghz / 1e3)))
    print("wrote", path)


def summarize_trace(stats_csv, command, bench_log=None, out_name="bench_4096x12288_T16384_kernel_trace.txt"):
    """Writes the kernel-trace summary (rocprofv3 --stats) under profiles/: all
    kernels, then each pass's mean over the timed steps (the last --steps
    dispatches of its BF16-output kernel) beside the HIP-event means that the
    traced run's own bench line reported (bench_log: that run's output)."""
    import csv
    m = re.search(r"--steps\s+(\d+)", command)
    steps = int(m.group(1)) if m else 10
    m = re.search(r"--warmup\s+(\d+)", command)
    warmup = int(m.group(1)) if m else 3
    events = {}
    if bench_log and os.path.exists(bench_log):
        lines = [l for l in open(bench_log) if l.startswith("{")]
        if lines:
            events = {k: v["us_mean"] for k, v in json.loads(lines[-1])["passes"].items()}
    rows = list(csv.DictReader(open(stats_csv)))
    path = os.path.join(PROFILE_DIR, out_name)
    with open(path, "w") as f:
        f.write("rocprofv3 kernel trace of bench.py on MI355X (gfx950)\n")
        f.write("command: %s\n" % command)
        f.write("kernel_source_hash: %s\n\n" % kernel_source_hash())
        f.write("%6s %10s %12s %8s  %s\n" % ("calls", "avg_us", "total_us", "pct", "kernel"))
        for r in rows:
            name = r["Name"].replace("void ", "").replace("(dpg::GemmParams)", "").replace("dpg::", "")
            f.write("%6s %10.1f %12.1f %8.2f  %s\n" % (r["Calls"], float(r["AverageNs"]) / 1e3,
                                                      float(r["TotalDurationNs"]) / 1e3, float(r["Percentage"]),
                                                      name[:150]))
        trace_csv = os.path.join(os.path.dirname(stats_csv), os.path.basename(stats_csv).replace(
            "kernel_stats", "kernel_trace"))
        if os.path.exists(trace_csv):
            per = {}
            for r in csv.DictReader(open(trace_csv)):
                for name, tag in PASS_KERNEL_TAG.items():
                    if "gemm_fast_kernel<256, 256" in r["Kernel_Name"] and (", %s, 0," % tag) in r["Kernel_Name"]:
                        per.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            f.write("\nper pass over the %d timed steps (dispatches %d..%d of its BF16-output kernel: after the %d "
                    "warmups, before the cold-cache runs), against the HIP-event mean of the same run's bench line:\n"
                    % (steps, warmup + 1, warmup + steps, warmup))
            for name, v in per.items():
                last = v[warmup:warmup + steps]
                f.write("  %-5s %10.1f us (trace)  %10s us (events)\n"
                        % (name, sum(last) / len(last), events.get(name, "n/a")))
        f.write("\ngemm_fast_kernel<256, 256, 2, 4, A K-major, B K-major, OUT>: forward = <true, true>, "
                "input gradient = <true, false>, weight gradient = <false, false>; 1.649e12 FLOP per launch.\n"
                "skinny_wgrad_kernel (N > 64, or forced small split counts), skinny_direct_kernel (N <= 64) and "
                "splitk_reduce_kernel: the skinny-N weight gradients (T=16384 and 65537).\n")
    print("wrote", path)


def cpu_baseline(target_s=20.0):
    """The FP64 oracle as it stands, on a bounded sample of the same workload:
    the forward pass's first R rows of Y[16384, 12288] (all columns)."""
    import numpy as np
    import dpg_inputs
    import oracle
    # the first rows of the seeded X[16384, 4096] draw (numpy fills row-major)
    max_rows = 4096
    x = dpg_inputs.normal_bf16((max_rows, K_BIG), 1.0, 0, 0)
    w = dpg_inputs.normal_bf16((N_BIG, K_BIG), dpg_inputs.SIGMA_W, 0, 1)
    oracle.forward(x[:1], w)
    # calibrate on 64 rows (enough to keep every host thread busy)
    t0 = time.perf_counter()
    oracle.forward(x[:64], w)
    dt = time.perf_counter() - t0
    rows = int(max(64, min(max_rows, target_s / max(dt / 64, 1e-6))))
    t0 = time.perf_counter()
    oracle.forward(x[:rows], w)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * N_BIG * K_BIG
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "forward 4096->12288: %d of 16384 rows of Y (%d x 12288 outputs, K=4096), FP64, %.1f s"
                      % (rows, rows, dt)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_small():
    """The FP64 oracle timed on the small workloads it finishes in seconds,
    wall-clock milliseconds per pass with all host threads and with one: the
    4096->1024 projection at T = 64 (BF16 operands) and the FP32 router
    (E = 256, H = 4096) at T = 64 / 256 / 1024 (exact FP64 products)."""
    import dpg_inputs
    import oracle
    n_all = oracle.num_threads()
    jobs = []
    x, w, dy = dpg_inputs.dense(64, 1024, 4096, seed_group=0)
    jobs.append(("projection_4096x1024_T64", x, w, dy))
    for T in (64, 256, 1024):
        rx, rw, rdy = dpg_inputs.router(T, 256, 4096, seed_group=0)
        jobs.append(("router_E256_H4096_T%d" % T, rx, rw, rdy))
    out = {"cpu_model": cpu_model(), "threads_all": n_all, "unit": "ms per pass"}
    for threads in (n_all, 1):
        oracle.set_num_threads(threads)
        key = "threads_%d" % threads
        for name, a, b, g in jobs:
            res = {}
            for pname, fn in (("fwd", lambda: oracle.forward(a, b)), ("dgrad", lambda: oracle.dgrad(g, b)),
                              ("wgrad", lambda: oracle.wgrad(g, a))):
                t0 = time.perf_counter()
                fn()
                res[pname] = round((time.perf_counter() - t0) * 1e3, 1)
            out.setdefault(name, {})[key] = res
    oracle.set_num_threads(n_all)
    return out


class ColdTimer:
    """The pages' cold-cache protocol: before every timed call a 1 GiB device
    buffer is zeroed (more than twice the 32 MB of L2 plus the 256 MB Infinity
    Cache), HIP events on the launch stream bracket the call only; after
    warm-ups, `groups` groups of `iters` calls; the result is the median of the
    per-group medians (microseconds).

    flush="read" flushes by reading the 1 GiB buffer instead (a sum): the
    caches then hold clean lines, whereas after the fill up to ~290 MB of dirty
    lines (L2 + Infinity Cache) are written back to HBM while the timed call
    runs, which a short HBM-bound call pays for in full.

    With spans=True the protocol runs again under torch's profiler
    (span_groups groups of iters calls, no events), and `last_span` holds the
    median of group medians of the call's kernel span: first kernel start to
    last kernel end of the library's kernels between two flushes, from the
    device timestamps (the pages time the span of an op's launches).  The
    events also hold the dispatch of the call (2-5 us); the span does not.
    None where the call runs no library kernel."""

    def __init__(self, torch, groups=15, iters=20, warmup=5, spans=True, span_groups=5):
        self.torch = torch
        self.groups, self.iters, self.warmup = groups, iters, warmup
        self.spans, self.span_groups = spans, span_groups
        self.last_span = None
        self.junk = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
        self.junk.zero_()
        n = groups * iters
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def _kernel_spans(self, prof):
        """Span of each call: the library's kernels (names in namespace dpg)
        that run between two flushes."""
        cuda = self.torch.autograd.DeviceType.CUDA
        ks = sorted((e.time_range.start, e.time_range.end, "dpg::" in e.name) for e in prof.events()
                    if e.device_type == cuda)
        spans, cur = [], None
        for s, t, mine in ks:
            if mine:
                cur = [s, t] if cur is None else [cur[0], max(cur[1], t)]
            elif cur is not None:
                spans.append(cur[1] - cur[0])
                cur = None
        if cur is not None:
            spans.append(cur[1] - cur[0])
        return spans

    def _flush(self, flush):
        if flush == "zero":
            self.junk.zero_()
        else:
            self.sink = self.junk.sum()

    def __call__(self, fn, flush="zero"):
        import numpy as np
        torch = self.torch
        stream = torch.cuda.current_stream()
        for _ in range(self.warmup):
            self._flush(flush)
            fn()
        torch.cuda.synchronize()
        medians = []
        for g in range(self.groups):
            evs = self.ev[g * self.iters:(g + 1) * self.iters]
            for e0, e1 in evs:
                self._flush(flush)
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            medians.append(float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])))
        self.last_span = None
        if self.spans:
            # a separate run under the profiler (its callbacks would shift the
            # event times above), span_groups groups of iters calls
            try:
                from torch.profiler import profile, ProfilerActivity
                with profile(activities=[ProfilerActivity.CUDA]) as prof:
                    for _ in range(self.span_groups * self.iters):
                        self._flush(flush)
                        fn()
                    torch.cuda.synchronize()
                spans = self._kernel_spans(prof)
            except Exception as e:  # the profiler is optional: keep the event times
                progress("kernel spans unavailable (%s: %s); event times only" % (type(e).__name__, e))
                self.spans = False
                spans = []
            if len(spans) == self.span_groups * self.iters:
                sm = [float(np.median(spans[g * self.iters:(g + 1) * self.iters])) for g in range(self.span_groups)]
                self.last_span = (float(np.median(sm)), min(sm), max(sm))
        return float(np.median(medians)), min(medians), max(medians)

    def close(self):
        del self.junk


def hbm_read_reference(torch, cold):
    """A plain read of 128 MiB (torch's sum over a BF16 tensor, the X of the
    4096-wide skinny weight gradients at T = 16384) under both flushes, and a
    warm back-to-back rate: the HBM read rate a streaming kernel can expect
    under each protocol."""
    t = torch.ones((16384, 4096), dtype=torch.bfloat16, device="cuda:0")
    nbytes = t.numel() * 2
    out = {}
    for flush in ("zero", "read"):
        us, _, _ = cold(lambda: t.sum(), flush=flush)
        out["cold_%s_flush" % flush] = {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1)}
    for _ in range(3):
        t.sum()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        t.sum()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 20
    out["warm"] = {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1)}
    del t
    return out


def cold_cache_passes(passes, cold):
    """Each big pass under the cold-cache protocol (ColdTimer)."""
    flop = 2.0 * T_BIG * N_BIG * K_BIG
    out = {}
    for name, fn in passes:
        us, lo, hi = cold(fn)
        out[name] = {"us_median": round(us, 1), "group_median_range_us": [round(lo, 1), round(hi, 1)],
                     "tflops": round(flop / us / 1e6, 1), "frac_peak": round(flop / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
        if cold.last_span:
            out[name]["us_span_median"] = round(cold.last_span[0], 1)
    return out


def config3_more(dpg, torch, X, W, DY, Y, DX, DW, passes):
    """More of the 4096->12288 workload (event means over 5 calls after 2
    warmups): the three passes at the ragged T = 16231 (row views of the same
    operands), an A/A control (the forward timed again after the plan cache
    is cleared and the plan rebuilt), the input gradient with FP32 output at
    T = 16384, and the step (three passes) as one captured HIP graph against
    its eager time (medians of three alternating rounds)."""
    stream = torch.cuda.current_stream()

    def timed(fn, reps=5):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def entry(us, T):
        flop = 2.0 * T * N_BIG * K_BIG
        return {"us": round(us, 1), "tflops": round(flop / us / 1e6, 1),
                "frac_peak": round(flop / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
    out = {}
    Tr = 16231
    xr, dyr, yr, dxr = X[:Tr], DY[:Tr], Y[:Tr], DX[:Tr]
    out["T16231_bf16"] = {
        "fwd": entry(timed(lambda: dpg.dpg_forward(xr, W, out=yr)), Tr),
        "dgrad": entry(timed(lambda: dpg.dpg_dgrad(dyr, W, out=dxr)), Tr),
        "wgrad": entry(timed(lambda: dpg.dpg_wgrad(dyr, xr, out=DW)), Tr)}
    # A/A control: the forward again from a plan built anew after clearing the
    # plan cache (a second, independently planned instance of the same call)
    first = timed(lambda: dpg.dpg_forward(X, W, out=Y))
    dpg.clear_plan_cache()
    second = timed(lambda: dpg.dpg_forward(X, W, out=Y))
    out["aa_control_fwd_us"] = {"cached_plan": round(first, 1), "replanned": round(second, 1)}
    dxf = torch.empty((T_BIG, K_BIG), dtype=torch.float32, device=X.device)
    out["T16384_dgrad_f32_out"] = entry(timed(lambda: dpg.dpg_dgrad(DY, W, out=dxf)), T_BIG)
    del dxf
    # the step captured once, replayed; eager time of the same three calls
    eager = timed(lambda: [fn() for _, fn in passes])
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _, fn in passes:
            fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, fn in passes:
            fn()
    import numpy as np
    eg, gr = [eager], [timed(g.replay)]
    for _ in range(2):  # alternate, so clock drift does not favour either mode
        eg.append(timed(lambda: [fn() for _, fn in passes]))
        gr.append(timed(g.replay))
    out["step_ms"] = {"eager": round(float(np.median(eg)) / 1e3, 3), "graph": round(float(np.median(gr)) / 1e3, 3),
                      "rounds": 3}
    return out


def skinny_sweep(dpg, dpg_inputs, torch, to_dev, cold):
    """The skinny-N weight gradients at every (K -> N, T) point, BF16 and FP32
    output, under the planner's plan and with one and two forced splits, each
    timed under the cold-cache protocol (ColdTimer).  GB/s are of algorithmic
    bytes 2TK + 2TN + ob N K (ob = 2 or 4), the split reduction included in the
    time.  The FP32 planner plans at T = 16384 and 65537 are also timed warm
    (back to back, operands in the Infinity Cache where they fit) for
    comparison."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    rows = []
    for T_S in SKINNY_T_ALL:
        progress("skinny weight gradients, T = %d" % T_S)
        for K, N in SKINNY:
            xs = to_dev(dpg_inputs.normal_bf16((T_S, K), 1.0, 0, 0))
            dys = to_dev(dpg_inputs.normal_bf16((T_S, N), 1.0, 0, 2))
            for out_dtype, ob, oname in ((torch.bfloat16, 2, "bf16"), (torch.float32, 4, "f32")):
                out = torch.empty((N, K), dtype=out_dtype, device=dev)
                for det, split in SKINNY_MODES:
                    ws_n = dpg.workspace_size(dpg.PASS_WGRAD, T_S, N, K, out_dtype, det, split)
                    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
                    call = (lambda det=det, split=split, ws=ws, out=out:
                            dpg.dpg_wgrad(dys, xs, out=out, deterministic=det, split_k=split, workspace=ws))
                    us, lo, hi = cold(call)
                    span = cold.last_span
                    rus, _, _ = cold(call, flush="read")
                    rspan = cold.last_span
                    nbytes = 2.0 * T_S * K + 2.0 * T_S * N + ob * N * K
                    plan = dpg.parse_plan(dpg.plan_describe(dpg.PASS_WGRAD, T_S, N, K, out_dtype, det, split))
                    row = {"shape": "%d->%d" % (K, N), "T": T_S, "out": oname,
                           "mode": "planner" if det else "split_k=%d" % split,
                           "us_cold_median": round(us, 2), "group_median_range_us": [round(lo, 2), round(hi, 2)],
                           "GBps": round(nbytes / us / 1e3, 1), "frac_hbm": round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4),
                           "us_cold_read_flush": round(rus, 2),
                           "frac_hbm_read_flush": round(nbytes / rus / 1e3 / PEAK_HBM_GBPS, 4),
                           "splits": int(plan["splits"]), "unit": plan["tile"], "grid": int(plan["grid"])}
                    if span and rspan:
                        row.update({"us_span_cold": round(span[0], 2),
                                    "frac_hbm_span": round(nbytes / span[0] / 1e3 / PEAK_HBM_GBPS, 4),
                                    "us_span_read_flush": round(rspan[0], 2),
                                    "frac_hbm_span_read_flush": round(nbytes / rspan[0] / 1e3 / PEAK_HBM_GBPS, 4)})
                    if det and oname == "f32" and T_S in (16384, 65537):
                        reps = 50
                        for _ in range(5):
                            call()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for _ in range(reps):
                            call()
                        e1.record(stream)
                        torch.cuda.synchronize()
                        wus = e0.elapsed_time(e1) * 1e3 / reps
                        row["us_warm_mean"] = round(wus, 2)
                        row["GBps_warm"] = round(nbytes / wus / 1e3, 1)
                    rows.append(row)
                    del ws
                del out
            del xs, dys
            torch.cuda.empty_cache()
    return rows


def secondary_configs(dpg, dpg_inputs, torch, to_dev, cold):
    """The other measured workloads, microseconds per call: the 4096->1024
    projection at T = 64 (BF16, deterministic), the FP32 router (E = 256,
    H = 4096) at T = 64 / 256 / 1024 in the deterministic mode, in the
    split-K mode and with FP32 fused multiply-adds forced (the plans are
    reported), and the
    checkpointed step (forward, forward, input gradient, weight gradient; FP32
    out) of 4096->1024 and 4096->512 at T = 16384, whole and per op (the op
    alone also under the cold-cache protocol).  Each is timed eagerly (host
    launch included) and as a captured HIP graph of the same calls (device
    time only); us_host is the host time of the eager calls (the binding's
    checks, the plan lookup and the launches), as the router page reports its
    entry points' host time per eager call."""
    import numpy as np
    dev = torch.device("cuda:0")

    def timed(calls, reps=20):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                for c in calls:
                    c()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        h0 = time.perf_counter()
        for _ in range(reps):
            for c in calls:
                c()
        host = (time.perf_counter() - h0) * 1e6 / reps
        e1.record()
        torch.cuda.synchronize()
        eager = e0.elapsed_time(e1) * 1e3 / reps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                for c in calls:
                    c()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph = e0.elapsed_time(e1) * 1e3 / reps
        timed.host = round(host, 2)
        return round(eager, 2), round(graph, 2)

    def ws(pass_, T, N, K, out_dtype, det, split):
        n = dpg.workspace_size(pass_, T, N, K, out_dtype, det, split)
        return torch.empty(max(n, 16), dtype=torch.uint8, device=dev)

    out = {}
    # 4096 -> 1024 at T = 64
    T, N, K = 64, 1024, 4096
    x, w, dy = dpg_inputs.dense(T, N, K, seed_group=0)
    X, W, DY = to_dev(x), to_dev(w), to_dev(dy)
    Y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    DX = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    DW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    wsf, wsd, wsw = (ws(p, T, N, K, torch.bfloat16, True, 0) for p in (0, 1, 2))
    small = {}
    for name, call in [("fwd", lambda: dpg.dpg_forward(X, W, out=Y, workspace=wsf)),
                       ("dgrad", lambda: dpg.dpg_dgrad(DY, W, out=DX, workspace=wsd)),
                       ("wgrad", lambda: dpg.dpg_wgrad(DY, X, out=DW, workspace=wsw))]:
        e, g = timed([call])
        small[name] = {"us_eager": e, "us_graph": g, "us_host": timed.host}
    out["projection_4096x1024_T64_bf16"] = small

    # router, FP32 via BF16x3
    E, H = 256, 4096
    router = {}
    for T in (64, 256, 1024):
        xr, wr, dyr = dpg_inputs.router(T, E, H, seed_group=0)
        Xr, Wr, DYr = (torch.from_numpy(a).to(dev) for a in (xr, wr, dyr))
        Yr = torch.empty((T, E), dtype=torch.float32, device=dev)
        DXr = torch.empty((T, H), dtype=torch.float32, device=dev)
        DWr = torch.empty((E, H), dtype=torch.float32, device=dev)
        modes = {}
        for mode, det, split in [("deterministic", True, 0), ("split_k_mode", False, 0), ("fp32fma", True, 0)]:
            prev_arith = dpg.set_router_arithmetic("fp32" if mode == "fp32fma" else "auto")
            w3 = [ws(p, T, E, H, torch.float32, det, split) for p in (3, 4, 5)]
            fwd = lambda: dpg.dpg_router_forward(Xr, Wr, out=Yr, deterministic=det, split_k=split, workspace=w3[0])
            dgr = lambda: dpg.dpg_router_dgrad(DYr, Wr, out=DXr, deterministic=det, split_k=split, workspace=w3[1])
            wgr = lambda: dpg.dpg_router_wgrad(DYr, Xr, out=DWr, deterministic=det, split_k=split, workspace=w3[2])
            rec = {}
            for name, calls in [("fwd", [fwd]), ("dgrad", [dgr]), ("wgrad", [wgr]),
                                ("2fwd+bwd", [fwd, fwd, dgr, wgr])]:
                e, g = timed(calls)
                rec[name] = {"us_eager": e, "us_graph": g, "us_host": timed.host}
            rec["plans"] = {n: "%(kernel)s %(arith)s splits=%(splits)s" % dpg.parse_plan(
                dpg.plan_describe(p, T, E, H, torch.float32, det, split)) for n, p in (("fwd", 3), ("dgrad", 4), ("wgrad", 5))}
            dpg.set_router_arithmetic(prev_arith)
            modes[mode] = rec
        router["T%d" % T] = modes
    out["router_E256_H4096_f32"] = router

    # checkpointed step, FP32 out: the step (graph and eager) and each op alone
    # (warm event mean and the cold-cache median)
    T, K = 16384, 4096
    xs = to_dev(dpg_inputs.normal_bf16((T, K), 1.0, 0, 0))
    step = {}
    for N in (1024, 512):
        Ws = to_dev(dpg_inputs.normal_bf16((N, K), dpg_inputs.SIGMA_W, 0, 1))
        DYs = to_dev(dpg_inputs.normal_bf16((T, N), 1.0, 0, 2))
        Ys = torch.empty((T, N), dtype=torch.float32, device=dev)
        DXs = torch.empty((T, K), dtype=torch.float32, device=dev)
        DWs = torch.empty((N, K), dtype=torch.float32, device=dev)
        w3 = [ws(p, T, N, K, torch.float32, True, 0) for p in (0, 1, 2)]
        ops = [("fwd", lambda: dpg.dpg_forward(xs, Ws, out=Ys, workspace=w3[0])),
               ("dgrad", lambda: dpg.dpg_dgrad(DYs, Ws, out=DXs, workspace=w3[1])),
               ("wgrad", lambda: dpg.dpg_wgrad(DYs, xs, out=DWs, workspace=w3[2]))]
        calls = [ops[0][1], ops[0][1], ops[1][1], ops[2][1]]
        e, g = timed(calls, reps=10)
        flop = 8.0 * T * N * K
        rec = {"us_eager": e, "us_graph": g, "tflops_graph": round(flop / g / 1e6, 1),
               "frac_peak_graph": round(flop / g / 1e6 / PEAK_BF16_TFLOPS, 4), "ops": {}}
        flop_op = 2.0 * T * N * K
        for name, fn in ops:
            e1, g1 = timed([fn], reps=10)
            cus, _, _ = cold(fn)
            cspan = cold.last_span
            p = dpg.parse_plan(dpg.plan_describe({"fwd": 0, "dgrad": 1, "wgrad": 2}[name], T, N, K, torch.float32))
            rec["ops"][name] = {"us_graph": g1, "tflops_graph": round(flop_op / g1 / 1e6, 1),
                                "frac_peak_graph": round(flop_op / g1 / 1e6 / PEAK_BF16_TFLOPS, 4),
                                "us_cold_median": round(cus, 1),
                                "frac_peak_cold": round(flop_op / cus / 1e6 / PEAK_BF16_TFLOPS, 4),
                                "us_span_cold": round(cspan[0], 1) if cspan else None,
                                "plan": "%s %s splits=%s" % (p["kernel"], p["tile"], p["splits"])}
            cnt = read_step5_counters(N, name)
            if cnt:
                rec["ops"][name]["counters"] = cnt
        step["4096x%d" % N] = rec
        del Ws, DYs, Ys, DXs, DWs
    out["checkpointed_step_T16384_f32"] = step
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-skinny", action="store_true")
    ap.add_argument("--no-spans", action="store_true",
                    help="cold-cache timings without torch's profiler (kernel spans), e.g. under rocprofv3")
    ap.add_argument("--skip-secondary", action="store_true", help="skip the small, router and step timings")
    ap.add_argument("--profile-run", action="store_true", help="one step + a 1 GiB calibration copy (for rocprofv3)")
    ap.add_argument("--clock-load", type=float, metavar="SECONDS",
                    help="run the forward GEMM in a loop for SECONDS (to read the clock under load)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "COMMAND"))
    ap.add_argument("--bench-log", help="with --summarize-trace: output of the traced bench run")
    ap.add_argument("--summarize-busy", nargs=2, metavar=("COUNTER_CSV", "COMMAND"))
    ap.add_argument("--profile-skinny", action="store_true",
                    help="the skinny weight gradients once each after a 1 GiB calibration copy (for rocprofv3)")
    ap.add_argument("--summarize-skinny-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"))
    ap.add_argument("--profile-step5", action="store_true",
                    help="the checkpointed step's ops once each after the calibration kernels (for rocprofv3)")
    ap.add_argument("--summarize-step5", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "BUSY_CSV", "COMMAND"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="OUT_NAME COMMAND CSV [CSV ...]: all counters of the GEMM passes")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, bench_log=args.bench_log)
        return
    if args.summarize_busy:
        summarize_busy(*args.summarize_busy)
        return
    if args.summarize_skinny_pmc:
        summarize_skinny_pmc(*args.summarize_skinny_pmc)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_step5:
        summarize_step5(*args.summarize_step5)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    if args.profile_run:
        profile_run()
        return
    if args.profile_skinny:
        profile_skinny()
        return
    if args.profile_step5:
        profile_step5()
        return
    if args.clock_load:
        clock_load(args.clock_load)
        return

    import numpy as np
    import torch
    import dpg_inputs
    import deterministic_bf16_projection_amd as dpg

    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, w, dy = dpg_inputs.dense(T_BIG, N_BIG, K_BIG, seed_group=0)
    X, W, DY = to_dev(x), to_dev(w), to_dev(dy)
    del x, w, dy
    Y = torch.empty((T_BIG, N_BIG), dtype=torch.bfloat16, device=dev)
    DX = torch.empty((T_BIG, K_BIG), dtype=torch.bfloat16, device=dev)
    DW = torch.empty((N_BIG, K_BIG), dtype=torch.bfloat16, device=dev)
    passes = [
        ("fwd", lambda: dpg.dpg_forward(X, W, out=Y)),
        ("dgrad", lambda: dpg.dpg_dgrad(DY, W, out=DX)),
        ("wgrad", lambda: dpg.dpg_wgrad(DY, X, out=DW)),
    ]
    plans = {name: dpg.plan_describe(i, T_BIG, N_BIG, K_BIG) for i, (name, _) in enumerate(passes)}
    flop_pass = 2.0 * T_BIG * N_BIG * K_BIG

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for _, fn in passes:
            fn()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps; events around every pass on the launch stream
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in passes]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for p, (_, fn) in enumerate(passes):
            ev[s][p][0].record(stream)
            fn()
            ev[s][p][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per_pass = {}
    for p, (name, _) in enumerate(passes):
        ts = [ev[s][p][0].elapsed_time(ev[s][p][1]) for s in range(args.steps)]
        us = 1e3 * float(np.mean(ts))
        per_pass[name] = {"us_mean": round(us, 1), "us_min": round(1e3 * min(ts), 1),
                          "tflops": round(flop_pass / us / 1e6, 1),
                          "frac_peak": round(flop_pass / us / 1e6 / PEAK_BF16_TFLOPS, 4),
                          "plan": plans[name]}
    value = 3 * flop_pass / (ms_step * 1e-3) / 1e12

    dominant = max(per_pass, key=lambda k: per_pass[k]["us_mean"])
    achieved = flop_pass / (per_pass[dominant]["us_mean"] * 1e-6) / 1e12
    traffic = read_traffic(dominant)
    roofline = {"bound": "mfma", "kernel": "gemm_fast_kernel (%s pass, 256x256x64 tile)" % dominant,
                "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flop_per_launch": flop_pass}
    clk = clock_under_load()
    if clk:
        adj = PEAK_BF16_TFLOPS * clk / 2.4
        roofline["clock_adjusted"] = {"clock_ghz": clk, "peak": round(adj, 1), "frac": round(achieved / adj, 4),
                                      "source": "rocm-smi sclk under sustained forward-GEMM load (profiles/)"}
    busy = read_mfma_busy(dominant)
    if busy:
        roofline["counters"] = busy
    progress("timed steps done")
    cold = ColdTimer(torch, spans=not args.no_spans)
    passes_cold = cold_cache_passes(passes, cold)
    progress("cold-cache passes done")
    more = config3_more(dpg, torch, X, W, DY, Y, DX, DW, passes)
    progress("4096->12288 extras done")

    skinny, hbm_ref = [], None
    if not args.skip_skinny:
        del Y, DX, DW
        torch.cuda.empty_cache()
        skinny = skinny_sweep(dpg, dpg_inputs, torch, to_dev, cold)
        hbm_ref = hbm_read_reference(torch, cold)

    progress("skinny done")
    secondary = None if args.skip_secondary else secondary_configs(dpg, dpg_inputs, torch, to_dev, cold)
    cold.close()
    progress("other workloads done")

    cpu = None if args.no_cpu_baseline else cpu_baseline()
    cpu_small = None if args.no_cpu_baseline else cpu_oracle_small()
    progress("cpu baseline done")

    line = {
        "metric": "TFLOP/s and % BF16 MFMA peak per pass, 4096->12288 T=16384; skinny wgrad GB/s",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "projection 4096->12288 (K=4096, N=12288), T=16384 tokens: forward + input "
                               "gradient + weight gradient, BF16 in/out, FP32 accumulation, deterministic plan",
                   "T": T_BIG, "N": N_BIG, "K": K_BIG, "global_batch": T_BIG, "parallelism": "single GPU"},
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "passes": per_pass,
        "passes_cold_cache": passes_cold,
        "projection_4096x12288_more": more,
        "skinny_wgrad": skinny,
        "hbm_read_reference": hbm_ref,
        "other_workloads": secondary,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_oracle_small_configs": cpu_small,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
