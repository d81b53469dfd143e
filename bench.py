"""Benchmark of the MoDA fused forward on one MI355X.

Workload: the long-context layer, B=1, T=65536, Hq=16, Hk=4 (G=4), d=128,
L=48 depth slots, bf16 inputs N(0,1), causal; the same shape with L=0 is the
causal-attention denominator (same library, same kernel family, same inputs).

One step is one pass of the whole path over the resident inputs:
  1. pack the depth K and V streams [B,T,L,Hk,d] -> [B,T,Hk,L,d],
  2. MoDA forward with L=48,
  3. the L=0 causal forward on the same q / k_seq / v_seq.
W untimed warm-up steps, then K timed steps between two device
synchronisations.  Every launch is also bracketed by HIP events on the stream
it runs on (torch's current stream), which give each kernel's average
duration.

value = forward flops of the L=48 MoDA forward / its average kernel time
(TFLOP/s); ratio_vs_l0 = that time / the L=0 kernel time.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from depth_stream_attention_amd import _lib, api  # noqa: E402
from depth_stream_attention_amd import accounting as acc  # noqa: E402
from depth_stream_attention_amd import inputs as I  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "depth_stream_attention_amd", "csrc", "moda_fwd_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moda_fwd_bf16_long_L48_traffic.json")


def _code_text(text):
    """Source text without comments and blank runs, so that comment edits keep the hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash():
    """Hash of the forward kernel's code (sources without comments) and its build flags: the
    counters describe one binary."""
    from depth_stream_attention_amd import build as pkg_build
    h = hashlib.sha256()
    for name in ("moda_fwd_bf16.hip", "moda_tile.h", "moda_device.h"):
        with open(os.path.join(ROOT, "depth_stream_attention_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_text(f.read()).encode())
    flags = [f for f in pkg_build.HIPCC_FLAGS if not f.startswith("-I")]  # include paths vary by checkout
    h.update(" ".join(flags + pkg_build.SOURCE_FLAGS.get("moda_fwd_bf16.hip", [])).encode())
    return h.hexdigest()[:16]


def traffic_record():
    """The committed rocprofv3 counter record of the forward (HBM bytes per launch of the
    L=48 and L=0 kernels), if it was taken on the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec


def cpu_baseline(shape, host, budget_s):
    """Time the fp64 oracle (test infrastructure) on a bounded sample of rows of the same
    workload; returns the record and the sampled rows' max error against the GPU output."""
    import oracle
    rng = np.random.default_rng(12345)
    threads = oracle.default_threads()
    done_flops, done_rows, spent = 0, 0, 0.0
    rows_all, ref_all = [], []
    while spent < budget_s:
        n = 64
        rows = np.stack([np.zeros(n, np.int64), rng.integers(0, shape.T, n), rng.integers(0, shape.Hq, n)],
                        axis=1).astype(np.int32)
        t0 = time.perf_counter()
        ref, ref_lse = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"], host["k_depth"],
                                            host["v_depth"], rows, causal=True, nthreads=threads)
        spent += time.perf_counter() - t0
        done_rows += n
        done_flops += int(sum(4 * shape.d * (int(t) + 1 + shape.L) for t in rows[:, 1]))
        rows_all.append(rows)
        ref_all.append(ref)
    rec = {"value": done_flops / spent / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": "%d uniformly drawn (t, h) rows of the L=%d workload, %.1f s of fp64 oracle time "
                     "on %d host threads" % (done_rows, shape.L, spent, threads)}
    return rec, np.concatenate(rows_all), np.concatenate(ref_all)


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _kernel_label(name):
    if "moda_fwd_bf16_kernel" in name:
        depth = name.split("<")[1].split(",")[1].strip()
        return "moda_fwd_bf16 L=48" if depth == "true" else "moda_fwd_bf16 L=0"
    if "pack_kernel" in name:
        return "moda_pack_depth"
    if "moda_decode_partial_kernel" in name:
        return "moda_decode partial"
    if "moda_decode_merge_kernel" in name:
        return "moda_decode merge"
    for k in ("rows", "depth", "dq", "dkv"):
        if "moda_bwd_%s_kernel" % k in name:
            return "moda_bwd %s" % k
    if "moda_kv_project_kernel" in name:
        return "moda_kv_project"
    return None


def _sq_lines(sq_dir, command):
    """Per-kernel SQ counter figures (one rocprofv3 --pmc pass)."""
    vals = {}
    for r in _read_csv(os.path.join(sq_dir, "run_counter_collection.csv")):
        lab = _kernel_label(r["Kernel_Name"])
        if lab:
            vals.setdefault(lab, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    lines = ["", "SQ counters (one rocprofv3 --pmc pass):", "  command: " + command, ""]
    for lab, v in sorted(vals.items()):
        gui = v.get("GRBM_GUI_ACTIVE", 0.0)
        simd_cycles = gui / 8.0 * 256 * 4  # GRBM_GUI_ACTIVE sums the 8 XCDs; 256 CUs x 4 SIMDs
        lines.append("  %s: " % lab + ", ".join("%s=%.4g" % (k, x) for k, x in sorted(v.items())))
        if gui and v.get("SQ_INSTS_MFMA"):
            lines.append("    MFMA busy %.1f%% of SIMD cycles; VALU/MFMA instructions %.2f; LDS bank conflicts / "
                         "LDS active %.4f" % (100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles,
                                              v["SQ_INSTS_VALU"] / v["SQ_INSTS_MFMA"],
                                              v["SQ_LDS_BANK_CONFLICT"] / max(1.0, v["SQ_LDS_IDX_ACTIVE"])))
        if gui and v.get("SQ_VALU_MFMA_COEXEC_CYCLES"):
            lines.append("    VALU issued while MFMA busy: %.1f%% of SIMD cycles"
                         % (100.0 * v["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles))
        for name, what in (("SQ_WAIT_INST_ANY", "waiting for an instruction to issue"),
                           ("SQ_WAIT_INST_LDS", "waiting to issue an LDS instruction")):
            if v.get("SQ_WAVE_CYCLES") and v.get(name):  # both in quad-cycles
                lines.append("    waves %s: %.1f%% of wave cycles" % (what, 100.0 * v[name] / v["SQ_WAVE_CYCLES"]))
    return lines


def _decode_summary(stats, counters, f_scale, w_scale, command):
    """profiles/moda_decode_b16_t64k.txt: the decode step of the same bench run."""
    ds = DECODE_SHAPE
    dbytes = acc.decode_bytes(ds["B"], ds["T"], ds["Hq"], ds["Hk"], ds["d"], ds["L"])
    lines = ["# rocprofv3 summary: MoDA decode step, B=%d T=%d Hq=%d Hk=%d d=%d L=%d, bf16"
             % (ds["B"], ds["T"], ds["Hq"], ds["Hk"], ds["d"], ds["L"]), "",
             "kernel trace (rocprofv3 --kernel-trace --stats):", "  command: " + command[0], "",
             "  %-22s %6s %12s %12s %12s" % ("kernel", "calls", "avg ms", "min ms", "max ms")]
    for lab in ("moda_decode partial", "moda_decode merge"):
        n, avg, mn, mx = stats[lab]
        lines.append("  %-22s %6d %12.4f %12.4f %12.4f" % (lab, n, avg, mn, mx))
    dms = stats["moda_decode partial"][1] + stats["moda_decode merge"][1]
    lines += ["", "  decode step: partial + merge %.4f ms; %d algorithmic bytes -> %.1f GB/s (%.1f%% of 8 TB/s)"
              % (dms, dbytes, dbytes / dms / 1e6, dbytes / dms / 1e6 / PEAK_HBM_GBS * 100), "",
              "HBM traffic per launch (FETCH_SIZE / WRITE_SIZE passes of the same commands, calibrated on the",
              "depth packer: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f):" % (f_scale, w_scale),
              "  commands: " + command[1], "            " + command[2], ""]
    for lab in ("moda_decode partial", "moda_decode merge"):
        rd = counters["FETCH_SIZE"].get(lab, 0.0) * f_scale
        wr = counters["WRITE_SIZE"].get(lab, 0.0) * w_scale
        lines.append("  %-22s read %.4g B  write %.4g B" % (lab, rd, wr))
    with open(os.path.join(os.path.dirname(TRAFFIC_FILE), "moda_decode_b16_t64k.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _bwd_summary(stats, counters, f_scale, w_scale, command):
    """profiles/moda_bwd_long_L48.txt: the backward kernels of the same bench run."""
    shape = I.workload(5, 0)
    B, T, Hq, Hk, d, L = shape.B, shape.T, shape.Hq, shape.Hk, shape.d, shape.L
    P = acc.visible_pairs(T, True)
    # Products each kernel executes (2*d flops per pair each): dq recomputes S and dP, then dS K;
    # dkv computes S, dP, then P^T dO and dS^T Q; depth does all five (and S, dP twice) on 16-row tiles.
    f_dq, f_dkv = 6 * d * B * Hq * P, 8 * d * B * Hq * P
    b_depth = 2 * acc.depth_bytes(shape) + 2 * B * T * Hq * d * 2 + B * T * Hq * d * 4
    lines = ["# rocprofv3 summary: MoDA backward, long-context layer B=%d T=%d Hq=%d Hk=%d d=%d, L=%d and L=0, bf16"
             % (B, T, Hq, Hk, d, L), "",
             "kernel trace (rocprofv3 --kernel-trace --stats):", "  command: " + command[0], "",
             "  %-22s %6s %12s %12s %12s" % ("kernel", "calls", "avg ms", "min ms", "max ms")]
    for lab in ("moda_bwd rows", "moda_bwd depth", "moda_bwd dq", "moda_bwd dkv"):
        if lab in stats:
            n, avg, mn, mx = stats[lab]
            lines.append("  %-22s %6d %12.4f %12.4f %12.4f" % (lab, n, avg, mn, mx))
    lines.append("")
    if "moda_bwd dq" in stats:
        lines.append("  dq:  %.1f TFLOP/s of its three products (%.4g flop)" % (f_dq / stats["moda_bwd dq"][1] / 1e9,
                                                                             f_dq))
    if "moda_bwd dkv" in stats:
        lines.append("  dkv: %.1f TFLOP/s of its four products (%.4g flop)"
                     % (f_dkv / stats["moda_bwd dkv"][1] / 1e9, f_dkv))
    if "moda_bwd depth" in stats:
        lines.append("  depth: %.1f GB/s of its minimum bytes (%.4g B: depth K/V in, their gradients out, "
                     "q and dout in, fp32 dq share out)" % (b_depth / stats["moda_bwd depth"][1] / 1e6, b_depth))
    lines += ["", "  (the rows and depth kernels run only in the L=48 call; dq and dkv in both, so their",
              "   averages mix the L=48 and L=0 calls, which differ only in the depth share dq adds)", "",
              "HBM traffic per launch (FETCH_SIZE / WRITE_SIZE passes, calibrated on the depth packer:",
              "FETCH_SIZE x %.4f, WRITE_SIZE x %.4f):" % (f_scale, w_scale),
              "  commands: " + command[1], "            " + command[2], ""]
    for lab in ("moda_bwd rows", "moda_bwd depth", "moda_bwd dq", "moda_bwd dkv"):
        rd = counters["FETCH_SIZE"].get(lab, 0.0) * f_scale
        wr = counters["WRITE_SIZE"].get(lab, 0.0) * w_scale
        lines.append("  %-22s read %.4g B  write %.4g B" % (lab, rd, wr))
    with open(os.path.join(os.path.dirname(TRAFFIC_FILE), "moda_bwd_long_L48.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _kvproj_summary(stats, counters, f_scale, w_scale, command):
    """profiles/moda_kv_project_long.txt: the depth-write KV projection of the same bench run."""
    s = KVPROJ_SHAPE
    F = acc.kv_project_flops(s["B"], s["T"], s["Dm"], s["Hk"], s["d"])
    byts = acc.kv_project_bytes(s["B"], s["T"], s["Dm"], s["Hk"], s["d"])
    n, avg, mn, mx = stats["moda_kv_project"]
    rd = counters["FETCH_SIZE"].get("moda_kv_project", 0.0) * f_scale
    wr = counters["WRITE_SIZE"].get("moda_kv_project", 0.0) * w_scale
    lines = ["# rocprofv3 summary: depth write (KV projection into the sequence K/V and one packed depth slot),",
             "# B=%d T=%d Dm=%d Hk=%d d=%d, bf16" % (s["B"], s["T"], s["Dm"], s["Hk"], s["d"]), "",
             "kernel trace (rocprofv3 --kernel-trace --stats):", "  command: " + command[0], "",
             "  %-22s %6s %12s %12s %12s" % ("kernel", "calls", "avg ms", "min ms", "max ms"),
             "  %-22s %6d %12.4f %12.4f %12.4f" % ("moda_kv_project", n, avg, mn, mx), "",
             "  %.1f TFLOP/s (%.4g flop; %.1f%% of the 2.5 PFLOP/s bf16 peak)" % (F / avg / 1e9, F,
                                                                                 F / avg / 1e9 / PEAK_BF16_TFLOPS * 100),
             "", "HBM traffic per launch (FETCH_SIZE / WRITE_SIZE passes, calibrated on the depth packer:",
             "FETCH_SIZE x %.4f, WRITE_SIZE x %.4f):" % (f_scale, w_scale),
             "  commands: " + command[1], "            " + command[2], "",
             "  read %.4g B  write %.4g B  (minimum: %.4g B = x and w read once, every output written to both"
             % (rd, wr, byts), "  destinations)"]
    with open(os.path.join(os.path.dirname(TRAFFIC_FILE), "moda_kv_project_long.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize(trace_dir, fetch_dir, write_dir, command, sq_dir=None):
    """Turn rocprofv3 CSVs of this benchmark into the committed summary and traffic record.

    FETCH_SIZE / WRITE_SIZE are calibrated on the depth packer, a plain copy kernel of known
    size (it reads and writes 2*B*T*L*Hk*d bytes per launch)."""
    shape = I.workload(5, 0)
    pack_bytes = acc.depth_bytes(shape) / 2  # one of K / V
    stats = {}
    for r in _read_csv(os.path.join(trace_dir, "run_kernel_stats.csv")):
        lab = _kernel_label(r["Name"])
        if lab:
            stats[lab] = (int(r["Calls"]), float(r["AverageNs"]) / 1e6, float(r["MinNs"]) / 1e6,
                          float(r["MaxNs"]) / 1e6)
    counters = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        vals = {}
        for r in _read_csv(os.path.join(d, "run_counter_collection.csv")):
            lab = _kernel_label(r["Kernel_Name"])
            if lab and r["Counter_Name"] == cname:
                vals.setdefault(lab, []).append(float(r["Counter_Value"]) * 1024.0)  # KiB -> bytes
        counters[cname] = {k: float(np.mean(v)) for k, v in vals.items()}
    f_scale = pack_bytes / counters["FETCH_SIZE"]["moda_pack_depth"]
    w_scale = pack_bytes / counters["WRITE_SIZE"]["moda_pack_depth"]
    lines = ["# rocprofv3 summary: MoDA forward, long-context layer B=1 T=65536 Hq=16 Hk=4 d=128, bf16",
             "", "kernel trace (rocprofv3 --kernel-trace --stats):", "  command: " + command[0], "",
             "  %-22s %6s %12s %12s %12s" % ("kernel", "calls", "avg ms", "min ms", "max ms")]
    for lab, (n, avg, mn, mx) in sorted(stats.items()):
        lines.append("  %-22s %6d %12.4f %12.4f %12.4f" % (lab, n, avg, mn, mx))
    F = acc.flops(shape)
    F0 = acc.flops(I.workload(5, 1))
    avg48, avg0 = stats["moda_fwd_bf16 L=48"][1], stats["moda_fwd_bf16 L=0"][1]
    lines += ["", "  MoDA L=48: %.1f TFLOP/s (%.4g flop / %.4f ms); L=0: %.1f TFLOP/s; ratio %.4f" % (
        F / avg48 / 1e9, F, avg48, F0 / avg0 / 1e9, avg48 / avg0)]
    lines += ["",
        "HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, separate runs):",
        "  commands: " + command[1], "            " + command[2],
        "  calibration on moda_pack_depth (reads and writes %d bytes): FETCH_SIZE x %.4f, WRITE_SIZE x %.4f"
        % (pack_bytes, f_scale, w_scale), ""]
    traffic, reads = {}, {}
    for lab in ("moda_fwd_bf16 L=48", "moda_fwd_bf16 L=0", "moda_pack_depth"):
        rd = counters["FETCH_SIZE"].get(lab, 0.0) * f_scale
        wr = counters["WRITE_SIZE"].get(lab, 0.0) * w_scale
        traffic[lab] = rd + wr
        reads[lab] = rd
        lines.append("  %-22s read %.4g B  write %.4g B  total %.4g B" % (lab, rd, wr, rd + wr))
    alg = acc.algorithmic_bytes(shape)
    lines.append("  algorithmic bytes of the L=48 forward: %.4g B (traffic / algorithmic = %.3f)"
                 % (alg, traffic["moda_fwd_bf16 L=48"] / alg))
    for k, d in enumerate(sq_dir or []):
        lines += _sq_lines(d, command[3 + k] if len(command) > 3 + k else "")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(os.path.join(os.path.dirname(TRAFFIC_FILE), "moda_fwd_bf16_long_L48.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if "moda_decode partial" in stats and "moda_decode merge" in stats:
        _decode_summary(stats, counters, f_scale, w_scale, command)
    if "moda_bwd dkv" in stats:
        _bwd_summary(stats, counters, f_scale, w_scale, command)
    if "moda_kv_project" in stats:
        _kvproj_summary(stats, counters, f_scale, w_scale, command)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"kernel": "moda_fwd_bf16 L=48", "kernel_source_hash": kernel_source_hash(),
                   "hbm_bytes_per_launch": traffic["moda_fwd_bf16 L=48"],
                   "read_bytes_per_launch": reads["moda_fwd_bf16 L=48"],
                   "l0_read_bytes_per_launch": reads["moda_fwd_bf16 L=0"],
                   "fetch_scale": f_scale, "write_scale": w_scale}, f, indent=1)
    print("\n".join(lines))


def peaks_leg(iters=10):
    """Attainable peaks on this GPU from the measurement kernels of libmoda_probe.so: the bf16
    matrix-core rate (register-only v_mfma_f32_32x32x16_bf16 chains, 32 waves per SIMD) with
    pseudo-random operands (switching data, as in real tiles) and with constant operands, and
    HBM copy and read bandwidth over 4 GiB buffers; each the median of `iters` HIP-event-timed
    launches after one warm-up.  Reported beside the published peaks, which stay the roofline
    denominators."""
    import ctypes
    probe = _lib.load_probe()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn):
        fn()
        t = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return float(np.median(t))

    def check(rc):
        if rc != 0:
            raise RuntimeError("probe failed with code %d" % rc)

    blocks, mf_iters = 8192, 2048  # 32768 waves: 32 per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    mf = {}
    for random in (1, 0):
        ms = timed(lambda: check(probe.moda_probe_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), blocks, mf_iters,
                                                            random, sp)))
        mf[random] = blocks * 4 * 4 * mf_iters * 32768 / (ms * 1e-3) / 1e12
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    gblocks = 16384
    rsink = torch.empty(gblocks * 256, dtype=torch.int32, device="cuda")
    ms_c = timed(lambda: check(probe.moda_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                                     nbytes, gblocks, sp)))
    ms_r = timed(lambda: check(probe.moda_probe_read(ctypes.c_void_p(src.data_ptr()), nbytes, gblocks,
                                                     ctypes.c_void_p(rsink.data_ptr()), sp)))
    del sink, src, dst, rsink
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mf[1], 1), "mfma_bf16_tflops_constant_operands": round(mf[0], 1),
            "hbm_copy_gbs": round(2 * nbytes / (ms_c * 1e-3) / 1e9, 1),
            "hbm_read_gbs": round(nbytes / (ms_r * 1e-3) / 1e9, 1),
            "note": "measured on this GPU by libmoda_probe.so (median of %d launches). mfma_bf16_tflops uses "
                    "pseudo-random operands; with constant operands the matrix core draws less power and "
                    "keeps a higher clock. The published peaks 2500 TFLOP/s bf16 dense and 8000 GB/s HBM "
                    "remain the roofline denominators" % iters}


DECODE_SHAPE = dict(B=16, T=65536, Hq=16, Hk=4, d=128, L=48)


def decode_leg(iters=20, warmup=3):
    """The decode step at the long-context layer's head shapes, batch 16: HBM-bound, timed with
    HIP events on the current stream after warm-up; inputs resident in HBM."""
    s = DECODE_SHAPE
    B, T, Hq, Hk, d, L = s["B"], s["T"], s["Hq"], s["Hk"], s["d"], s["L"]
    g = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn(B, Hq, d, device="cuda", generator=g).bfloat16()
    kc = torch.randn(B, T, Hk, d, device="cuda", generator=g).bfloat16()
    vc = torch.randn(B, T, Hk, d, device="cuda", generator=g).bfloat16()
    kd = torch.randn(B, Hk, L, d, device="cuda", generator=g).bfloat16()
    vd = torch.randn(B, Hk, L, d, device="cuda", generator=g).bfloat16()
    ws = torch.empty(api.moda_attn_decode_workspace(B, T, Hq, Hk, d, L), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        api.moda_attn_decode(q, kc, vc, kd, vd, out, lse, ws)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        api.moda_attn_decode(q, kc, vc, kd, vd, out, lse, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    byts = acc.decode_bytes(B, T, Hq, Hk, d, L)
    gbs = byts / (ms * 1e-3) / 1e9
    del q, kc, vc, kd, vd, ws
    return {"workload": "decode step B=16 T=65536 Hq=16 Hk=4 d=128 L=48 (KV cache + depth slots)",
            "ms": round(ms, 4), "bytes": byts,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def backward_leg(shape, dev, kd, vd, out, lse, out0, lse0, iters=4):
    """The backward of the long-context layer (L=48, and L=0 for the ratio) for the forward's
    saved (out, lse), timed with HIP events on the current stream after one warm-up call;
    inputs and the output gradient resident in HBM, L=48 and L=0 calls interleaved."""
    shape0 = I.workload(5, 1)
    dout = I.random_dout(shape, 7005, device="cuda")
    B, T, Hq, Hk, d, L = shape.B, shape.T, shape.Hq, shape.Hk, shape.d, shape.L
    ws = torch.empty(api.moda_attn_bwd_workspace(B, T, Hq, Hk, d, L), dtype=torch.uint8, device="cuda")
    grads = (torch.empty_like(dev["q"]), torch.empty_like(dev["k_seq"]), torch.empty_like(dev["v_seq"]),
             torch.empty_like(kd), torch.empty_like(vd))
    grads0 = grads[:3] + (None, None)
    stream = torch.cuda.current_stream()

    def run(depth):
        if depth:
            api.moda_attn_bwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, out, lse, dout, causal=True,
                              grads=grads, workspace=ws)
        else:
            api.moda_attn_bwd(dev["q"], dev["k_seq"], dev["v_seq"], None, None, out0, lse0, dout, causal=True,
                              grads=grads0, workspace=ws)

    run(True)
    run(False)
    t = {True: [], False: []}
    for _ in range(iters):
        for depth in (True, False):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(depth)
            e1.record(stream)
            torch.cuda.synchronize()
            t[depth].append(e0.elapsed_time(e1))
    ms, ms0 = float(np.median(t[True])), float(np.median(t[False]))
    F, F0 = acc.bwd_flops(shape), acc.bwd_flops(shape0)
    tf = F / (ms * 1e-3) / 1e12
    del dout, ws, grads, grads0
    return {"workload": "backward of the long-context layer B=1 T=65536 Hq=16 Hk=4 d=128 L=48 causal "
                        "(dq, dk, dv, depth dk, dv from the saved out and lse)",
            "ms": round(ms, 3), "l0_ms": round(ms0, 3), "ratio_vs_l0": round(ms / ms0, 4),
            "flops": F, "tflops": round(tf, 2), "l0_tflops": round(F0 / (ms0 * 1e-3) / 1e12, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def comparator_leg(dev, out0, iters=5):
    """Context only: PyTorch's own flash-attention SDPA backend (restricted to that backend, so
    it raises rather than fall back to another path) on the L=0 shape of the long-context
    layer, with the same q / k_seq / v_seq, against this library's L=0 forward."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    shape0 = I.workload(5, 1)
    q = dev["q"].transpose(1, 2).contiguous()  # [B,Hq,T,d]
    k = dev["k_seq"].transpose(1, 2).contiguous()
    v = dev["v_seq"].transpose(1, 2).contiguous()
    stream = torch.cuda.current_stream()
    res = {"workload": "causal GQA attention B=1 T=65536 Hq=16 Hk=4 d=128 (the L=0 shape)",
           "impl": "torch.nn.functional.scaled_dot_product_attention, FLASH_ATTENTION backend, enable_gqa"}
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            def run():
                return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
            o = run()
            torch.cuda.synchronize()
            ts = []
            for _ in range(iters):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
    except RuntimeError as ex:  # the backend does not take this shape on this build
        res["error"] = str(ex).splitlines()[0][:200]
        return res
    ms = float(np.median(ts))
    res.update({"ms": round(ms, 3), "tflops": round(acc.flops(shape0) / (ms * 1e-3) / 1e12, 1),
                "max_abs_diff_vs_moda_l0_out": float((o.transpose(1, 2).float() - out0.float()).abs().max()),
                "note": "median of %d HIP-event-timed calls; context, not a target" % iters})
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


KVPROJ_SHAPE = dict(B=1, T=65536, Dm=2048, Hk=4, d=128)


def depth_write_leg(kd, vd, iters=10):
    """The depth write path at the long-context layer: the KV projection of 65536 hidden states
    (Dm = Hq*d = 2048) into the layer's sequence K/V and the last slot of the step's packed depth
    buffers, one fused launch, timed with HIP events after warm-up."""
    s = KVPROJ_SHAPE
    B, T, Dm, Hk, d = s["B"], s["T"], s["Dm"], s["Hk"], s["d"]
    g = torch.Generator(device="cuda").manual_seed(13)
    x = torch.randn(B, T, Dm, device="cuda", generator=g).bfloat16()
    w = (torch.randn(2 * Hk * d, Dm, device="cuda", generator=g) / 8).bfloat16()
    k = torch.empty(B, T, Hk, d, dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    slot = kd.shape[3] - 1

    def run():
        api.moda_kv_project(x, w, Hk, d, k_out=k, v_out=v, k_depth=kd, v_depth=vd, slot=slot)

    run()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    F = acc.kv_project_flops(B, T, Dm, Hk, d)
    tf = F / (ms * 1e-3) / 1e12
    del x, w, k, v
    return {"workload": "depth write: KV projection of B=1 T=65536 hidden states (Dm=2048) into the sequence "
                        "K/V and slot %d of the packed depth stream (Hk=4 d=128), one launch" % slot,
            "ms": round(ms, 4), "flops": F, "bytes": acc.kv_project_bytes(B, T, Dm, Hk, d),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def workloads_leg(iters=8):
    """Forward timings at the other benchmark workloads of the pages' kernel study: the
    700M-class layer, the depth sweep (L = 0, 12, 48, 96) and the GQA group sweep (G = 1..8,
    keys x 0.5).  Each L > 0 shape is timed against an L=0 forward on the same q / k_seq /
    v_seq (calls interleaved, median of HIP-event times after one warm-up call each); inputs
    are drawn on the GPU from each workload's seeds, depth packed once before timing.  The
    depth sweep also gives the marginal depth-stream rate: the slope of time against depth
    bytes over its four points."""
    stream = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    rows = []
    sweep = []  # (depth bytes, ms) of the depth sweep
    cases = [(2, 0)] + [(3, v) for v in range(4)] + [(4, v) for v in range(4)]
    for c, v in cases:
        shape = I.workload(c, v)
        dev = I.workload_inputs(c, v, device="cuda")
        kd = api.moda_pack_depth(dev.pop("k_depth")) if shape.L else None
        vd = api.moda_pack_depth(dev.pop("v_depth")) if shape.L else None
        dev.pop("k_depth", None), dev.pop("v_depth", None)
        out = torch.empty_like(dev["q"])
        lse = torch.empty((shape.B, shape.Hq, shape.T), dtype=torch.float32, device="cuda")
        out0, lse0 = torch.empty_like(out), torch.empty_like(lse)

        def run():
            api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, causal=True, out=out, lse=lse)

        def run0():
            api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], None, None, causal=True, out=out0, lse=lse0)

        run(), run0()
        t, t0 = [], []
        for _ in range(iters):
            t.append(timed(run))
            t0.append(timed(run0))
        ms, ms0 = float(np.median(t)), float(np.median(t0))
        F = acc.flops(shape)
        Fseq = acc.flops_seq(shape.B, shape.T, shape.Hq, shape.d)
        row = {"workload": c, "shape": shape.describe(), "ms": round(ms, 4), "l0_ms": round(ms0, 4),
               "ratio_vs_l0": round(ms / ms0, 4), "tflops": round(F / (ms * 1e-3) / 1e12, 1),
               "seq_mfma_util": round(Fseq / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "depth_gb": round(acc.depth_bytes(shape) / 1e9, 3)}
        if shape.L:
            row["depth_marginal_gbs"] = round(acc.depth_bytes(shape) / max(1e-9, (ms - ms0) * 1e-3) / 1e9, 1)
        # The L=0 call's q, k_seq, v_seq and out fit in the 256 MB last-level cache (MALL) for
        # the smaller shapes, so back-to-back calls find them there: those L=0 times are warm.
        l0_set = sum(dev[n].numel() * dev[n].element_size() for n in ("q", "k_seq", "v_seq")) + \
            out0.numel() * out0.element_size()
        row["l0_working_set_mb"] = round(l0_set / 2 ** 20, 1)
        row["l0_warm"] = l0_set < 256 * 2 ** 20
        rows.append(row)
        if c == 3:
            sweep.append((acc.depth_bytes(shape), ms))
        del dev, kd, vd, out, lse, out0, lse0
        torch.cuda.empty_cache()
    x = np.array([b for b, _ in sweep], dtype=np.float64)
    y = np.array([m for _, m in sweep], dtype=np.float64) * 1e-3
    slope = np.polyfit(x, y, 1)[0]  # seconds per depth byte
    return {"rows": rows,
            "depth_sweep_marginal_gbs": round(1.0 / slope / 1e9, 1) if slope > 0 else None,
            "note": "each ratio is against an L=0 forward on the same sequence inputs; depth_marginal_gbs = "
                    "depth bytes / (t - t_L0); the sweep figure is the slope of t over depth bytes, L=0..96; "
                    "l0_warm marks L=0 working sets under the 256 MB MALL (no flush between calls)"}


def table2_leg(iters=5):
    """Timings at the shape of the pages' kernel table (B=1, d=64, G=8, Hq=64, Hk=8, L=64,
    causal; T from 4096 to 65536), each against L=0 on the same sequence inputs: the
    forward alone, and forward + backward as the pages time it (their figures are Triton
    kernels on another GPU, so only the trend of the extra time with T is comparable).
    Both conventions are given: (t - t0) / t as in the pages' table and (t - t0) / t0."""
    stream = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    rows = []
    for T in (4096, 8192, 16384, 32768, 65536):
        shape = I.Shape(1, T, 64, 8, 64, 64)
        dev = I.make_inputs(shape, {n: 8000 + k for k, n in enumerate(I.TENSORS)}, device="cuda")
        kd = api.moda_pack_depth(dev.pop("k_depth"))
        vd = api.moda_pack_depth(dev.pop("v_depth"))
        out = torch.empty_like(dev["q"])
        lse = torch.empty((1, shape.Hq, T), dtype=torch.float32, device="cuda")

        def run():
            api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, causal=True, out=out, lse=lse)

        def run0():
            api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], None, None, causal=True, out=out, lse=lse)

        dout = I.random_dout(shape, 8100, device="cuda")
        grads = (torch.empty_like(dev["q"]), torch.empty_like(dev["k_seq"]), torch.empty_like(dev["v_seq"]),
                 torch.empty_like(kd), torch.empty_like(vd))
        ws = torch.empty(api.moda_attn_bwd_workspace(1, T, 64, 8, 64, 64), dtype=torch.uint8, device="cuda")

        def run_fb():
            run()
            api.moda_attn_bwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, out, lse, dout, causal=True,
                              grads=grads, workspace=ws)

        def run0_fb():
            run0()
            api.moda_attn_bwd(dev["q"], dev["k_seq"], dev["v_seq"], None, None, out, lse, dout, causal=True,
                              grads=grads[:3] + (None, None), workspace=ws)

        run(), run0(), run_fb(), run0_fb()
        t, t0, tb, tb0 = [], [], [], []
        for _ in range(iters):
            t.append(timed(run))
            t0.append(timed(run0))
            tb.append(timed(run_fb))
            tb0.append(timed(run0_fb))
        ms, ms0 = float(np.median(t)), float(np.median(t0))
        fb, fb0 = float(np.median(tb)), float(np.median(tb0))
        rows.append({"T": T, "ms": round(ms, 4), "l0_ms": round(ms0, 4),
                     "extra_over_t": round((ms - ms0) / ms, 4), "extra_over_t0": round((ms - ms0) / ms0, 4),
                     "time_ratio_l0_over_moda": round(ms0 / ms, 4),
                     "tflops": round(acc.flops(shape) / (ms * 1e-3) / 1e12, 1),
                     "fwd_bwd_ms": round(fb, 4), "fwd_bwd_l0_ms": round(fb0, 4),
                     "fwd_bwd_extra_over_t": round((fb - fb0) / fb, 4)})
        del dev, kd, vd, out, lse, dout, grads, ws
        torch.cuda.empty_cache()
    return {"workload": "forward, and forward + backward, at the pages' kernel-table shape B=1 d=64 G=8 Hq=64 "
                        "Hk=8 L=64 causal, T=4096..65536, each against L=0 on the same inputs", "rows": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-peaks", action="store_true", help="skip the attainable-peak measurement kernels")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-depth-write", action="store_true", help="skip the depth-write (KV projection) measurement")
    ap.add_argument("--no-comparator", action="store_true",
                    help="skip the context timing of PyTorch's flash-attention SDPA at the L=0 shape")
    ap.add_argument("--table2", action="store_true",
                    help="only time the forward at the pages' kernel-table shape over T and print that JSON line")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the forward timings at the 700M-class, depth-sweep and GQA-sweep workloads")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summary from rocprofv3 CSV output directories and exit")
    ap.add_argument("--sq", metavar="SQ_DIR", nargs="+", help="with --summarize: also summarise SQ counter passes")
    ap.add_argument("--commands", nargs="+", default=["", "", ""],
                    help="the rocprofv3 commands (trace, fetch, write[, sq...]), for the record")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize, command=args.commands, sq_dir=args.sq)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the MoDA forward has no multi-GPU path here (each (batch, KV head) "
              "unit is independent; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    _lib.ensure_built()
    torch.cuda.set_device(0)
    if args.table2:
        print(json.dumps(table2_leg()), flush=True)
        return

    shape = I.workload(5, 0)
    shape0 = I.workload(5, 1)
    dev = I.workload_inputs(5, 0, device="cuda")
    kd = torch.empty((shape.B, shape.T, shape.Hk, shape.L, shape.d), dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((shape.B, shape.Hq, shape.T), dtype=torch.float32, device="cuda")
    out0 = torch.empty_like(out)
    lse0 = torch.empty_like(lse)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        api.moda_pack_depth(dev["k_depth"], kd)
        api.moda_pack_depth(dev["v_depth"], vd)
        if ev: ev[1].record(stream)
        api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, causal=True, out=out, lse=lse)
        if ev: ev[2].record(stream)
        api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], None, None, causal=True, out=out0, lse=lse0)
        if ev: ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pack = [e[0].elapsed_time(e[1]) for e in events]
    t_fwd = [e[1].elapsed_time(e[2]) for e in events]
    t_fwd0 = [e[2].elapsed_time(e[3]) for e in events]
    pack_ms, fwd_ms, fwd0_ms = (float(np.mean(t)) for t in (t_pack, t_fwd, t_fwd0))

    def spread(t):
        return {"mean": round(float(np.mean(t)), 4), "median": round(float(np.median(t)), 4),
                "min": round(float(np.min(t)), 4), "max": round(float(np.max(t)), 4), "n": len(t)}

    F = acc.flops(shape)
    F0 = acc.flops(shape0)
    Fseq = acc.flops_seq(shape.B, shape.T, shape.Hq, shape.d)
    tflops = F / (fwd_ms * 1e-3) / 1e12
    tflops0 = F0 / (fwd0_ms * 1e-3) / 1e12
    trec = traffic_record()
    traffic = trec.get("hbm_bytes_per_launch") if trec else None
    rec = {
        "metric": "MoDA fwd TFLOP/s + time ratio vs L=0 causal attn, bf16, T=64K, 1 MI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long-context layer B=1 T=65536 Hq=16 Hk=4 G=4 d=128 L=48 causal, "
                               "denominator L=0", "B": shape.B, "T": shape.T, "Hq": shape.Hq, "Hk": shape.Hk,
                   "d": shape.d, "L": shape.L, "causal": True,
                   "step": "pack depth K,V + MoDA fwd (L=48) + causal fwd (L=0)"},
        "fwd_ms": round(fwd_ms, 4),
        "fwd_l0_ms": round(fwd0_ms, 4),
        "pack_kv_ms": round(pack_ms, 4),
        "ratio_vs_l0": round(fwd_ms / fwd0_ms, 4),
        "ratio_vs_l0_median": round(float(np.median(t_fwd)) / float(np.median(t_fwd0)), 4),
        "timing_ms": {"fwd_L48": spread(t_fwd), "fwd_L0": spread(t_fwd0), "pack_kv": spread(t_pack),
                      "note": "HIP-event time of each launch over the K timed steps; value, roofline and "
                              "ratio_vs_l0 use the mean (the profile's average), ratio_vs_l0_median the medians"},
        "l0_tflops": round(tflops0, 2),
        "seq_mfma_util": round(Fseq / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "depth_marginal_gbs": round(acc.depth_bytes(shape) / max(1e-9, (fwd_ms - fwd0_ms) * 1e-3) / 1e9, 1),
        "depth_hbm_gbs_counters": (round((trec["read_bytes_per_launch"] - trec["l0_read_bytes_per_launch"])
                                         / (fwd_ms * 1e-3) / 1e9, 1)
                                   if trec and "l0_read_bytes_per_launch" in trec else None),
        "pack_gbs": round(2 * acc.depth_bytes(shape) / (pack_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    if not args.no_peaks:
        rec["measured_peaks"] = peaks_leg()
        rec["roofline"]["frac_of_measured_peak"] = round(tflops / rec["measured_peaks"]["mfma_bf16_tflops"], 4)
    if not args.no_backward:
        rec["backward"] = backward_leg(shape, dev, kd, vd, out, lse, out0, lse0)
    if not args.no_comparator:
        rec["comparator"] = comparator_leg(dev, out0)
    if not args.no_decode:
        rec["decode"] = decode_leg()
    if not args.no_depth_write:  # last: it overwrites the final depth slot of the step's buffers
        rec["depth_write"] = depth_write_leg(kd, vd)
    if not args.no_workloads:
        rec["workloads"] = workloads_leg()
    if not args.no_cpu_baseline:
        host = {k: v.cpu() for k, v in dev.items()}
        cpu, rows, ref = cpu_baseline(shape, host, args.cpu_seconds)
        b, t, h = (torch.from_numpy(rows[:, i].astype(np.int64)).cuda() for i in range(3))
        got = out[b, t, h].float().cpu().numpy()
        cpu["sample_max_abs_err_vs_gpu"] = float(np.abs(got - ref).max())
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
