"""Benchmark of the 32-bit two-state optimizer update on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Headline ("step"): one Adam update (fp32 param/grad/states) of a flat tensor
of 2^28 elements, inputs resident in HBM.  value = algorithmic bytes
(28 B/element: read p, g, m, v; write p, m, v) / time per step, in GB/s.

Also measured (same JSON line): the headline traffic's ceilings on the
headline's own buffers (its reads alone, its writes alone and the
read/write mix with no arithmetic, several launch shapes each); the other
kinds and storages at 2^28, Adam and AdEMAMix with fp32 and bf16 storage at
2^30; a plain device copy; the model-like collection (505 bf16 tensors,
AdamW) as an eager per-tensor loop, one plan launch and graph replay, its
small-tensor subsets, the page's direct cells and the launch floors; the
CPU oracle on the headline workload for a bounded number of steps.

Timing: HIP events on the stream the kernels run on, W untimed warmups, then
K timed steps between device synchronisations, with an event between steps
so that every step's time is recorded (step_samples_ms).  Secondary cases
report the median, p10/p90 and every sample of 7 rounds.  The small-tensor
subsets fit in the 256 MB Infinity Cache, which serves back-to-back steps
in part: their plan step is also timed cold (plan_cold), each sample after
a 1 GiB write that evicts them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "optimizer-update GB/s (% of HBM peak) on 256M elems; µs per mixed small-tensor step"
# the kernels and the launch selection that shapes them
KERNEL_SOURCES = ("optimizer_update_amd/csrc/kernels.hip", "optimizer_update_amd/csrc/stream.hpp",
                  "optimizer_update_amd/csrc/elem.hpp", "optimizer_update_amd/csrc/stepdiv.hpp",
                  "optimizer_update_amd/csrc/host.hip")
# the 8-bit kernels and their launch selection
KERNEL8_SOURCES = ("optimizer_update_amd/csrc/kernels8.hip", "optimizer_update_amd/csrc/qmap.hpp",
                   "optimizer_update_amd/csrc/elem.hpp", "optimizer_update_amd/csrc/stepdiv.hpp",
                   "optimizer_update_amd/csrc/host8.hip")
# VALU issue peak for the kernels as built (packed-fp32 instructions off),
# from the chip's unit counts and clock: MI355X's 157.3 TFLOP/s fp32 vector
# rate counts packed FMAs (2 per lane); unpacked, each SIMD retires 16 lanes
# per cycle, one full-rate wave64 instruction per 4 cycles (a quad-cycle):
# 256 CUs x 4 SIMDs x 2.4 GHz / 4 = 614.4 G wave64 instructions/s.  The 8-bit
# cases' ALU roofline counts the kernels' VALU work in busy quad-cycles
# (SQ_ACTIVE_INST_VALU), which weights the binary64 and transcendental
# instructions that take more than one, against this peak, and reports
# beside it what VALU-only probe kernels reach in the same run.
VALU_PEAK_G = 256 * 4 * 2.4 / 4
# Step at which the late-training cases start: far past the step where
# fl32(1 - beta^t) reaches 1 for the default betas (0.9, 0.999).
LATE_STEP = 1_000_000


def code_text(src: str) -> str:
    """C/C++/HIP source with its comments and blank lines removed and each
    line's surrounding whitespace stripped; string and character literals
    are kept whole (a "//" inside one is not a comment)."""
    out = []
    i, n = 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    lines = (ln.strip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_sha(files=KERNEL_SOURCES) -> str:
    """Hash of the code (not the comments) of the sources that shape a
    kernel: the committed counter records are keyed by it, so a record
    stays valid across comment edits and lapses with any change of code."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--case", default="adam:fp32:28",
                    help="headline case kind:storage:log2n[:clip|:late] (profiling runs; late: steps from "
                         "1,000,001, where the bias corrections are 1)")
    ap.add_argument("--collection-only", action="store_true",
                    help="only the model-like collection measurements (profiling runs)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only a plain device copy of 2^28 floats (1 GiB each way): the "
                         "known-size kernel that calibrates HBM byte counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only. The update is elementwise, so it shards with no "
              "exchange inside a step: each GPU would run the same kernels on its own slice of "
              "the parameters (grads reduce-scattered before, parameters all-gathered after). "
              "Rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import optimizer_update_amd as ou
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = ou.load()
    props = torch.cuda.get_device_properties(dev)

    def make_flat(kind, storage, n, seed):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        p = torch.empty(n, device=dev).uniform_(-1.0, 1.0, generator=gen).to(W.STORAGE_TORCH[storage])
        g = (torch.randn(n, device=dev, generator=gen) * 1e-3).to(W.STORAGE_TORCH[storage])
        if kind.endswith("8"):         # 8-bit block-wise states
            c1, c2, a1, a2 = ou.state8_sizes(kind[:-1], n)
            return (p, g, torch.zeros(c1, dtype=torch.uint8, device=dev),
                    torch.zeros(c2, dtype=torch.uint8, device=dev),
                    torch.zeros(a1, device=dev), torch.zeros(a2, device=dev))
        s1n, s2n = ou.state_sizes(kind, n)
        return (p, g, torch.zeros(s1n, device=dev),
                torch.zeros(s2n, device=dev) if s2n else None)

    hp_adam = ou.HParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    hp_mix = ou.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                        weight_decay=0.01)
    hp_kind = {"adam": hp_adam, "ademamix": hp_mix,
               "momentum": ou.HParams(lr=1e-2, beta1=0.9, beta2=0.0, eps=0.0, weight_decay=0.0),
               "rmsprop": ou.HParams(lr=1e-2, beta1=0.99, beta2=0.0, eps=1e-8, weight_decay=0.0),
               "adagrad": ou.HParams(lr=1e-2, beta1=0.0, beta2=0.0, eps=1e-10, weight_decay=0.0),
               "lion": ou.HParams(lr=1e-4, beta1=0.9, beta2=0.99, eps=0.0, weight_decay=0.1)}

    def flat_stepper(kind, tensors, hp, start=0):
        state = {"t": start}
        if kind.endswith("8"):
            def step8():
                state["t"] += 1
                ou.optimizer_update_8bit_blockwise(kind[:-1], *tensors, step=state["t"], lr=hp.lr,
                                                   beta1=hp.beta1, beta2=hp.beta2, beta3=hp.beta3,
                                                   alpha=hp.alpha, eps=hp.eps,
                                                   weight_decay=hp.weight_decay)
            return step8
        p, g, s1, s2 = tensors

        def step():
            state["t"] += 1
            ou.optimizer_update_32bit(kind, p, g, s1, s2, step=state["t"], lr=hp.lr, beta1=hp.beta1,
                                      beta2=hp.beta2, beta3=hp.beta3, alpha=hp.alpha, eps=hp.eps,
                                      weight_decay=hp.weight_decay, skip_zeros=hp.skip_zeros)
        return step

    def time_exact(step, steps, warmup):
        """W warmups, then exactly K steps between synchronisations; HIP events
        on the current stream (where the library launches), one before every
        step and one after the last, so every step's time is recorded as
        well as the total."""
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return ev[0].elapsed_time(ev[-1]) / steps, wall / steps * 1e3, per_step

    def time_rounds(step, iters, rounds=7, warmup=20):
        """Median, p10, p90 of per-step ms over `rounds` samples of `iters` steps."""
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        samples = []
        for _ in range(rounds):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                step()
            e1.record()
            torch.cuda.synchronize()
            samples.append(e0.elapsed_time(e1) / iters)
        srt = sorted(samples)
        q = lambda f: srt[min(len(srt) - 1, int(round(f * (len(srt) - 1))))]
        return {"median_ms": statistics.median(srt), "p10_ms": q(0.1), "p90_ms": q(0.9),
                "samples_ms": [round(x, 5) for x in samples]}

    if args.copy_only:
        src = torch.empty(1 << 28, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": 4 << 28, "launches": args.steps}))
        return

    if args.collection_only:
        print(json.dumps(bench_collection(torch, ou, W, dev, time_rounds)))
        return

    valu8 = None   # committed VALU counts of the 8-bit kernel (per 256-element block)
    vf = os.path.join(ROOT, "profiles", "valu_k8_single_256M.json")
    if os.path.exists(vf):
        with open(vf) as f:
            v = json.load(f)
        if v.get("kernel8_sources_sha") == kernel_sha(KERNEL8_SOURCES):
            valu8 = v
    valu_peak = None if args.quick else valu_issue_rate(torch, ou, dev, time_rounds)

    def alu_roofline(case_key, n, ms, valu_peak):
        """VALU work of an 8-bit case (committed SQ_ACTIVE_INST_VALU per block,
        in quad-cycles) per second, against the issue peak from the chip's
        unit counts and clock (614.4 G/s); beside it the rate the VALU-only
        probes reached in this run (the clock under load sits below 2.4 GHz)."""
        if not valu8 or case_key not in valu8.get("valu_quad_cycles_per_block", {}):
            return None
        blocks = n // 256
        cycles = valu8["valu_quad_cycles_per_block"][case_key] * blocks / (ms * 1e-3) / 1e9
        instrs = valu8["valu_wave_instructions_per_block"][case_key] * blocks / (ms * 1e-3) / 1e9
        r = {"bound": "alu", "achieved": round(cycles, 1), "peak": VALU_PEAK_G,
             "unit": "G VALU quad-cycles/s", "frac": round(cycles / VALU_PEAK_G, 4),
             "wave_instructions_G_per_s": round(instrs, 1)}
        if valu_peak:
            r["measured_issue_G_per_s"] = valu_peak["G_per_s"]
            r["frac_of_measured"] = round(cycles / valu_peak["G_per_s"], 4)
        return r

    # ---------------------------------------------------------------- headline
    parts = args.case.split(":")
    kind, storage, log2n = parts[:3]
    clip = len(parts) > 3 and parts[3] == "clip"
    late = len(parts) > 3 and parts[3] == "late"   # steps from LATE_STEP (bias corrections of 1)
    n = 1 << int(log2n)
    bpe = (W.bytes_per_element_8bit(kind[:-1], storage) if kind.endswith("8")
           else W.bytes_per_element(kind, storage))
    hp_head = hp_kind[kind.rstrip("8")]
    head = make_flat(kind, storage, n, seed=0)
    stepper = flat_stepper(kind, head, hp_head, start=LATE_STEP if late else 0)
    if clip:   # update-norm clipping (profiling runs): three launches, 40 B/element
        ws = ou.clip_workspace(n, dev)
        cst = {"t": 0}

        def stepper():
            cst["t"] += 1
            ou.optimizer_update_32bit_clip(kind, *head, step=cst["t"], lr=hp_head.lr,
                                           beta1=hp_head.beta1, beta2=hp_head.beta2,
                                           beta3=hp_head.beta3, alpha=hp_head.alpha,
                                           eps=hp_head.eps, weight_decay=hp_head.weight_decay,
                                           max_unorm=1e-3, workspace=ws)
        bpe = 40 if (kind, storage) == ("adam", "fp32") else bpe
    ms, wall_ms, step_ms = time_exact(stepper, args.steps, args.warmup)
    gbs = bpe * n / (ms * 1e-3) / 1e9

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{kind}_{storage}_flat_2^{log2n}" + ("_max_unorm" if clip else "")
                   + ("_late" if late else ""),
                   "n": n, "kind": kind,
                   "param_grad_storage": storage,
                   "states": "8-bit block-wise, 256 per block" if kind.endswith("8") else "fp32",
                   "params": "U(-1,1)", "grads": "N(0, (1e-3)^2), fixed",
                   "hparams": {k: v for k, v in hp_head.__dict__.items()},
                   "bytes_per_element": bpe, "device": props.name, "cu_count": props.multi_processor_count,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "host_wall_ms_per_step": round(wall_ms, 4),
        "step_samples_ms": [round(x, 5) for x in step_ms],
        "kernel_sources_sha": kernel_sha(),
        "env": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                "device": props.name, "arch": getattr(props, "gcnArchName", None),
                "cu_count": props.multi_processor_count,
                "hbm_bytes": props.total_memory, "l2_bytes": getattr(props, "L2_cache_size", None),
                "kernel_sources_sha": kernel_sha(), "kernel8_sources_sha": kernel_sha(KERNEL8_SOURCES),
                "binding": ("_fast" if isinstance(ou.load().optimizer_update_32bit, type(len)) else "ctypes")},
    }
    if kind.endswith("8") and not clip:
        alu = alu_roofline(f"{kind[:-1]}_{storage}", n, ms, valu_peak)
        if alu:   # the 8-bit kernel is bound by VALU issue, not by HBM
            out["roofline_hbm"] = out["roofline"]
            out["roofline"] = {**alu, "traffic": None}
    probe = None
    if not args.quick and args.case == "adam:fp32:28":
        probe = bandwidth_ceilings(torch, ou, head, n, time_rounds)
        out["roofline"]["stream_probe_GBps"] = probe["mix_4r3w"]["GBps"]
        out["roofline"]["frac_of_stream_probe"] = round(gbs / probe["mix_4r3w"]["GBps"], 4)
        out["roofline"]["read_only_GBps"] = probe["read_4"]["GBps"]
        out["roofline"]["write_only_GBps"] = probe["write_3"]["GBps"]
        out["roofline"]["serial_bound_GBps"] = probe["serial_bound_GBps"]
        out["roofline"]["frac_of_serial_bound"] = round(gbs / probe["serial_bound_GBps"], 4)
    tr = os.path.join(ROOT, "profiles", "traffic_single_adam_fp32_256M.json")
    if os.path.exists(tr) and args.case == "adam:fp32:28":
        with open(tr) as f:
            t = json.load(f)
        if t.get("kernel_sources_sha") == out["kernel_sources_sha"]:
            out["roofline"]["traffic"] = t["hbm_bytes_per_launch"]
    del head
    torch.cuda.empty_cache()

    if not args.quick:
        cases = {}
        # achievable bandwidth reference: device copy of 2^28 floats
        src = torch.empty(1 << 28, device=dev).uniform_()
        dst = torch.empty_like(src)
        r = time_rounds(lambda: dst.copy_(src), iters=20)
        cases["copy_fp32_2^28"] = {**r, "GBps": round(2 * 4 * (1 << 28) / (r["median_ms"] * 1e-3) / 1e9, 1)}
        if probe:
            cases["bandwidth_ceilings_fp32_2^28"] = probe
        if valu_peak:
            cases["valu_issue_probe"] = valu_peak
        del src, dst
        torch.cuda.empty_cache()
        for ck, cs, cl in (("adam", "bf16", 28), ("ademamix", "fp32", 28), ("ademamix", "bf16", 28),
                           ("adam", "fp32", 30), ("adam", "bf16", 30), ("ademamix", "fp32", 30),
                           ("ademamix", "bf16", 30),
                           ("lion", "fp32", 28), ("momentum", "bf16", 28),
                           ("adam8", "fp32", 28), ("adam8", "bf16", 28), ("ademamix8", "bf16", 28)):
            cn = 1 << cl
            hp = hp_kind[ck.rstrip("8")]
            ts = make_flat(ck, cs, cn, seed=cl)
            r = time_rounds(flat_stepper(ck, ts, hp), iters=10 if cl == 28 else 4)
            b = (W.bytes_per_element_8bit(ck[:-1], cs) if ck.endswith("8")
                 else W.bytes_per_element(ck, cs))
            gb = b * cn / (r["median_ms"] * 1e-3) / 1e9
            cases[f"{ck}_{cs}_2^{cl}"] = {**r, "GBps": round(gb, 1), "frac_of_peak": round(gb / HBM_PEAK_GBS, 4),
                                          "elements_per_s": round(cn / (r["median_ms"] * 1e-3), 0),
                                          "bytes_per_element": b}
            del ts
            torch.cuda.empty_cache()
        # the VALU probes again, right after the VALU-bound 8-bit cases; their
        # roofline takes the faster of the two measurements
        if valu_peak:
            again = valu_issue_rate(torch, ou, dev, time_rounds)
            cases["valu_issue_probe_after_8bit"] = again
            if again["G_per_s"] > valu_peak["G_per_s"]:
                valu_peak = again
        for ck, cs in (("adam8", "fp32"), ("adam8", "bf16"), ("ademamix8", "bf16")):
            c = cases[f"{ck}_{cs}_2^28"]
            c["alu_roofline"] = alu_roofline(f"{ck[:-1]}_{cs}", 1 << 28, c["median_ms"], valu_peak)
        # the 8-bit cases above run steps 1-90, where both bias corrections
        # differ from 1; late in training (from step 17,318 for beta2 = 0.999)
        # both are exactly 1 and the kernels leave the divisions out
        for ck, cs in (("adam8", "bf16"), ("ademamix8", "bf16")):
            cn = 1 << 28
            hp = hp_kind[ck.rstrip("8")]
            ts = make_flat(ck, cs, cn, seed=28)
            r = time_rounds(flat_stepper(ck, ts, hp, start=LATE_STEP), iters=10)
            b = W.bytes_per_element_8bit(ck[:-1], cs)
            gb = b * cn / (r["median_ms"] * 1e-3) / 1e9
            cases[f"{ck}_{cs}_2^28_late"] = {
                **r, "from_step": LATE_STEP + 1, "GBps": round(gb, 1), "frac_of_peak": round(gb / HBM_PEAK_GBS, 4),
                "bytes_per_element": b,
                "alu_roofline": alu_roofline(f"{ck[:-1]}_{cs}_late", cn, r["median_ms"], valu_peak)}
            del ts
            torch.cuda.empty_cache()
        # update-norm clipping: three launches, 40 B/element for fp32 Adam
        # (pass 1 reads p, g, m, v and writes m, v; pass 3 reads p, m, v and writes p)
        cn = 1 << 28
        ts = make_flat("adam", "fp32", cn, seed=28)
        ws = ou.clip_workspace(cn, dev)
        cstate = {"t": 0}

        def clip_step():
            cstate["t"] += 1
            ou.optimizer_update_32bit_clip("adam", *ts, step=cstate["t"], lr=1e-3, max_unorm=1e-3,
                                           workspace=ws)
        r = time_rounds(clip_step, iters=10)
        gb = 40 * cn / (r["median_ms"] * 1e-3) / 1e9
        cases["adam_fp32_2^28_max_unorm"] = {**r, "GBps": round(gb, 1), "frac_of_peak": round(gb / HBM_PEAK_GBS, 4),
                                             "bytes_per_element": 40, "clip_factor": ou.clip_scale(ws)}
        del ts, ws
        torch.cuda.empty_cache()
        cases["adam_fp32_2^28"] = {"median_ms": out["ms_per_step"], "GBps": out["value"],
                                   "frac_of_peak": out["roofline"]["frac"]} if args.case == "adam:fp32:28" else None
        copy_gbs = cases["copy_fp32_2^28"]["GBps"]
        out["roofline"]["frac_of_copy"] = round(gbs / copy_gbs, 4)
        out["cases"] = cases
        out["small_step_us"] = bench_collection(torch, ou, W, dev, time_rounds)
        if not args.no_cpu:
            out["cpu_baseline"] = cpu_baseline(torch, W, dev)
    print(json.dumps(out))


def valu_issue_rate(torch, ou, dev, time_rounds):
    """The device's VALU issue rate, measured: the probe kernel runs 64
    full-rate binary32 operations per round on registers, 2,048 rounds per
    lane, 8 blocks of 4 waves per CU (every SIMD full), and nothing else;
    once with fused multiply-adds and once with additions, which draw less
    power (the clock under load depends on it).  The faster of the two is
    the rate."""
    lib = ou._lib.load()
    out = torch.zeros(1, device=dev)
    blocks = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    rounds = 2048
    instr = blocks * 4 * rounds * 64
    sh = torch.cuda.current_stream().cuda_stream
    by_op = {}
    for op, name in ((0, "v_fmac_f32"), (1, "v_add_f32")):
        def run(op=op):
            st = lib.ou__valu_probe(op, blocks, rounds, out.data_ptr(), sh)
            if st != 0:
                raise RuntimeError(lib.ou_last_error().decode())
        r = time_rounds(run, iters=5, rounds=7, warmup=3)
        by_op[name] = {"G_per_s": round(instr / (r["median_ms"] * 1e-3) / 1e9, 1),
                       "median_ms": round(r["median_ms"], 4)}
    best = max(by_op, key=lambda k: by_op[k]["G_per_s"])
    return {"G_per_s": by_op[best]["G_per_s"], "best_op": best, "by_op": by_op, "wave_instructions": instr,
            "blocks": blocks,
            "what": "64 independent full-rate binary32 operations per round per lane (8 chains), 2,048 rounds, "
                    "4-wave blocks, 8 per CU"}


# LDS per CU of gfx950 (160 KiB): a kernel with no LDS of its own that
# reserves lds_for(b) bytes of dynamic LDS runs at most b blocks per CU.
LDS_PER_CU = 160 * 1024


def lds_for(blocks_per_cu: int) -> int:
    if blocks_per_cu <= 0:
        return -1                      # no cap (the library's "off" value)
    return (LDS_PER_CU // (blocks_per_cu + 1) + 1024) & ~1023


def bandwidth_ceilings(torch, ou, head, n, time_rounds):
    """What the headline's traffic reaches with no arithmetic, on the
    headline's own buffers in the same run: its four reads alone, its three
    writes alone and the 4-read/3-write mix, each in several launch shapes
    (threads per block x groups per lane, resident blocks per CU, tiles per
    XCD run); the best shape of each is reported.  The serial bound is the
    rate if the reads ran at the read-only rate and then the writes at the
    write-only rate: 28 / (16 / R + 12 / W) B per element."""
    lib = ou._lib.load()
    sh = torch.cuda.current_stream().cuda_stream
    ptrs = [t.data_ptr() for t in head]
    nvec = n // 4
    shapes = {"64x2 8/CU run64": (64, 2, 8, 64), "64x2 8/CU run128": (64, 2, 8, 128),
              "128x2 4/CU run64": (128, 2, 4, 64), "256x2 2/CU run16": (256, 2, 2, 16),
              "128x4 2/CU run32": (128, 4, 2, 32), "256x2 full run16": (256, 2, 0, 16),
              "512x2 full run16": (512, 2, 0, 16), "256x4 full block order": (256, 4, 0, -1)}
    modes = (("read_4", 1, 16), ("mix_4r3w", 0, 28), ("write_3", 2, 12))   # writes last: they clobber
    res = {}
    try:
        for name, mode, bpe in modes:
            by = {}
            for sname, (blk, unr, per_cu, run) in shapes.items():
                lib.ou__force_single(blk, 4, unr, nvec // (blk * unr), 0, lds_for(per_cu))
                lib.ou__force_xcd(run)

                def step(mode=mode):
                    st = lib.ou__stream_probe(mode, *ptrs, n, sh)
                    if st != 0:
                        raise RuntimeError(lib.ou_last_error().decode())
                r = time_rounds(step, iters=10, rounds=5, warmup=5)
                by[sname] = round(bpe * n / (r["median_ms"] * 1e-3) / 1e9, 1)
            best = max(by, key=by.get)
            res[name] = {"GBps": by[best], "best_shape": best, "GBps_by_shape": by,
                         "bytes_per_element": bpe}
    finally:
        lib.ou__force_single(0, 0, 0, 0, 0, 0)
        lib.ou__force_xcd(0)
    r, w = res["read_4"]["GBps"], res["write_3"]["GBps"]
    res["serial_bound_GBps"] = round(28 / (16 / r + 12 / w), 1)
    res["what"] = ("fp32 streams of 2^28 elements: read_4 reads p, g, m, v; write_3 writes p, m, v; "
                   "mix_4r3w reads four and writes three back; no arithmetic")
    return res


def time_cold(torch, step, flush, samples=50, warmup=3):
    """Per-step ms of `step` run cold: before each sample a write over
    `flush` (1 GiB, four times what MI355X's 256 MB Infinity Cache holds)
    evicts the step's tensors, as the forward and backward passes of a
    training step would; two events bracket the step alone.  Median, p10,
    p90 and every sample."""
    for _ in range(warmup):
        step()
    out = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for _ in range(samples):
        flush.zero_()
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    srt = sorted(out)
    q = lambda f: srt[min(len(srt) - 1, int(round(f * (len(srt) - 1))))]
    return {"median_ms": statistics.median(srt), "p10_ms": q(0.1), "p90_ms": q(0.9),
            "samples_ms": [round(x, 5) for x in out]}


def _us(r: dict) -> dict:
    """A time_rounds result in microseconds: median, p10, p90 and every sample."""
    return {"median_us": round(r["median_ms"] * 1e3, 2), "p10_us": round(r["p10_ms"] * 1e3, 2),
            "p90_us": round(r["p90_ms"] * 1e3, 2),
            "samples_us": [round(x * 1e3, 2) for x in r["samples_ms"]]}


def bench_collection(torch, ou, W, dev, time_rounds):
    """Model-like collection (bf16 AdamW): full step, the subsets of tensors
    of <= 16,384 and <= 4,096 elements, each as per-tensor loop, one plan
    launch, graph replay; the same collection as AdamW8bit (min_8bit_size
    4,096) and AdEMAMix32; the page's direct cells; launch floors (a
    one-element update through the binding, a bare one-element kernel, a
    one-node graph replay)."""
    res = {}
    shapes = W.model_collection()
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)

    def mk(subset):
        ps, gs = [], []
        for name, shp in subset:
            m = W.numel(shp)
            ps.append(torch.empty(m, device=dev).uniform_(-1, 1, generator=gen).to(torch.bfloat16))
            gs.append((torch.randn(m, device=dev, generator=gen) * 0.01).to(torch.bfloat16))
        return ou.AdamW32(ps, lr=1e-3, weight_decay=0.01, grads=gs)

    for label, subset in (("full_505", shapes), ("small_408", [s for s in shapes if W.numel(s[1]) <= 16384]),
                          ("le4096_216", [s for s in shapes if W.numel(s[1]) <= 4096])):
        opt = mk(subset)
        elems = sum(W.numel(s[1]) for s in subset)
        bytes_ = elems * W.bytes_per_element("adam", "bf16")
        d = {"tensors": len(subset), "elements": elems, "roofline_us": round(bytes_ / HBM_PEAK_GBS / 1e3, 2)}
        for mode, fn in (("per_tensor_loop", opt.step_per_tensor), ("plan", lambda: opt.step()),
                         ("graph", lambda: opt.step(graph=True))):
            iters = 5 if mode == "per_tensor_loop" else 50
            r = time_rounds(fn, iters=iters, rounds=7, warmup=5)
            d[mode] = _us(r)
        d["plan_GBps"] = round(bytes_ / (d["plan"]["median_us"] * 1e-6) / 1e9, 1)
        if bytes_ < (1 << 30):
            # back-to-back steps over tensors this small are served partly by the
            # Infinity Cache; the same step after a 1 GiB write is the cold figure
            flush = torch.empty(1 << 28, device=dev)
            d["plan_cold"] = _us(time_cold(torch, lambda: opt.step(), flush))
            del flush
        d["plan_describe"] = opt.plan.describe()
        if label == "full_505":
            # update-norm clipping per tensor over the same collection: pass 1
            # reads p, g, m, v and writes m, v (20 B/element in bf16), pass 3
            # reads p, m, v and writes p (12 B/element)
            copt = ou.AdamW32(opt.params, lr=1e-3, weight_decay=0.01, grads=opt.grads, max_unorm=1e-3)
            r = time_rounds(lambda: copt.step(), iters=20, rounds=7, warmup=5)
            d["plan_max_unorm"] = _us(r)
            d["plan_max_unorm_GBps"] = round(32 * elems / (r["median_ms"] * 1e-3) / 1e9, 1)
            copt.close()
        res[label] = d
        opt.close()
        torch.cuda.empty_cache()
    # the page's AdamW8bit collection: tensors of >= 4,096 elements keep 8-bit
    # block-wise states, smaller ones fp32 states (min_8bit_size = 4,096)
    ps, gs = [], []
    for name, shp in shapes:
        m = W.numel(shp)
        ps.append(torch.empty(m, device=dev).uniform_(-1, 1, generator=gen).to(torch.bfloat16))
        gs.append((torch.randn(m, device=dev, generator=gen) * 0.01).to(torch.bfloat16))
    opt = ou.AdamW8bit(ps, lr=1e-3, weight_decay=0.01, grads=gs, min_8bit_size=4096)
    big = [W.numel(s[1]) for s in shapes if W.numel(s[1]) >= 4096]
    small = [W.numel(s[1]) for s in shapes if W.numel(s[1]) < 4096]
    bytes8 = (sum(big) * W.bytes_per_element_8bit("adam", "bf16")
              + sum(small) * W.bytes_per_element("adam", "bf16"))
    d = {"tensors": len(shapes), "tensors_8bit": len(big), "tensors_32bit": len(small),
         "elements": sum(big) + sum(small), "roofline_us": round(bytes8 / HBM_PEAK_GBS / 1e3, 2)}
    for mode, fn in (("per_tensor_loop", opt.step_per_tensor), ("plans", lambda: opt.step()),
                     ("graph", lambda: opt.step(graph=True))):
        iters = 5 if mode == "per_tensor_loop" else 50
        r = time_rounds(fn, iters=iters, rounds=7, warmup=5)
        d[mode] = _us(r)
    d["plans_GBps"] = round(bytes8 / (d["plans"]["median_us"] * 1e-6) / 1e9, 1)
    # the plans' rounds above run steps 41-395 (m's bias correction reaches 1
    # at step 165); late in training both corrections are 1
    opt.step_count = LATE_STEP
    d["plans_late"] = _us(time_rounds(lambda: opt.step(), iters=50, rounds=7, warmup=5))
    d["plans_late_GBps"] = round(bytes8 / (d["plans_late"]["median_us"] * 1e-6) / 1e9, 1)
    res["adamw8bit_505"] = d
    opt.close()
    # the page's AdEMAMix32bit collection: fp32 states for every tensor
    opt = ou.AdEMAMix32(ps, lr=1e-3, weight_decay=0.01, grads=gs)
    bytes_m = sum(big + small) * W.bytes_per_element("ademamix", "bf16")
    d = {"tensors": len(shapes), "elements": sum(big) + sum(small),
         "roofline_us": round(bytes_m / HBM_PEAK_GBS / 1e3, 2)}
    for mode, fn in (("per_tensor_loop", opt.step_per_tensor), ("plan", lambda: opt.step())):
        iters = 5 if mode == "per_tensor_loop" else 30
        r = time_rounds(fn, iters=iters, rounds=7, warmup=5)
        d[mode] = _us(r)
    d["plan_GBps"] = round(bytes_m / (d["plan"]["median_us"] * 1e-6) / 1e9, 1)
    res["ademamix32_505"] = d
    opt.close()
    del ps, gs
    torch.cuda.empty_cache()
    # the page's direct cells: one preallocated tensor per (kind, storage, n),
    # one optimizer_update_32bit call per step through the C ABI (ctypes)
    lib = ou.load()
    stream = torch.cuda.current_stream().cuda_stream
    cells = {}
    for kind, code in (("adam", 0), ("ademamix", 1)):
        for storage, dt in (("fp32", 0), ("fp16", 1), ("bf16", 2)):
            for n in W.DIRECT_N:
                p = torch.zeros(n, dtype=W.STORAGE_TORCH[storage], device=dev)
                g = torch.full((n,), 1e-3, dtype=W.STORAGE_TORCH[storage], device=dev)
                s1 = torch.zeros((2 if kind == "ademamix" else 1) * n, device=dev)
                s2 = torch.zeros(n, device=dev)
                args = (code, dt, p.data_ptr(), g.data_ptr(), s1.data_ptr(), s2.data_ptr(), n,
                        0.9, 0.999, 0.9999, 5.0, 1e-8, 0.01)
                assert lib.optimizer_update_32bit(*args, 1, 1e-3, 0, stream) == 0, \
                    lib.ou_last_error().decode()
                st = {"t": 1}

                def call():
                    st["t"] += 1
                    lib.optimizer_update_32bit(*args, st["t"], 1e-3, 0, stream)
                r = time_rounds(call, iters=100, rounds=7, warmup=20)
                cells[f"{kind}_{storage}_{n}"] = _us(r)
    res["direct_cells_us"] = cells
    # launch floor: a 1-element update through the C ABI, back to back
    one = [torch.zeros(1, device=dev) for _ in range(4)]
    t = {"i": 0}

    def tiny():
        t["i"] += 1
        ou.optimizer_update_32bit("adam", one[0], one[1], one[2], one[3], step=t["i"], lr=1e-3)
    r = time_rounds(tiny, iters=200, rounds=7, warmup=50)
    res["launch_floor_1_element_us"] = _us(r)
    # the floors under it: a one-element kernel launched straight through
    # ctypes (the library's test hook that rounds one value to bf16), and the
    # replay of a one-node graph (a plan over one one-element tensor)
    one_in = torch.zeros(1, device=dev)
    one_out = torch.zeros(1, dtype=torch.int16, device=dev)

    def empty_launch():
        lib.ou__narrow(2, one_in.data_ptr(), one_out.data_ptr(), 1, stream)
    r = time_rounds(empty_launch, iters=200, rounds=7, warmup=50)
    res["launch_floor_bare_kernel_us"] = _us(r)
    plan1 = ou.Plan("adam", [tuple(one)])
    hp1 = ou.HParams(lr=1e-3)
    t1 = {"i": 0}

    def graph1():
        t1["i"] += 1
        plan1.graph_step(hp1, t1["i"])
    r = time_rounds(graph1, iters=100, rounds=7, warmup=20)
    res["graph_floor_1_node_us"] = _us(r)
    plan1.close()
    return res


def cpu_baseline(torch, W, dev):
    """The CPU oracle on bounded samples: the headline workload's 2^28-element
    fp32 Adam inputs (same generator and seed), 10 steps on all host cores
    (the reported value) and 2 more on one thread; and the model-like
    collection (505 bf16 tensors, AdamW, the collection benchmark's
    generator and seed), 3 steps on all host cores.  About 25 s of
    single-core work in all."""
    import numpy as np

    import oracle as O

    orc = O.load()
    cores = len(os.sched_getaffinity(0))
    n = 1 << 28
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    p = torch.empty(n, device=dev).uniform_(-1.0, 1.0, generator=gen).cpu().numpy()
    g = (torch.randn(n, device=dev, generator=gen) * 1e-3).cpu().numpy()
    s1 = np.zeros(n, np.float32)
    s2 = np.zeros(n, np.float32)
    hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    steps = 10
    t0 = time.perf_counter()
    for t in range(1, steps + 1):
        orc.update_f32(O.ADAM, O.F32, p, g, s1, s2, hp, t, nthreads=cores)
    dt = time.perf_counter() - t0
    gbs = W.bytes_per_element("adam", "fp32") * n * steps / dt / 1e9
    out = {"value": round(gbs, 2), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"the headline workload itself (fp32 Adam, 2^28 elements, same seed), {steps} "
                     f"steps, {dt:.2f} s wall on {cores} threads, OpenMP static schedule",
           "elements_per_s": round(n * steps / dt, 0)}
    # the same tensor, two more steps on one thread
    t0 = time.perf_counter()
    for t in range(steps + 1, steps + 3):
        orc.update_f32(O.ADAM, O.F32, p, g, s1, s2, hp, t, nthreads=1)
    dt1 = time.perf_counter() - t0
    out["single_thread"] = {"value": round(W.bytes_per_element("adam", "fp32") * n * 2 / dt1 / 1e9, 2),
                            "unit": "GB/s", "steps": 2, "elements_per_s": round(n * 2 / dt1, 0)}
    del p, g, s1, s2
    # the model-like collection: bf16 AdamW over 505 tensors, 3 steps
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    tensors = []
    for _, shp in W.model_collection():
        m = W.numel(shp)
        pb = torch.empty(m, device=dev).uniform_(-1, 1, generator=gen).to(torch.bfloat16)
        gb = (torch.randn(m, device=dev, generator=gen) * 0.01).to(torch.bfloat16)
        tensors.append((pb.cpu().view(torch.int16).numpy().view(np.uint16).copy(),
                        gb.cpu().view(torch.int16).numpy().view(np.uint16).copy(),
                        np.zeros(m, np.float32), np.zeros(m, np.float32)))
    hpc = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    elems = sum(t[0].size for t in tensors)
    t0 = time.perf_counter()
    for t in range(1, 4):
        for pc, gc, m1, m2 in tensors:
            orc.update_f32(O.ADAM, O.BF16, pc, gc, m1, m2, hpc, t, nthreads=cores)
    dtc = (time.perf_counter() - t0) / 3
    out["collection_505"] = {"us_per_step": round(dtc * 1e6, 1),
                             "GBps": round(W.bytes_per_element("adam", "bf16") * elems / dtc / 1e9, 2),
                             "steps": 3, "cores": cores, "tensors": len(tensors), "elements": elems}
    return out


if __name__ == "__main__":
    main()
