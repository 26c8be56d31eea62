#!/usr/bin/env python3
"""Benchmark of the batched verify step on one MI355X.

One step = one spec_verify call (the whole verify: statistics, acceptance,
residual/bonus draw) over one batch of the B=64, gamma=4, V=128256 bf16,
T=1.0 sampling workload (target N(0, 3^2) plus a +8 spike per position,
draft = target + N(0, 1.5^2)), with all inputs already in HBM.  Several
device copies of the logits are rotated so that successive steps do not hit
the 256 MB Infinity Cache.

Prints one JSON line.  `value` is verified rows per second; the roofline
object gives the dominant (only) kernel's achieved HBM rate from the
compulsory logit bytes (every row of the call: (2 g_b + 1) V e per batch row
when sampling) and its event-timed average launch duration.  Every mode runs
the kernel that reads the rows position by position and stops at the walk's
first rejection, so it reads fewer bytes than that: `walk_bytes_per_step`
counts the rows the walk uses (t_i, and d_i when sampling, for i <= n; t_g
after g acceptances), and --one-pass times the kernel that streams every row
instead.

With --top-k / --top-p a step is the filtered verify: the threshold kernel,
then the verify on the filtered rows (two launches); the draft tokens are
the workload's (drawn from the unfiltered q).  The threshold kernel is also
timed alone, and the roofline names the longer of the two kernels.

--mode ngram times prompt-lookup drafting alone (spec_ngram_draft over 64
contexts of 16k..32k tokens, n = 4..1, gamma = 4; context copies rotated like
the logits).  --mode round times a whole model-free speculative round: the
drafter, then the point-mode verify of its drafts against the B=64,
V=128256 target logits, both launches on one stream; with --adapt the
draft-length rule runs in the drafting launch's last step
(spec_ngram_draft_adaptive; --unfused: as its own launch between them),
capped by the draft lengths and fed the previous round's accepted counts.
--mode adapt times the controller alone over the same 64 rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 1 << 30  # at least this much distinct logit memory in rotation
# HBM byte counters of the kernel per workload and mode (committed summaries of
# rocprofv3 FETCH_SIZE / WRITE_SIZE runs); used only while the kernel source
# still has the hash they were taken on
COUNTERS = os.path.join(ROOT, "profiles", "{kernel}_c{config}_{mode}{filt}_counters.json")
KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_verification_07_amd", "csrc",
                          "spec_verify.hip")
NGRAM_SRC = os.path.join(ROOT, "speculative_decoding_verification_07_amd", "csrc",
                         "spec_ngram.hip")
NGRAM_COUNTERS = os.path.join(ROOT, "profiles", "ngram_kernel_{contexts}_counters.json")
# controller bytes per row: accepted count, previous length, length limit
# and state {A, T} read; length and state written
CONTROL_BYTES_PER_ROW = 4 + 4 + 4 + 16 + 4 + 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3)")
    ap.add_argument("--mode", default="sample",
                    choices=["sample", "greedy", "point", "ngram", "round", "adapt"])
    ap.add_argument("--adapt", action="store_true",
                    help="round: insert the adaptive draft-length controller")
    ap.add_argument("--draft-cost", type=float, default=0.05,
                    help="controller: cost of one draft token, in target passes")
    ap.add_argument("--unfused", action="store_true",
                    help="round --adapt: the controller as its own launch instead of inside "
                         "the drafting launch")
    ap.add_argument("--contexts", default="ctx32k", help="drafting workload (ngram, round)")
    ap.add_argument("--top-k", type=int, default=0, help="top-k filter of p and q (0: off)")
    ap.add_argument("--top-p", type=float, default=1.0, help="top-p filter of p and q (1: off)")
    ap.add_argument("--rotate", type=int, default=0, help="device copies (0: enough for 1 GiB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=18.0)
    ap.add_argument("--with-copy", action="store_true",
                    help="also run the reference copy kernel (counter calibration)")
    ap.add_argument("--tune", default="", help="vectors[,target_workgroups]")
    ap.add_argument("--one-pass", action="store_true",
                    help="stream every row in one pass instead of reading the rows "
                         "position by position")
    return ap.parse_args()


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def source_hash(path=KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_ceiling(sv, torch, dev, stream, with_copy=False) -> float:
    """HBM read ceiling of this machine: plain streaming read of 4 GiB (GB/s)."""
    probe = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    pout = None
    for _ in range(3):
        pout = sv.probe_read(probe, pout)
    torch.cuda.synchronize()
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record(stream)
    for _ in range(10):
        sv.probe_read(probe, pout)
    pe1.record(stream)
    torch.cuda.synchronize()
    ceiling = probe.numel() * 10 / (pe0.elapsed_time(pe1) * 1e-3) / 1e9
    if with_copy:
        dst = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
        for _ in range(5):
            sv.probe_copy(probe[: 1 << 28], dst)
        torch.cuda.synchronize()
        del dst
    del probe
    return ceiling


def timed(run, K, warmup, stream, torch):
    """K back-to-back calls of run(k) between two events on the launch
    stream, after `warmup` untimed ones; returns (total ms, wall s)."""
    for k in range(warmup):
        run(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for k in range(K):
        run(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), time.perf_counter() - wall0


def bench_drafting(args):
    """--mode ngram (drafting alone) and --mode round (drafting + point verify)."""
    import ctypes

    import numpy as np
    import torch

    import speculative_decoding_verification_07_amd as sv
    from speculative_decoding_verification_07_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = sv.load()
    if args.one_pass:
        sv.tune(one_pass=True)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    hs = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p

    t0 = time.time()
    cc = inputs.CONTEXT_CONFIGS[args.contexts]
    ctx, lens = inputs.make_contexts(cc, rnd=0)
    B, G = cc.B, cc.gamma
    draft_bytes = inputs.context_bytes(lens, G)
    ctx0 = torch.from_numpy(ctx).to(dev)
    ln = torch.from_numpy(lens).to(dev)
    rot_c = args.rotate or max(1, -(-ROTATE_BYTES // ctx.nbytes))
    ctxs = [ctx0] + [ctx0.clone() for _ in range(rot_c - 1)]
    nws = sv.Workspace(sv.ngram_workspace_bytes(B))
    d_tok = torch.empty((B, G), dtype=torch.int32, device=dev)
    d_len, d_n, d_pos = (torch.empty(B, dtype=torch.int32, device=dev) for _ in range(3))
    sv.ngram_draft(ctx0, ln, n_min=cc.n_min, n_max=cc.n_max, gamma=G, workspace=nws,
                   out=(d_tok, d_len, d_n, d_pos))  # argument checks, once
    dargs = [(P(c.data_ptr()), P(ln.data_ptr()), B, cc.stride, cc.n_min, cc.n_max, G,
              P(d_tok.data_ptr()), P(d_len.data_ptr()), P(d_n.data_ptr()), P(d_pos.data_ptr()),
              P(nws.ptr), nws.nbytes, hs) for c in ctxs]

    def draft(k):
        lib.spec_ngram_draft(*dargs[k % rot_c])

    # the controller: previous round's counts in, this round's lengths out
    # (in place), capped by the draft lengths
    ctl = sv.GammaControl(B, gamma_max=G, draft_cost=args.draft_cost)
    c_nacc = torch.full((B,), -1, dtype=torch.int32, device=dev)
    c_gam = torch.zeros(B, dtype=torch.int32, device=dev)
    ctl(c_nacc, c_gam, gamma_limit=d_len, out=c_gam)  # argument checks, once
    cargs = (P(c_nacc.data_ptr()), P(c_gam.data_ptr()), None, P(d_len.data_ptr()),
             P(ctl.state.data_ptr()), B, *ctl.params,
             P(c_gam.data_ptr()), None, hs)

    def control(k):
        lib.spec_gamma_control(*cargs)

    fargs = [(P(c.data_ptr()), P(ln.data_ptr()), B, cc.stride, cc.n_min, cc.n_max, G,
              P(c_nacc.data_ptr()), P(c_gam.data_ptr()), None, P(ctl.state.data_ptr()),
              *ctl.params[1:], P(d_tok.data_ptr()), P(d_len.data_ptr()), P(d_n.data_ptr()),
              P(d_pos.data_ptr()), P(c_gam.data_ptr()), None, P(nws.ptr), nws.nbytes, hs)
             for c in ctxs]

    def draft_adapt(k):
        lib.spec_ngram_draft_adaptive(*fargs[k % rot_c])

    fused = args.mode == "round" and args.adapt and not args.unfused
    if fused:
        draft_adapt(0)  # argument checks, once
        torch.cuda.synchronize()

    K = args.steps
    adapt = args.mode == "adapt" or (args.mode == "round" and args.adapt)
    calls, case, step_bytes, rot_v = [draft], None, draft_bytes, 0
    if args.mode == "adapt":
        calls, step_bytes = [control], B * CONTROL_BYTES_PER_ROW
    if args.mode == "round":
        case = inputs.make_case(args.config, rnd=0, mode="point")
        if case.G < G or case.B != B:
            raise SystemExit("round: the verify workload must have the drafter's batch and "
                             "at least its gamma")
        V = case.V
        dt = sv.BF16 if case.target.dtype == np.uint16 else sv.F32

        def logits(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        tgt0 = logits(np.ascontiguousarray(case.target[:, :G + 1]))
        rot_v = args.rotate or max(1, -(-ROTATE_BYTES // (tgt0.numel() * tgt0.element_size())))
        tgts = [tgt0] + [tgt0.clone() for _ in range(rot_v - 1)]
        uni = torch.from_numpy(np.ascontiguousarray(case.uniforms[:, :G + 1])).to(dev)
        kv = torch.from_numpy(case.kv_len).to(dev)
        vws = sv.Workspace(sv.workspace_bytes(B, G, V, dt, sv.POINT))
        vout = (torch.empty((B, G + 1), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))
        vout = (vout[0], c_nacc, vout[2]) if adapt else vout
        verifies = [sv.Prepared(t, None, d_tok, uni, c_gam if adapt else d_len, kv,
                                temperature=case.T, mode=sv.POINT, workspace=vws, out=vout)
                    for t in tgts]
        def verify(k):
            verifies[k % rot_v]()

        if fused:
            calls = [draft_adapt]
        elif adapt:
            calls.append(control)
        calls.append(verify)
        # compulsory verify bytes: g_b + 1 target rows per row, g_b the draft length
        e = tgt0.element_size()

    gen_s = time.time() - t0

    def step(k):
        for c in calls:
            c(k)

    total_ms, wall = timed(step, K, args.warmup, stream, torch)
    draft_ms, _ = timed(draft, K, args.warmup, stream, torch)
    control_us = fused_us = None
    if adapt:
        control_ms, _ = timed(control, K, args.warmup, stream, torch)
        control_us = control_ms / K * 1e3
    if fused:
        fused_ms, _ = timed(draft_adapt, K, args.warmup, stream, torch)
        fused_us = fused_ms / K * 1e3
    ms_per_step = total_ms / K
    draft_us = draft_ms / K * 1e3
    if case is not None:
        # the verify alone, on the drafts the last step left
        verify_ms, _ = timed(verify, K, args.warmup, stream, torch)
    g_b = d_len.cpu().numpy()
    n_b = d_n.cpu().numpy()
    line_extra = {"control_kernel_us": control_us} if adapt else {}
    if fused:
        line_extra["draft_and_control_kernel_us"] = fused_us
    if adapt:
        line_extra["mean_controlled_gamma"] = float(c_gam.float().mean())
    if args.mode == "round":
        g_v = (c_gam if adapt else d_len).cpu().numpy().astype(np.int64)
        step_bytes = (draft_bytes + int((g_v + 1).sum()) * V * e
                      + (B * CONTROL_BYTES_PER_ROW if adapt else 0))
        verify_us = verify_ms / K * 1e3
        n_acc = vout[1].cpu().numpy()
        emitted = int((n_acc + 1).sum())
        vname = "verify_kernel" if args.one_pass else "verify_rows_kernel"
        kern_name, kern_us = ((vname, verify_us) if verify_us >= draft_us
                              else ("ngram_kernel", draft_us))
        kern_bytes = int((g_v + 1).sum()) * V * e if kern_name == vname else draft_bytes
        line_extra.update({"verify_kernel_us": verify_us, "emitted_tokens_per_s":
                           emitted * K / (total_ms * 1e-3), "mean_emitted_per_row": emitted / B,
                           "diagnostics": vws.diagnostics()})
    elif args.mode == "adapt":
        kern_name, kern_us, kern_bytes = "gamma_kernel", control_us, step_bytes
    else:
        kern_name, kern_us, kern_bytes = "ngram_kernel", draft_us, draft_bytes
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9
    ceiling = read_ceiling(sv, torch, dev, stream, args.with_copy)

    traffic = None
    if kern_name == "ngram_kernel" and os.path.exists(NGRAM_COUNTERS.format(contexts=args.contexts)):
        with open(NGRAM_COUNTERS.format(contexts=args.contexts)) as f:
            cnt = json.load(f)
        if cnt.get("source_sha256_16") == source_hash(NGRAM_SRC):
            traffic = cnt.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu:
        import oracle
        reps, t_cpu = 0, 0.0
        ost = np.zeros((B, 2))
        o_n = np.full(B, -1, np.int32)
        o_g = np.zeros(B, np.int32)
        while t_cpu < args.cpu_seconds and reps < 100000:
            c0 = time.perf_counter()
            if args.mode == "adapt":
                oracle.gamma_control(ost, o_n, o_g, gamma_limit=g_b, gamma_max=G,
                                     draft_cost=args.draft_cost)
            else:
                w = oracle.ngram_draft(ctx, lens, n_min=cc.n_min, n_max=cc.n_max, gamma=G)
            if case is not None:
                gv = w.length
                if adapt:
                    gv, _ = oracle.gamma_control(ost, o_n, o_g, gamma_limit=w.length,
                                                 gamma_max=G, draft_cost=args.draft_cost)
                r = oracle.verify(case.target[:, :G + 1], None, np.maximum(w.draft, 0),
                                  case.uniforms[:, :G + 1], gv, case.kv_len,
                                  temperature=case.T, mode=oracle.POINT, threads=1)
                o_n, o_g = r.n_accepted, gv
            t_cpu += time.perf_counter() - c0
            reps += 1
        what = {"ngram": "drafting", "adapt": "draft-length control",
                "round": "drafting + " + ("control + " if adapt else "") + "point verify"}[args.mode]
        cpu = {"value": B * reps / t_cpu, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} full batches of this workload ({B} rows each), "
                         f"{t_cpu:.1f} s of oracle {what}"}

    wl = (f"prompt-lookup drafting B={B} contexts {cc.L_lo}..{cc.stride} tokens "
          f"n={cc.n_max}..{cc.n_min} gamma={G} ({args.contexts})")
    if adapt:
        wl += (f" + adaptive gamma (draft cost {args.draft_cost}"
               + (", in the drafting launch)" if fused else ", own launch)"))
    if args.mode == "adapt":
        wl = (f"adaptive draft length B={B} gamma_max={G} draft cost {args.draft_cost}, "
              f"capped by the {args.contexts} draft lengths")
    if case is not None:
        wl += f" + point verify V={V} bf16 T={case.T} (config {args.config})"
    metric = {"ngram": "drafted rows/s (prompt-lookup drafting)",
              "adapt": "controlled rows/s (adaptive draft length)",
              "round": "verified rows/s (model-free round: prompt-lookup draft + "
                       + ("adaptive gamma + " if adapt else "") + "point verify)"}[args.mode]
    line = {
        "metric": metric,
        "value": B * K / (total_ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"ngram": "int32", "adapt": "f64", "round": "f32"}[args.mode],
        "data": "synthetic",
        "config": {"workload": wl, "B": B, "stride": cc.stride, "gamma": G,
                   "n_max": cc.n_max, "n_min": cc.n_min, "rotated_context_copies": rot_c,
                   "rotated_logit_copies": rot_v, "compulsory_bytes_per_step": step_bytes},
        "ngram_kernel_us": draft_us,
        "draft_rows_matched": int((n_b > 0).sum()),
        "mean_draft_len": float(g_b.mean()),
        "step_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "read_ceiling_gbps": ceiling, "wall_s_timed": wall, "input_gen_s": gen_s,
        **line_extra,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": kern_name, "bytes_per_launch": kern_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the verify step is "
              "independent per batch row, so N GPUs would each run this same benchmark on "
              "their own rows", file=sys.stderr)
        sys.exit(2)
    if args.mode in ("ngram", "round", "adapt"):
        bench_drafting(args)
        return

    import numpy as np
    import torch

    import speculative_decoding_verification_07_amd as sv
    from speculative_decoding_verification_07_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sv.load()
    if args.tune or args.one_pass:
        tv = [int(v) for v in args.tune.split(",")] if args.tune else []
        sv.tune(*tv, one_pass=args.one_pass)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    t0 = time.time()
    case = inputs.make_case(args.config, rnd=0, mode=args.mode)
    gen_s = time.time() - t0
    B, G, V = case.B, case.G, case.V
    dt = sv.BF16 if case.target.dtype == np.uint16 else sv.F32
    mode = {"sample": sv.SAMPLE, "greedy": sv.GREEDY, "point": sv.POINT}[args.mode]
    step_bytes = inputs.algorithmic_bytes(case)
    logit_bytes = case.target.nbytes + (case.draft.nbytes if mode == sv.SAMPLE else 0)
    rot = args.rotate or max(1, -(-ROTATE_BYTES // logit_bytes))

    def logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # point-mass drafts come without draft logits: none are passed
    tgt0 = logits(case.target)
    dft0 = logits(case.draft) if mode == sv.SAMPLE else None
    sets = [(tgt0, dft0)] + [(tgt0.clone(), None if dft0 is None else dft0.clone())
                             for _ in range(rot - 1)]
    tok = torch.from_numpy(case.tokens).to(dev)
    uni = torch.from_numpy(case.uniforms).to(dev)
    gam = torch.from_numpy(case.gamma).to(dev)
    kv = torch.from_numpy(case.kv_len).to(dev)
    ws = sv.Workspace(sv.workspace_bytes(B, G, V, dt, mode))
    out = (torch.empty((B, G + 1), dtype=torch.int32, device=dev),
           torch.empty(B, dtype=torch.int32, device=dev),
           torch.empty(B, dtype=torch.int32, device=dev))

    filt = mode != sv.GREEDY and ((0 < args.top_k < V) or args.top_p < 1.0)
    calls = [sv.Prepared(t, d, tok, uni, gam, kv, temperature=case.T, mode=mode, workspace=ws,
                         out=out, top_k=args.top_k if filt else 0,
                         top_p=args.top_p if filt else 1.0) for t, d in sets]

    for k in range(args.warmup):
        calls[k % rot]()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps between two events on the launch stream
    K = args.steps
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e_start.record(stream)
    for k in range(K):
        calls[k % rot]()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = e_start.elapsed_time(e_end)
    # second timed pass: an event pair around every launch gives each
    # kernel's own duration on the stream
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for k in range(K):
        ev0[k].record(stream)
        calls[k % rot]()
        ev1[k].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([ev0[k].elapsed_time(ev1[k]) for k in range(K)])
    filter_us = None
    if filt:
        # the threshold kernel alone, back to back, into a scratch array
        import ctypes
        thr = torch.empty((B, 2 * G + 1), dtype=torch.float32, device=dev)
        sv.filter_thresholds(tgt0, dft0, gam, temperature=case.T, mode=mode, top_k=args.top_k,
                             top_p=args.top_p, out=thr)  # argument checks, once
        lib = sv.load()
        hs = ctypes.c_void_p(stream.cuda_stream)
        fargs = [(ctypes.c_void_p(t_.data_ptr()),
                  ctypes.c_void_p(d_.data_ptr()) if d_ is not None else None) for t_, d_ in sets]
        def thresholds(k):
            t_, d_ = fargs[k % rot]
            lib.spec_filter_thresholds(t_, d_, ctypes.c_void_p(gam.data_ptr()), B, G, V, dt,
                                       ctypes.c_float(case.T), mode, args.top_k,
                                       ctypes.c_float(args.top_p), ctypes.c_void_p(thr.data_ptr()),
                                       hs)
        for k in range(args.warmup):
            thresholds(k)
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for k in range(K):
            thresholds(k)
        f1.record(stream)
        torch.cuda.synchronize()
        filter_us = f0.elapsed_time(f1) / K * 1e3
    diag = ws.diagnostics()
    n_acc = out[1].cpu().numpy()

    ms_per_step = total_ms / K
    # one launch per step: the kernel's average launch duration on its stream
    # is the back-to-back time per step (event pairs around single launches
    # add their own overhead and are reported separately)
    kern_s = ms_per_step * 1e-3
    # every mode reads the rows position by position unless --one-pass
    kernel_name = "verify_kernel" if args.one_pass else "verify_rows_kernel"
    if filter_us is not None:
        # two launches per step: the longer one is the dominant kernel
        verify_s = kern_s - filter_us * 1e-6
        kern_s = max(verify_s, filter_us * 1e-6)
        if verify_s < filter_us * 1e-6:
            kernel_name = "filter_kernel"
    achieved = step_bytes / kern_s / 1e9
    emitted = int((n_acc + 1).sum())
    tested = int(np.minimum(n_acc + 1, case.gamma).sum())
    # the rows the walk uses: (t_i, d_i) for i <= n, t_g when every draft is
    # accepted (sampling); t_0..t_n (greedy, point-mass drafts)
    gb = np.clip(case.gamma.astype(np.int64), 0, G)
    na = n_acc.astype(np.int64)
    if mode == sv.SAMPLE:
        walk_rows = np.where(na < 0, 0, np.where(na < gb, 2 * (na + 1), 2 * gb + 1))
    else:
        walk_rows = np.where(na < 0, 0, na + 1)
    walk_bytes = int(walk_rows.sum()) * V * case.target.itemsize

    ceiling = read_ceiling(sv, torch, dev, stream, args.with_copy)

    traffic = None
    counters = COUNTERS.format(kernel=kernel_name, config=args.config, mode=args.mode,
                               filt=f"_k{args.top_k}_p{args.top_p:g}" if filt else "")
    if os.path.exists(counters):
        with open(counters) as f:
            cnt = json.load(f)
        if cnt.get("source_sha256_16") == source_hash() and cnt.get("workload_config") == args.config \
                and cnt.get("mode") == args.mode:
            traffic = cnt.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu:
        import oracle
        omode = {sv.SAMPLE: oracle.SAMPLE, sv.GREEDY: oracle.GREEDY, sv.POINT: oracle.POINT}[mode]

        def oracle_rate(threads, batches):
            c0 = time.perf_counter()
            for _ in range(batches):
                oracle.verify(case.target, case.draft, case.tokens, case.uniforms, case.gamma,
                              case.kv_len, temperature=case.T, mode=omode, threads=threads,
                              top_k=args.top_k if filt else 0,
                              top_p=args.top_p if filt else 1.0)
            return B * batches / (time.perf_counter() - c0)

        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
        # size each run from one timed batch: about cpu_seconds / 6 per run,
        # three runs on one thread and three on all threads (median of each)
        t1 = B / oracle_rate(1, 1)
        n1 = max(1, int(args.cpu_seconds / 6 / t1))
        one = sorted(oracle_rate(1, n1) for _ in range(3))
        tn = B / oracle_rate(threads, 1)
        nn = max(1, int(args.cpu_seconds / 6 / tn))
        alln = sorted(oracle_rate(threads, nn) for _ in range(3))
        cpu = {"value": alln[1], "unit": "rows/s", "cores": threads, "kind": "oracle",
               "value_1_thread": one[1], "runs_1_thread": one, "runs_all_threads": alln,
               "cpu_model": cpu_model(),
               "sample": f"median of 3 runs of {nn} full batches ({B} rows each) on {threads} "
                         f"threads, and of 3 runs of {n1} batches on 1 thread; "
                         f"double-precision oracle"}

    ftxt = f" top_k={args.top_k} top_p={args.top_p}" if filt else ""
    cfgd = {"workload": f"verify B={B} gamma={G} V={V} "
                        f"{'bf16' if dt == sv.BF16 else 'fp32'} logits T={case.T} {args.mode}"
                        f"{ftxt} (config {args.config})",
            "B": B, "gamma": G, "V": V, "logits_dtype": "bf16" if dt == sv.BF16 else "fp32",
            "mode": args.mode, "temperature": case.T, "rotated_copies": rot,
            "compulsory_bytes_per_step": step_bytes}
    if filt:
        cfgd.update(top_k=args.top_k, top_p=args.top_p)
    line = {
        "metric": "verified rows/s (batched speculative-decoding verify step)",
        "value": B * K / (total_ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": cfgd,
        "emitted_tokens_per_s": emitted * K / (total_ms * 1e-3),
        "step_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "walk_bytes_per_step": walk_bytes,
        "walk_gbps": walk_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kernel_us": kern_s * 1e6,
        "filter_kernel_us": filter_us,
        "kernel_us_event_pair_mean": float(launch_ms.mean()) * 1e3,
        "kernel_us_event_pair_p50": float(np.median(launch_ms)) * 1e3,
        "acceptance_rate": (emitted - B) / max(tested, 1),
        "mean_emitted_per_row": emitted / B,
        "read_ceiling_gbps": ceiling,
        "wall_s_timed": wall,
        "input_gen_s": gen_s,
        "diagnostics": diag,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": kernel_name, "bytes_per_launch": step_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
