#!/usr/bin/env python3
"""Throughput of the gated delta-rule layer on one MI355X.

A step is one forward plus one backward of the chunked per-channel-decay layer
(gdn_forward_train then gdn_backward_train: every kernel of the hot path; the
backward reuses the forward's residuals, as a training step does) over one batch of
synthetic inputs shaped like the pages' training workload: B=8, T=4096, H=6,
Dk=Dv=128, chunk 64, bf16 q/k/v with fp32 decay, gates and state (Marin note,
"Single-device benchmark"; atomic_ops card, "Benchmarks").  Inputs are resident
in HBM before timing starts.  The result is gated on correctness first: sampled
heads are checked against the CPU oracle (atomic_ops card, "Reproduce": timings
are correctness-gated).

Printed: ONE JSON line.  value = tokens/s of the fwd+bwd step (tokens = B*T
per call, each token carrying all H heads).  The step is timed as one HIP-graph
replay of the two library calls (captured once; the library allocates nothing
and issues no memset on this path), used only when three check replays, each
after its outputs were overwritten with NaN, reproduce the eager calls bitwise;
the eager calls' time is reported beside it (and is the headline otherwise,
or with --no-graph).  Also reported: forward-only
tokens/s, the decode step (B=256, H=16, 128x128 state) in GB/s, per-kernel
device times from HIP events recorded around each launch on its stream, the
roofline of the dominant kernel, and the CPU oracle timed on this host.

    python bench.py [--steps K] [--warmup W] [--dtype bf16|f32] [--batch B]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense)
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
# TPU v6e, Sept-2026 prototype, B=8 T=4096 H=6 d=128 BF16 fwd+bwd: 22.44 ms
# (Marin note, "Single-device benchmark") -> B*T / 22.44 ms
PAGES_FWDBWD_TOKENS_S = 8 * 4096 / 22.44e-3
# kernel launch name -> the source file that defines it (for the counter digest)
KERNEL_SOURCE = {"prep": "chunk_fwd.hip", "prep_T": "chunk_fwd.hip",
                 "scan": "chunk_fwd.hip",
                 "scan_save": "chunk_fwd.hip", "scan_train": "chunk_fwd.hip",
                 "bscan": "chunk_bwd.hip", "bchunk1": "chunk_bwd.hip", "bchunk2": "chunk_bwd.hip",
                 "bchunk2_finish": "chunk_bwd.hip", "l2norm_bwd": "chunk_bwd.hip",
                 "decode": "decode.hip"}
CSRC = os.path.join(ROOT, "gated_delta_rule_52_amd", "csrc")
COUNTERS_MD = os.path.join(ROOT, "profiles", "hbm_traffic_fwdbwd_b8_t4096_h6_d128_bf16.md")


def kernel_source_digest(name):
    """sha256 over the file that defines a kernel and every shared header: HBM
    counters taken on another digest describe different code."""
    import hashlib
    h = hashlib.sha256()
    files = [KERNEL_SOURCE[name]] + sorted(f for f in os.listdir(CSRC) if f.endswith(".h"))
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch of `name` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or None
    when there is none or the kernel's sources changed since it was taken."""
    try:
        with open(COUNTERS_MD) as fh:
            text = fh.read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        ent = blob["kernels"][name]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    if ent.get("source_sha256") != kernel_source_digest(name):
        return None
    return ent["traffic_bytes"]


def kernel_work(name, B, T, H, C, DK, DV, in_bytes, per_channel=True, l2n=False):
    """Algorithmic work of one launch of a chunked kernel: HBM bytes (each
    input read once, each output written once, in this design's data layout)
    and the matrix-product flops it must do, split by the operand type of its
    matrix-core instructions.  Counts are per chunk-head, times the launch's
    B*H*ceil(T/C) chunk-heads.  l2n: with use_qk_l2norm (the prep writes and
    bchunk2 reads the rows' scales r).  Returns (bytes, {"f32": flops, "bf16": flops})."""
    NC = (T + C - 1) // C
    n = B * H * NC
    f4 = 4
    bt = in_bytes == 2 and C == 64 and DK >= 64  # bf16 chunk tables and intermediates
    ft = in_bytes == 4 and C == 64 and DK >= 64  # fp32 chunk tables of the fp32-operand kernels
    tb = 2 if bt else 4                          # bytes per table element
    db = 2 if bt else 4 if ft else 0             # bytes per saved chunk delta D
    ib = in_bytes
    cd, cv, cc, kv = C * DK, C * DV, C * C, DK * DV
    tri = C * (C + 1) // 2                       # lower triangle incl. diagonal
    gb = cd * f4 if per_channel else C * f4      # log-decay bytes per chunk
    mt = "bf16" if in_bytes == 2 else "f32"      # operand type of the big products
    fl = {"f32": 0.0, "bf16": 0.0}
    if name in ("prep", "prep_T"):
        by = 2 * cd * ib + gb + C * f4                             # q k, g, beta
        by += 3 * cd * tb + cc * tb + DK * f4                      # W Qg Kh^T Ps, gam
        by += cv * ib + cv * f4                                    # v in, U out
        fl[mt] += 2 * (2 * tri * DK) + 2 * tri * (DK + DV)         # P, A; W = T X_K, U = T X_V
        if name == "prep_T":
            by += cc * f4                                          # T
        by += 2 * C * f4 if l2n else 0                             # r of the q and k rows
        fl["f32"] += 2 * C ** 3 / 3                                # (I + A)^-1
    elif name in ("scan", "scan_save", "scan_train"):
        by = 3 * cd * tb + cc * tb + cv * f4 + DK * f4             # W Qg Kh Ps, U, gam
        if name == "scan_save":                                    # deltas and states only
            by -= cd * tb + cc * tb
            by += kv * tb + cv * db
            fl[mt] += 4 * C * DK * DV
        else:
            by += cv * ib                                          # o
            if name == "scan_train":
                by += kv * tb + cv * db                            # chunk-start states, D
            fl[mt] += 6 * C * DK * DV + 2 * tri * DV
    elif name == "bscan":
        by = cc * tb + 3 * cd * tb + DK * f4 + cv * ib             # Ps Kh^T Qg W, gam, dO
        by += kv * tb + cv * tb                                    # dS (chunk ends), dD
        fl[mt] += 6 * C * DK * DV + 2 * tri * DV
    elif name == "bchunk1":
        it = 2 if bt else 4
        by = 2 * cv * ib + C * f4 + cc * f4 + 2 * kv * tb + cv * tb   # v dO, beta, T, S, dS, dD
        by += (cv * 2 + cd * tb) if bt else cv * f4 if ft else (cd + cv) * f4  # D, W | D | W, U
        by += cv * ib + 3 * cd * it + 2 * cc * it + DK * f4 + C * f4  # dv, dQg dX_K|dW dKh, dPs dA|dT1, dgam, dbeta
        fl[mt] += 6 * C * DK * DV + 2 * tri * DV + 2 * C * C * DV     # dQg dW dKh, dPs, dX_V V^T | dD X_V^T
        fl["f32"] += 2 * tri * DV                                      # dX_V = T^T dD
        if bt:   # keys' WY adjoint: dX_K = T^T dW, G1 = (dX_V V^T) diag(beta) T^T,
                 # dA = -(G1 + dX_K W^T) strictly lower
            fl["bf16"] += 2 * tri * DK + 2 * tri * C + 2 * (C * (C - 1) // 2) * DK
        elif not ft:
            fl[mt] += 2 * C * DK * DV                                  # D = U - W S
    elif name == "bchunk2_finish":  # dbeta (and per-head dg) from the channel-half partials
        by = (3 * C * f4 + C * f4) + (0 if per_channel else 2 * C * f4 + C * f4)
    elif name == "bchunk2":
        it = 2 if bt else 4
        by = 2 * cd * ib + gb + C * f4                                # q k, g, beta
        by += 3 * cd * it + 2 * cc * it + DK * f4                     # dQg dX_K|dW dKh, dPs dA|dT1, dgam
        by += 2 * cd * ib + (gb if per_channel else 0)                # dq dk, dg
        if bt:   # two channel halves: partial dbeta (and per-head dg) sums
            by += 2 * C * f4 + (0 if per_channel else 2 * C * f4)
        else:    # T, dbeta part in; dX_K = T^T dW, dT = dT1 + dW X_K^T, dA = -T^T dT T^T
            by += cc * f4 + C * f4 + C * f4 + (0 if per_channel else C * f4)
            fl["f32"] += 2 * (2 * tri * DK) + 2 * (2 * C ** 3 / 3)
        fl[mt] += 2 * (2 * tri * DK) + 2 * (2 * tri * DK)             # score gradients of P and A
        by += 2 * C * f4 if l2n else 0                                # r of the q and k rows
    elif name == "l2norm_bwd":  # use_qk_l2norm adjoint, in place on dq, dk
        by = 4 * cd * ib + 2 * C * f4 + 2 * cd * ib                   # q k dq dk, r in; dq dk out
    else:
        return None
    return by * n, {k_: v_ * n for k_, v_ in fl.items()}


# The method's own work per token-head (one token of one head), as the layer's
# inputs are read once and its outputs written once: q, k, v, g, beta, o in the
# forward; q, k, v, g, beta, dO in and dq, dk, dv, dg, dbeta out in the backward.
# bf16 inputs at 128 x 128 with per-channel decay: 1,540 B forward, 2,824 B
# backward, 4,364 B forward + backward; fp32 inputs: 2,564, 4,616, 7,180 B.  The
# chunk tables, chunk-start states and gradients handed between kernels are this
# design's choice, not the method's, and are not counted.  Matrix-product work of
# the chunked form per chunk of 64 tokens of one head (Dk = Dv = 128): forward
# 8.52 MFLOP (cross-block scores 0.52, T21 merge 0.13, U and W 1.05, scan 6.82),
# backward about 17.2 MFLOP.
def method_bytes_per_token_head(name, D, in_bytes, per_channel=True):
    """Share of the layer's own inputs and outputs that kernel `name` must move
    per token-head (each input it reads once, each output it writes once).
    Summing over the kernels counts an input read by two kernels twice; the
    step totals use method_step_bytes."""
    ib, gb = in_bytes, (D * 4 if per_channel else 4)
    return {"prep": 3 * D * ib + gb + 4, "prep_T": 3 * D * ib + gb + 4,
            "scan": D * ib, "scan_train": D * ib, "scan_save": 0,
            "bscan": D * ib,                                   # dO
            "bchunk1": 3 * D * ib + 4,                         # v, dO, beta in; dv out
            "bchunk2": 4 * D * ib + 2 * gb + 4,                # q, k, g, beta in; dq, dk, dg out
            "bchunk2_finish": 4,                               # dbeta out
            "l2norm_bwd": 4 * D * ib}.get(name)


def method_step_bytes(D, in_bytes, per_channel=True, backward=True):
    """The method's bytes per token-head for a forward (or forward + backward)
    pass: each input of the pass read once, each output written once."""
    ib, gb = in_bytes, (D * 4 if per_channel else 4)
    fwd = 3 * D * ib + gb + 4 + D * ib
    bwd = (3 * D * ib + gb + 4 + D * ib) + (3 * D * ib + gb + 4)
    return fwd + bwd if backward else fwd


METHOD_MFLOP_PER_CHUNK_HEAD = {"fwd": 0.52 + 0.13 + 1.05 + 6.82, "bwd": 17.2}


def roofline(name, dur_s, B, T, H, C, D, in_bytes, l2n=False, per_channel=True):
    """Roofline of one launch.  achieved = the method's bytes for this kernel
    (method_bytes_per_token_head x the B*T*H token-heads of one launch) over
    the launch's duration; the bound is the larger of that byte floor at the
    HBM peak and the kernel's matrix-product work at the dense MFMA peak of its
    operand type.  The bytes this design moves (chunk tables, hand-offs) are
    reported beside it as design_bytes_per_launch and frac_design."""
    units = B * T * H
    mb = method_bytes_per_token_head(name, D, in_bytes, per_channel) * units
    by, fl = kernel_work(name, B, T, H, C, D, D, in_bytes, per_channel=per_channel, l2n=l2n)
    terms = {"hbm": mb / (PEAK_HBM_GBS * 1e9)}
    for mt, f in fl.items():
        if f:
            terms["mfma_" + mt] = f / (PEAK_TFLOPS[mt] * 1e12)
    bound = max(terms, key=terms.get)
    if bound == "hbm":
        r = {"bound": "hbm", "achieved": mb / dur_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        mt = bound[5:]
        r = {"bound": "mfma", "achieved": fl[mt] / dur_s / 1e12, "peak": PEAK_TFLOPS[mt],
             "unit": "TFLOP/s", "mfma_dtype": mt}
    r["frac"] = r["achieved"] / r["peak"]
    r["floor_us"] = {k_: v_ * 1e6 for k_, v_ in terms.items()}
    r["method_bytes_per_token_head"] = mb / units
    r["token_heads_per_launch"] = units
    r["method_bytes_per_launch"] = mb
    r["design_bytes_per_launch"] = by
    r["frac_design"] = by / dur_s / 1e9 / PEAK_HBM_GBS
    r["mfma_flops_per_launch"] = fl
    return r


def step_roofline(ms, B, T, H, C, D, in_bytes, backward=True, per_channel=True):
    """The whole pass against the method's floor: bytes (each input read once,
    each output written once) at the HBM peak, and the chunked form's
    matrix-product flops at the dense MFMA peak of the operand type."""
    units = B * T * H
    by = method_step_bytes(D, in_bytes, per_channel, backward) * units
    n_ch = B * H * ((T + C - 1) // C)
    mflop = METHOD_MFLOP_PER_CHUNK_HEAD["fwd"] + (METHOD_MFLOP_PER_CHUNK_HEAD["bwd"] if backward else 0.0)
    fl = mflop * 1e6 * n_ch * (D / 128) ** 2
    mt = "bf16" if in_bytes == 2 else "f32"
    s = ms * 1e-3
    return {"method_bytes_per_token_head": by / units, "method_bytes": by,
            "achieved_GBs": by / s / 1e9, "frac_hbm": by / s / 1e9 / PEAK_HBM_GBS,
            "hbm_floor_us": by / (PEAK_HBM_GBS * 1e9) * 1e6,
            "mfma_flops": fl, "mfma_dtype": mt, "achieved_TFLOPs": fl / s / 1e12,
            "frac_mfma": fl / s / 1e12 / PEAK_TFLOPS[mt],
            "mfma_floor_us": fl / (PEAK_TFLOPS[mt] * 1e12) * 1e6,
            "bound": "hbm" if by / PEAK_HBM_GBS / 1e9 >= fl / PEAK_TFLOPS[mt] / 1e12 else "mfma"}


def parity_gate(checks):
    """Refuse to report throughput when a correctness check failed (atomic_ops
    card, "Reproduce": a row that does not match is rejected; Marin note,
    "Single-device benchmark": results are checked before timing).  `checks`
    maps a row name to its pass flag; on any failure the names go to stderr and
    the process exits with status 3 before anything is printed on stdout."""
    bad = [name for name, ok in checks.items() if not ok]
    if bad:
        print("bench.py: parity check failed for " + ", ".join(bad)
              + "; no throughput is reported", file=sys.stderr, flush=True)
        sys.exit(3)


def emit(line, checks):
    """Print the one JSON result line, only if every check in `checks` passed."""
    parity_gate(checks)
    print(json.dumps(line), flush=True)


def median_sync_ms(fn, n=20):
    """Median over n calls of fn, each between two synchronisations and timed
    with events on the current stream (the Marin note's protocol: median of 20
    synchronised calls)."""
    import torch
    times = []
    for _ in range(n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def graph_replay(fn, outs, args):
    """Capture one call of fn (all its launches) in a HIP graph and time
    --steps replays.  Each of three check replays must reproduce the eager
    call's outputs bitwise: the outputs are overwritten with NaN before each
    replay, and an eager call and a synchronization sit between replays."""
    import torch
    fn()
    torch.cuda.synchronize()
    want = [x.clone() for x in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    same = True
    for _ in range(3):
        for x in outs:
            x.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        same &= all(torch.equal(x, y) for x, y in zip(outs, want))
        fn()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    del graph
    return {"ms_per_step": ms, "replays_equal_eager_bitwise": bool(same)}


def graph_entry(fn, outs, args, tokens):
    """graph_replay of a variant's training pair, with its token rate, or None
    under --no-graph"""
    if args.no_graph:
        return None
    res = graph_replay(fn, outs, args)
    res["tokens_per_s"] = tokens / (res["ms_per_step"] * 1e-3)
    return res


def graph_note(gr):
    if not gr:
        return ""
    return (f"; graph replay {gr['ms_per_step']:.3f} ms "
            f"(replays equal eager: {gr['replays_equal_eager_bitwise']})")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-head", action="store_true", help="skip the per-head decay measurement")
    ap.add_argument("--no-l2norm", action="store_true",
                    help="skip the use_qk_l2norm (raw q, k) measurement")
    ap.add_argument("--no-safety", action="store_true",
                    help="skip the numerical-safety options measurement (wy_eps, clip, diag)")
    ap.add_argument("--no-fwd", action="store_true",
                    help="skip the forward-only measurement (profiling runs: one launch name per kernel)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other-dtype and half-batch measurements")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer shards over (batch, head) with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_52_amd as gdn
    import gdn_inputs as gi
    from gated_delta_rule_52_amd.profile import LaunchRecorder

    # the measurement build: the library's kernels and entry points plus the
    # launch recorder that times each launch on its stream
    gdn.use_measurement_build()

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    B, T, H, D, C = args.batch, 4096, 6, 128, 64
    dt = args.dtype
    in_bytes = 2 if dt == "bf16" else 4
    log(f"[bench] workload B={B} T={T} H={H} D={D} dtype={dt}: generating inputs")
    inp = gi.train(dtype=dt, B=B, grads=True)

    def to_device(d):
        out = {}
        for k_, x in d.items():
            if isinstance(x, np.ndarray):
                if x.dtype == np.uint16:
                    out[k_] = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
                else:
                    out[k_] = torch.from_numpy(x).cuda()
        return out

    to = to_device(inp)
    scale = inp["meta"]["scale"]
    q, k, v, g, beta, dO, dhT = (to[n] for n in ("q", "k", "v", "g", "beta", "dO", "dhT"))
    sh = gdn.make_shape(q, v, g, scale, C)
    ws_f = gdn.workspace(sh, False, q.device)
    ws_b = gdn.workspace(sh, True, q.device)
    o = torch.empty_like(v)
    hT = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    gout = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
            torch.empty_like(beta), torch.empty_like(hT))

    def fwd():
        gdn.gdn_forward(q, k, v, g, beta, None, scale=scale, chunk=C, o=o, hT=hT, ws=ws_f)

    def step():
        # training step: the backward reuses the forward's residuals
        gdn.gdn_forward_train(q, k, v, g, beta, None, scale=scale, chunk=C, o=o, hT=hT, ws=ws_b)
        return gdn.gdn_backward_train(q, k, v, g, beta, dO, ws_b, dhT, scale=scale, chunk=C,
                                      out=gout)

    # ---- correctness gate on sampled heads (oracle = token-serial CPU reference)
    import oracle
    log("[bench] correctness gate")
    grads = step()
    torch.cuda.synchronize()
    pairs = [(0, 0), (B // 2 - 1, H // 2), (B // 2, 1), (B - 1, H - 1)]

    def pick(x, b, h):
        return x[b, :, h].float().cpu().numpy().astype(np.float64)

    sub = {n: np.stack([inp[n][b, :, h] for b, h in pairs], axis=1)[None]
           for n in ("q", "k", "v", "g", "beta", "dO")}
    sub["dhT"] = np.stack([inp["dhT"][b, h] for b, h in pairs])[None]
    o_ref, h_ref = oracle.forward(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale)
    g_ref = oracle.backward(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale, sub["dO"],
                            dhT=sub["dhT"])

    def rel(x, y):
        return float(np.max(np.abs(x - y)) / np.max(np.abs(y)))

    par = {"o": rel(np.stack([pick(o, b, h) for b, h in pairs], 1)[None], o_ref),
           "hT": rel(np.stack([hT[b, h].cpu().numpy() for b, h in pairs])[None], h_ref)}
    gn = dict(zip(("dq", "dk", "dv", "dg", "dbeta"), grads[:5]))
    for name, x in gn.items():
        got = np.stack([pick(x, b, h) for b, h in pairs], 1)[None]
        par[name] = rel(got, g_ref[name])
    par["dh0"] = rel(np.stack([grads[5][b, h].cpu().numpy() for b, h in pairs])[None], g_ref["dh0"])
    tol = 2e-2 if dt == "bf16" else 1e-5
    parity_ok = all(e <= tol for e in par.values())
    log(f"[bench] parity (max rel err, tol {tol}): " + ", ".join(f"{k_} {e:.2e}" for k_, e in par.items()))
    checks = {f"fwd+bwd B={B} {dt}": parity_ok}
    parity_gate(checks)  # nothing is timed unless the headline workload is correct

    # ---- fwd+bwd: warmup, then exactly K timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rec = LaunchRecorder(args.steps * 16 + 16)  # room for every launch of the timed steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    with rec:
        for _ in range(args.steps):
            step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    value = B * T / (ms_step * 1e-3)
    per = {name: (float(np.mean(ms)), len(ms)) for name, ms in rec.by_kernel().items()}
    rec.close()
    log(f"[bench] fwd+bwd {ms_step:.3f} ms/step ({value / 1e6:.2f} M tokens/s); wall {wall:.3f} s")
    med_step = median_sync_ms(step)
    log(f"[bench] fwd+bwd median of 20 synchronised calls {med_step:.3f} ms")
    for name, (ms, cnt) in sorted(per.items(), key=lambda x: -x[1][0] * x[1][1]):
        log(f"[bench]   {name:8s} {ms * 1e3:9.1f} us x {cnt // args.steps}/step")

    # dominant kernel by device time per step, and its roofline
    dom = max(per, key=lambda n: per[n][0] * per[n][1])
    roof = roofline(dom, per[dom][0] * 1e-3, B, T, H, C, D, in_bytes)
    roof["traffic"] = measured_traffic(dom) if dt == "bf16" and B == 8 else None
    roof["traffic_over_method_bytes"] = (roof["traffic"] / roof["method_bytes_per_launch"]
                                         if roof["traffic"] else None)
    roof["kernel"] = dom
    roof["avg_launch_us"] = per[dom][0] * 1e3
    roof["launches_timed"] = per[dom][1]
    others = {n: {"us": ms * 1e3, "bound": r["bound"], "frac": r["frac"],
                  "frac_design": r["frac_design"]}
              for n, (ms, _) in per.items()
              for r in [roofline(n, ms * 1e-3, B, T, H, C, D, in_bytes)]}
    log(f"[bench] dominant {dom}: {roof['achieved']:.0f} {roof['unit']} of {roof['peak']:.0f} "
        f"({100 * roof['frac']:.1f}%, {roof['bound']}-bound); traffic {roof['traffic']}")

    # ---- forward only
    ms_fwd = fwd_tps = med_fwd = None
    fwd_kernels = fwd_graph = None
    if not args.no_fwd:
        for _ in range(3):
            fwd()
        torch.cuda.synchronize()
        frec = LaunchRecorder(args.steps * 8 + 8)
        ev0.record()
        with frec:
            for _ in range(args.steps):
                fwd()
        ev1.record()
        torch.cuda.synchronize()
        fwd_kernels = {name: float(np.mean(ms)) * 1e3 for name, ms in frec.by_kernel().items()}
        frec.close()
        ms_fwd = ev0.elapsed_time(ev1) / args.steps
        fwd_tps = B * T / (ms_fwd * 1e-3)
        med_fwd = median_sync_ms(fwd)
        log(f"[bench] fwd {ms_fwd:.3f} ms ({fwd_tps / 1e6:.2f} M tokens/s); median of 20 "
            f"synchronised calls {med_fwd:.3f} ms")
        if not args.no_graph:
            fwd_graph = graph_replay(fwd, (o, hT), args)
            fwd_graph["tokens_per_s"] = B * T / (fwd_graph["ms_per_step"] * 1e-3)
            log(f"[bench] fwd graph replay {fwd_graph['ms_per_step']:.3f} ms "
                f"({fwd_graph['tokens_per_s'] / 1e6:.2f} M tokens/s), replays equal eager: "
                f"{fwd_graph['replays_equal_eager_bitwise']}")

    # ---- the same step captured once in a HIP graph and replayed (the library
    # allocates nothing and issues no memset on this path, so it can be
    # captured; replays remove the launch gaps between the step's kernels)
    graph_res = graph_replay(step, (o, hT) + tuple(gout), args) if not args.no_graph else None
    if graph_res:
        graph_res["tokens_per_s"] = B * T / (graph_res["ms_per_step"] * 1e-3)
        log(f"[bench] graph replay {graph_res['ms_per_step']:.3f} ms/step "
            f"({graph_res['tokens_per_s'] / 1e6:.2f} M tokens/s), replays equal eager: "
            f"{graph_res['replays_equal_eager_bitwise']}")

    # ---- the same layer at the other input dtype and at B/2 (the pages quote
    # their training-shape figures for fp32 and bf16 inputs and for B = 4 and 8)
    def variant(vdt, vB, label):
        vinp = gi.train(dtype=vdt, B=vB, grads=True)
        vd = to_device(vinp)
        vq, vk, vv, vg, vbeta, vdO, vdhT = (vd[n] for n in ("q", "k", "v", "g", "beta", "dO", "dhT"))
        vsh = gdn.make_shape(vq, vv, vg, scale, C)
        vws_f = gdn.workspace(vsh, False, vq.device)
        vws_b = gdn.workspace(vsh, True, vq.device)
        vo = torch.empty_like(vv)
        vhT = torch.empty((vB, H, D, D), dtype=torch.float32, device="cuda")
        vgout = (torch.empty_like(vq), torch.empty_like(vk), torch.empty_like(vv),
                 torch.empty_like(vg), torch.empty_like(vbeta), torch.empty_like(vhT))

        def vstep():
            gdn.gdn_forward_train(vq, vk, vv, vg, vbeta, None, scale=scale, chunk=C, o=vo, hT=vhT,
                                  ws=vws_b)
            return gdn.gdn_backward_train(vq, vk, vv, vg, vbeta, vdO, vws_b, vdhT, scale=scale,
                                          chunk=C, out=vgout)

        def vfwd():
            gdn.gdn_forward(vq, vk, vv, vg, vbeta, None, scale=scale, chunk=C, o=vo, hT=vhT,
                            ws=vws_f)

        vgr = vstep()
        torch.cuda.synchronize()
        vp = [(0, 0), (vB - 1, H - 1)]
        vs = {n: np.stack([vinp[n][b, :, h] for b, h in vp], axis=1)[None]
              for n in ("q", "k", "v", "g", "beta", "dO")}
        vs["dhT"] = np.stack([vinp["dhT"][b, h] for b, h in vp])[None]
        vo_ref, vh_ref = oracle.forward(vs["q"], vs["k"], vs["v"], vs["g"], vs["beta"], scale)
        vg_ref = oracle.backward(vs["q"], vs["k"], vs["v"], vs["g"], vs["beta"], scale, vs["dO"],
                                 dhT=vs["dhT"])
        vpar = {"o": rel(np.stack([pick(vo, b, h) for b, h in vp], 1)[None], vo_ref),
                "hT": rel(np.stack([vhT[b, h].cpu().numpy() for b, h in vp])[None], vh_ref)}
        for name, x in zip(("dq", "dk", "dv", "dg", "dbeta"), vgr[:5]):
            got = np.stack([pick(x, b, h) for b, h in vp], 1)[None]
            vpar[name] = rel(got, vg_ref[name])
        vpar["dh0"] = rel(np.stack([vgr[5][b, h].cpu().numpy() for b, h in vp])[None], vg_ref["dh0"])
        vtol = 2e-2 if vdt == "bf16" else 1e-5
        for _ in range(args.warmup):
            vstep()
        torch.cuda.synchronize()
        vrec = LaunchRecorder(args.steps * 16 + 16)
        ev0.record()
        with vrec:
            for _ in range(args.steps):
                vstep()
        ev1.record()
        torch.cuda.synchronize()
        vms = ev0.elapsed_time(ev1) / args.steps
        vker = {n: float(np.mean(ms)) * 1e3 for n, ms in vrec.by_kernel().items()}
        vrec.close()
        for _ in range(args.warmup):
            vfwd()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            vfwd()
        ev1.record()
        torch.cuda.synchronize()
        vfms = ev0.elapsed_time(ev1) / args.steps
        vgraph = graph_entry(vstep, (vo, vhT) + vgout, args, vB * T)
        vin_bytes = 2 if vdt == "bf16" else 4
        vdom = max(vker, key=vker.get)
        res = {"workload": f"{label}: per-channel decay, B={vB} T={T} H={H} Dk=Dv={D}, chunk {C}, "
                           f"{vdt} q/k/v, fp32 state; eager library calls",
               "fwdbwd_tokens_per_s": vB * T / (vms * 1e-3), "ms_per_step": vms,
               "fwd_tokens_per_s": vB * T / (vfms * 1e-3), "fwd_ms": vfms,
               "graph_replay": vgraph, "kernels_avg_us": vker,
               "dominant_kernel_roofline": dict(roofline(vdom, vker[vdom] * 1e-6, vB, T, H, C, D,
                                                         vin_bytes), kernel=vdom),
               "step_roofline": step_roofline(vms, vB, T, H, C, D, vin_bytes),
               "fwd_roofline": step_roofline(vfms, vB, T, H, C, D, vin_bytes, backward=False),
               "parity_max_rel_err": vpar, "parity_ok": all(e <= vtol for e in vpar.values())}
        log(f"[bench] {label}: fwd+bwd {vms:.3f} ms, fwd {vfms:.3f} ms, parity ok {res['parity_ok']}"
            + graph_note(vgraph))
        del vws_f, vws_b
        return res

    variants = None
    if not args.no_variants:
        other = "f32" if dt == "bf16" else "bf16"
        variants = {other: variant(other, B, f"{other} inputs"),
                    f"B{B // 2}": variant(dt, B // 2, f"B={B // 2}")}
        for key, res in variants.items():
            checks[f"variant {key}"] = res["parity_ok"]

    # ---- per-head decay (one log-decay per token and head) at the same shape
    head = None
    if not args.no_head:
        hinp = gi.train(dtype=dt, B=B, grads=True, decay="head")
        hd = to_device(hinp)
        hg = hd["g"]
        hq, hk, hv, hbeta, hdO, hdhT = (hd[n] for n in ("q", "k", "v", "beta", "dO", "dhT"))

        hgout = (torch.empty_like(hq), torch.empty_like(hk), torch.empty_like(hv),
                 torch.empty_like(hg), torch.empty_like(hbeta), torch.empty_like(hT))

        def hstep():
            gdn.gdn_forward_train(hq, hk, hv, hg, hbeta, None, scale=scale, chunk=C, o=o, hT=hT, ws=ws_b)
            return gdn.gdn_backward_train(hq, hk, hv, hg, hbeta, hdO, ws_b, hdhT, scale=scale,
                                          chunk=C, out=hgout)

        hgr = hstep()
        torch.cuda.synchronize()
        hp = [(0, 0), (B - 1, H - 1)]
        hs = {n: np.stack([hinp[n][b, :, h] for b, h in hp], axis=1)[None]
              for n in ("q", "k", "v", "g", "beta", "dO")}
        hs["dhT"] = np.stack([hinp["dhT"][b, h] for b, h in hp])[None]
        ho_ref, _ = oracle.forward(hs["q"], hs["k"], hs["v"], hs["g"], hs["beta"], scale)
        hg_ref = oracle.backward(hs["q"], hs["k"], hs["v"], hs["g"], hs["beta"], scale, hs["dO"],
                                 dhT=hs["dhT"])
        hpar = {"o": rel(np.stack([pick(o, b, h) for b, h in hp], 1)[None], ho_ref)}
        for name, x in zip(("dq", "dk", "dv", "dg", "dbeta"), hgr[:5]):
            got = (np.stack([x[b, :, h].float().cpu().numpy().astype(np.float64) for b, h in hp], 1)[None])
            hpar[name] = rel(got, hg_ref[name])
        for _ in range(args.warmup):
            hstep()
        torch.cuda.synchronize()
        hrec = LaunchRecorder(args.steps * 16 + 16)
        ev0.record()
        with hrec:
            for _ in range(args.steps):
                hstep()
        ev1.record()
        torch.cuda.synchronize()
        hms = ev0.elapsed_time(ev1) / args.steps
        hker = {n: float(np.mean(ms)) * 1e3 for n, ms in hrec.by_kernel().items()}
        hrec.close()
        ev0.record()
        for _ in range(args.steps):
            gdn.gdn_forward(hq, hk, hv, hg, hbeta, None, scale=scale, chunk=C, o=o, hT=hT, ws=ws_f)
        ev1.record()
        torch.cuda.synchronize()
        hfwd = ev0.elapsed_time(ev1) / args.steps
        hgraph = graph_entry(hstep, (o, hT) + hgout, args, B * T)
        head = {"workload": f"per-head decay (g [B,T,H]), otherwise as above",
                "fwdbwd_tokens_per_s": B * T / (hms * 1e-3), "ms_per_step": hms,
                "graph_replay": hgraph,
                "fwd_tokens_per_s": B * T / (hfwd * 1e-3), "fwd_ms": hfwd,
                "kernels_avg_us": hker, "parity_max_rel_err": hpar,
                "parity_ok": all(e <= tol for e in hpar.values())}
        checks["per-head decay"] = head["parity_ok"]
        log(f"[bench] per-head: fwd+bwd {hms:.3f} ms ({head['fwdbwd_tokens_per_s'] / 1e6:.2f} M tokens/s), "
            f"fwd {hfwd:.3f} ms; parity " + ", ".join(f"{k_} {e:.1e}" for k_, e in hpar.items())
            + graph_note(hgraph))
        log("[bench] per-head kernels: " + ", ".join(f"{n} {u:.0f} us" for n, u in hker.items()))

    # ---- use_qk_l2norm: raw q, k rows normalised inside the layer, same shape
    l2 = None
    if not args.no_l2norm:
        linp = gi.train(dtype=dt, B=B, grads=True, qk_scale=1.0)
        ld = to_device(linp)
        lq, lk, lv, lg, lbeta, ldO, ldhT = (ld[n] for n in ("q", "k", "v", "g", "beta", "dO", "dhT"))
        lsh = gdn.make_shape(lq, lv, lg, scale, C, use_qk_l2norm=True)
        lws_f = gdn.workspace(lsh, False, q.device)
        lws_b = gdn.workspace(lsh, True, q.device)

        def lstep():
            gdn.gdn_forward_train(lq, lk, lv, lg, lbeta, None, scale=scale, chunk=C, o=o, hT=hT,
                                  ws=lws_b, use_qk_l2norm=True)
            return gdn.gdn_backward_train(lq, lk, lv, lg, lbeta, ldO, lws_b, ldhT, scale=scale,
                                          chunk=C, out=gout, use_qk_l2norm=True)

        lgr = lstep()
        torch.cuda.synchronize()
        lp = [(0, 0), (B - 1, H - 1)]
        ls = {n: np.stack([linp[n][b, :, h] for b, h in lp], axis=1)[None]
              for n in ("q", "k", "v", "g", "beta", "dO")}
        ls["dhT"] = np.stack([linp["dhT"][b, h] for b, h in lp])[None]
        lo_ref, _ = oracle.forward(ls["q"], ls["k"], ls["v"], ls["g"], ls["beta"], scale,
                                   qk_l2norm=True)
        lg_ref = oracle.backward(ls["q"], ls["k"], ls["v"], ls["g"], ls["beta"], scale, ls["dO"],
                                 dhT=ls["dhT"], qk_l2norm=True)
        lpar = {"o": rel(np.stack([pick(o, b, h) for b, h in lp], 1)[None], lo_ref)}
        for name, x in zip(("dq", "dk", "dv", "dg", "dbeta"), lgr[:5]):
            got = np.stack([pick(x, b, h) for b, h in lp], 1)[None]
            lpar[name] = rel(got, lg_ref[name])
        for _ in range(args.warmup):
            lstep()
        torch.cuda.synchronize()
        lrec = LaunchRecorder(args.steps * 16 + 16)
        ev0.record()
        with lrec:
            for _ in range(args.steps):
                lstep()
        ev1.record()
        torch.cuda.synchronize()
        lms = ev0.elapsed_time(ev1) / args.steps
        lker = {n: float(np.mean(ms)) * 1e3 for n, ms in lrec.by_kernel().items()}
        lrec.close()
        ev0.record()
        for _ in range(args.steps):
            gdn.gdn_forward(lq, lk, lv, lg, lbeta, None, scale=scale, chunk=C, o=o, hT=hT,
                            ws=lws_f, use_qk_l2norm=True)
        ev1.record()
        torch.cuda.synchronize()
        lfwd = ev0.elapsed_time(ev1) / args.steps
        lroof = roofline("l2norm_bwd", lker["l2norm_bwd"] * 1e-6, B, T, H, C, D, in_bytes)
        lgraph = graph_entry(lstep, (o, hT) + tuple(gout), args, B * T)
        l2 = {"workload": "use_qk_l2norm: raw q, k rows (N(0,1) times a log-normal length per "
                          "row), normalised inside the layer; otherwise as above",
              "fwdbwd_tokens_per_s": B * T / (lms * 1e-3), "ms_per_step": lms,
              "fwd_tokens_per_s": B * T / (lfwd * 1e-3), "fwd_ms": lfwd, "graph_replay": lgraph,
              "kernels_avg_us": lker, "l2norm_bwd_frac_hbm_peak": lroof["frac"],
              "parity_max_rel_err": lpar, "parity_ok": all(e <= tol for e in lpar.values())}
        checks["use_qk_l2norm"] = l2["parity_ok"]
        log(f"[bench] use_qk_l2norm: fwd+bwd {lms:.3f} ms ({l2['fwdbwd_tokens_per_s'] / 1e6:.2f} M tokens/s), "
            f"fwd {lfwd:.3f} ms; parity " + ", ".join(f"{k_} {e:.1e}" for k_, e in lpar.items())
            + graph_note(lgraph))
        log("[bench] use_qk_l2norm kernels: " + ", ".join(f"{n} {u:.0f} us" for n, u in lker.items())
            + f"; l2norm_bwd at {100 * lroof['frac']:.1f}% of HBM peak")

    # ---- numerical-safety options on the main workload: damping, a bound, counters
    safety = None
    if not args.no_safety:
        from oracle import chunked
        sopt = dict(wy_eps=1e-3, clip=1e4, diag=True)
        ssh = gdn.make_shape(q, v, g, scale, C, **sopt)
        sws_b = gdn.workspace(ssh, True, q.device)

        def sstep():
            gdn.gdn_forward_train(q, k, v, g, beta, None, scale=scale, chunk=C, o=o, hT=hT,
                                  ws=sws_b, **sopt)
            return gdn.gdn_backward_train(q, k, v, g, beta, dO, sws_b, dhT, scale=scale, chunk=C,
                                          out=gout, **sopt)

        sstep()
        counts = gdn.gdn_diag_read(ssh, sws_b)
        sp = [(0, 0), (B - 1, H - 1)]
        ss = {n: np.stack([inp[n][b, :, h] for b, h in sp], axis=1)[None]
              for n in ("q", "k", "v", "g", "beta")}
        so_ref, sh_ref = chunked.forward(ss["q"], ss["k"], ss["v"], ss["g"], ss["beta"], scale,
                                         chunk=C, wy_eps=sopt["wy_eps"], clip=sopt["clip"])
        spar = {"o": rel(np.stack([pick(o, b, h) for b, h in sp], 1)[None], so_ref),
                "hT": rel(np.stack([hT[b, h].cpu().numpy() for b, h in sp])[None], sh_ref)}
        for _ in range(args.warmup):
            sstep()
        torch.cuda.synchronize()
        srec = LaunchRecorder(args.steps * 32 + 32)
        ev0.record()
        with srec:
            for _ in range(args.steps):
                sstep()
        ev1.record()
        torch.cuda.synchronize()
        sms = ev0.elapsed_time(ev1) / args.steps
        sker = {n: float(np.mean(ms)) * 1e3 for n, ms in srec.by_kernel().items()}
        scnt = {n: len(ms) // args.steps for n, ms in srec.by_kernel().items()}
        srec.close()
        sgraph = graph_entry(sstep, (o, hT) + tuple(gout), args, B * T)
        safety = {"workload": "main workload with wy_eps=1e-3, clip=1e4, diag on (training pair)",
                  "fwdbwd_tokens_per_s": B * T / (sms * 1e-3), "ms_per_step": sms,
                  "graph_replay": sgraph,
                  "kernels_avg_us": sker, "launches_per_step": scnt, "diag_counts": counts,
                  "parity_max_rel_err_fwd": spar, "parity_ok": all(e <= tol for e in spar.values())}
        checks["safety options"] = safety["parity_ok"]
        log(f"[bench] safety options: fwd+bwd {sms:.3f} ms ({safety['fwdbwd_tokens_per_s'] / 1e6:.2f} M tokens/s); "
            f"fwd parity vs chunked oracle " + ", ".join(f"{k_} {e:.1e}" for k_, e in spar.items())
            + f"; counts {counts}" + graph_note(sgraph))
        log("[bench] safety kernels: " + ", ".join(f"{n} {u:.0f} us x{scnt[n]}" for n, u in sker.items()))

    # ---- decode: B=256 H=16 128x128 fp32 state, one token per step
    decode = None
    if not args.no_decode:
        dinp = gi.decode(steps=8)
        Bd, Hd = 256, 16
        state = torch.from_numpy(dinp["h0"]).cuda()
        steps_in = []
        for t in range(8):
            steps_in.append(tuple(torch.from_numpy(np.ascontiguousarray(dinp[n][:, t])).cuda()
                                  for n in ("q", "k", "v", "g", "beta")))
        od = torch.empty((Bd, 1, Hd, D), dtype=torch.float32, device="cuda")
        o_steps = []
        for t in range(8):
            gdn.gdn_decode_step(*steps_in[t], state, o=od)
            o_steps.append(od.clone())
        torch.cuda.synchronize()
        # correctness: the 8 steps against the oracle's forward over the same 8
        # tokens from the same h0, on sampled (batch, head) pairs
        dp = [(0, 0), (97, 5), (Bd - 1, Hd - 1)]
        dsub = {n: np.stack([dinp[n][b, :, h] for b, h in dp], axis=1)[None]
                for n in ("q", "k", "v", "g", "beta")}
        dh0 = np.stack([dinp["h0"][b, h] for b, h in dp])[None]
        do_ref, dh_ref = oracle.forward(dsub["q"], dsub["k"], dsub["v"], dsub["g"], dsub["beta"],
                                        scale, h0=dh0)
        do_got = np.stack([np.stack([o_steps[t][b, 0, h].cpu().numpy() for t in range(8)])
                           for b, h in dp], axis=1)[None]
        dh_got = np.stack([state[b, h].cpu().numpy() for b, h in dp])[None]
        dpar = {"o": rel(do_got, do_ref), "state": rel(dh_got, dh_ref)}
        checks["decode"] = all(e <= 1e-5 for e in dpar.values())
        log(f"[bench] decode parity after 8 steps: o {dpar['o']:.1e}, state {dpar['state']:.1e}")
        nd = 64
        drec = LaunchRecorder(nd)
        ev0.record()
        with drec:
            for i in range(nd):
                gdn.gdn_decode_step(*steps_in[i % 8], state, o=od)
        ev1.record()
        torch.cuda.synchronize()
        ms_dec = ev0.elapsed_time(ev1) / nd
        kdec = float(np.mean(drec.by_kernel()["decode"]))
        drec.close()
        dbytes = Bd * Hd * (2 * D * D * 4 + 4 * D * 4 + 4) + Bd * Hd * D * 4
        decode = {"workload": "decode step B=256 H=16 Dk=Dv=128, fp32 state, per-channel g",
                  "ms_per_step": ms_dec, "kernel_us": kdec * 1e3,
                  "tokens_per_s": Bd / (ms_dec * 1e-3),
                  "achieved_GBs": dbytes / (kdec * 1e-3) / 1e9,
                  "frac_hbm_peak": dbytes / (kdec * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "algorithmic_bytes_per_step": dbytes,
                  "parity_max_rel_err_8_steps": dpar}
        log(f"[bench] decode {kdec * 1e3:.1f} us/step, {decode['achieved_GBs']:.0f} GB/s")

        # the same decode from a checkpoint plus a buffer of recent tokens: a step
        # reads the checkpoint, the buffer folds into it once per `depth` steps
        s0 = torch.from_numpy(dinp["h0"]).cuda()
        ref_state = s0.clone()
        for t in range(8):
            gdn.gdn_decode_step(*steps_in[t], ref_state, o=od)
        replay = {"workload": "the decode workload above through gdn_replay_step (checkpoint "
                              "read each step; buffer of depth tokens folded in when full)"}
        for depth in (4, 8, 16):
            ck = s0.clone()
            buf = gdn.gdn_replay_buffer(Bd, Hd, D, D, depth)
            for t in range(8):
                gdn.gdn_replay_step(*steps_in[t], ck, buf, depth, o=od)
            gdn.gdn_replay_fold(ck, buf, depth)
            torch.cuda.synchronize()
            agree = float((ck - ref_state).abs().max() / ref_state.abs().max())
            gdn.gdn_replay_fold(ck, buf, depth)
            rrec = LaunchRecorder(nd)
            ev0.record()
            with rrec:
                for i in range(nd):
                    gdn.gdn_replay_step(*steps_in[i % 8], ck, buf, depth, o=od)
            ev1.record()
            torch.cuda.synchronize()
            ms_rep = ev0.elapsed_time(ev1) / nd
            krep = float(np.mean(rrec.by_kernel()["replay_step"]))
            rrec.close()
            # per (b, h) and step, averaged over a fill of the buffer: checkpoint read,
            # its write once per depth steps, the buffer read (on average (depth-1)/2
            # tokens of key, decays and delta) and one token appended, the inputs and o
            tokb = 3 * D * 4
            rbytes = Bd * Hd * (D * D * 4 * (1 + 1 / depth) + (depth - 1) / 2 * tokb + tokb
                                + 4 * D * 4 + 4 + D * 4)
            replay[f"depth{depth}"] = {
                "ms_per_step": ms_rep, "kernel_us": krep * 1e3,
                "tokens_per_s": Bd / (ms_rep * 1e-3),
                "speedup_vs_decode_kernel": kdec / krep,
                "algorithmic_bytes_per_step": rbytes,
                "achieved_GBs": rbytes / (krep * 1e-3) / 1e9,
                "frac_hbm_peak": rbytes / (krep * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "state_rel_diff_vs_decode_after_8": agree}
            checks[f"replay depth {depth}"] = agree <= 1e-5
            log(f"[bench] replay decode depth {depth}: {krep * 1e3:.1f} us/step "
                f"({kdec / krep:.2f}x the decode step), {replay[f'depth{depth}']['achieved_GBs']:.0f} GB/s "
                f"algorithmic; state vs decode {agree:.1e}")
        decode["replay"] = replay

    # ---- CPU oracle on this host: the token-serial reference as it stands
    # (float64, and its float32 instantiation), OpenMP over the (batch, head)
    # sequences, on the same inputs widened exactly from the device's bits;
    # each figure the median of 3 runs
    cpu = None
    if not args.no_cpu:
        nthr = oracle.max_threads()

        def f64(x):
            return np.ascontiguousarray(gi.as_f64(x))

        def med3(fn):
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                fn()
                ts.append(time.perf_counter() - t0)
            return float(np.median(ts))

        s = {n: f64(inp[n]) for n in ("q", "k", "v", "g", "beta", "dO", "dhT")}
        s32 = {n: x.astype(np.float32) for n, x in s.items()}
        log(f"[bench] cpu oracle: B={B} T={T} H={H} fwd and fwd+bwd, float64 and float32, "
            f"{nthr} threads, median of 3")
        t_fwd = med3(lambda: oracle.forward(s["q"], s["k"], s["v"], s["g"], s["beta"], scale))
        t_fb = med3(lambda: (oracle.forward(s["q"], s["k"], s["v"], s["g"], s["beta"], scale),
                             oracle.backward(s["q"], s["k"], s["v"], s["g"], s["beta"], scale,
                                             s["dO"], dhT=s["dhT"])))
        t_fwd32 = med3(lambda: oracle.forward_f32(s32["q"], s32["k"], s32["v"], s32["g"],
                                                  s32["beta"], scale))
        t_fb32 = med3(lambda: (oracle.forward_f32(s32["q"], s32["k"], s32["v"], s32["g"],
                                                  s32["beta"], scale),
                               oracle.backward_f32(s32["q"], s32["k"], s32["v"], s32["g"],
                                                   s32["beta"], scale, s32["dO"], dhT=s32["dhT"])))
        del s, s32
        # decode: 64 consecutive steps of the B=256 H=16 128x128 workload from its
        # h0 (the oracle's forward over the 64 tokens is those 64 steps)
        dci = gi.decode(steps=64)
        sd = {n: f64(dci[n]) for n in ("q", "k", "v", "g", "beta", "h0")}
        t_dec = med3(lambda: oracle.forward(sd["q"], sd["k"], sd["v"], sd["g"], sd["beta"], scale,
                                            h0=sd["h0"]))
        sd32 = {n: x.astype(np.float32) for n, x in sd.items()}
        del sd
        t_dec32 = med3(lambda: oracle.forward_f32(sd32["q"], sd32["k"], sd32["v"], sd32["g"],
                                                  sd32["beta"], scale, h0=sd32["h0"]))
        del sd32, dci
        Bd = 256
        cpu = {"value": B * T / t_fb, "unit": "tokens/s", "cores": nthr, "kind": "oracle",
               "sample": (f"the whole workload: all {B * H} (batch, head) sequences of T={T}, "
                          f"forward + backward (oracle.forward then oracle.backward, which "
                          f"recomputes its states from 64-token checkpoints), float64 "
                          f"token-serial, inputs widened exactly from {dt}; median of 3 runs "
                          f"({t_fb:.2f} s); tokens = B*T"),
               "os_cpu_count": os.cpu_count(), "omp_threads": nthr,
               "fwd_tokens_per_s": B * T / t_fwd,
               "f32_fwdbwd_tokens_per_s": B * T / t_fb32,
               "f32_fwd_tokens_per_s": B * T / t_fwd32,
               "decode_tokens_per_s": Bd * 64 / t_dec,
               "f32_decode_tokens_per_s": Bd * 64 / t_dec32,
               "seconds_median": {"fwdbwd": t_fb, "fwd": t_fwd, "decode64": t_dec,
                                  "f32_fwdbwd": t_fb32, "f32_fwd": t_fwd32, "f32_decode64": t_dec32},
               "decode_sample": "64 steps of B=256 H=16 Dk=Dv=128 per-channel decay from h0 "
                                "(tokens = 256 per step)"}
        log(f"[bench] cpu oracle (float64): fwd+bwd {cpu['value']:.0f} tokens/s, fwd "
            f"{cpu['fwd_tokens_per_s']:.0f}, decode {cpu['decode_tokens_per_s']:.0f}; float32: "
            f"fwd+bwd {cpu['f32_fwdbwd_tokens_per_s']:.0f}, fwd {cpu['f32_fwd_tokens_per_s']:.0f}, "
            f"decode {cpu['f32_decode_tokens_per_s']:.0f}; {nthr} threads of {os.cpu_count()} cpus")

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")
        del src, dst

    # headline: the step as one HIP-graph replay when every check replay
    # reproduced the eager step bitwise, else the eager calls
    use_graph = bool(graph_res and graph_res["replays_equal_eager_bitwise"])
    eager = {"ms_per_step": ms_step, "tokens_per_s": value}
    if use_graph:
        ms_step, value = graph_res["ms_per_step"], graph_res["tokens_per_s"]
    use_fgraph = bool(fwd_graph and fwd_graph["replays_equal_eager_bitwise"])
    fwd_eager = {"ms": ms_fwd, "tokens_per_s": fwd_tps}
    if use_fgraph:
        ms_fwd, fwd_tps = fwd_graph["ms_per_step"], fwd_graph["tokens_per_s"]
    line = {
        "metric": "tokens/s fwd and fwd+bwd at B=8 T=4096 H=6 d=128; % MFMA/HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": value / PAGES_FWDBWD_TOKENS_S if (dt == "bf16" and B == 8) else None,
        "baseline_note": "pages' figure for this workload is TPU v6e (22.44 ms, Sept-2026 "
                         "prototype): context, not a like-for-like target",
        "dtype": dt,
        "data": "synthetic (seeded PCG64; L2-normalised q,k; beta=sigmoid, g=-softplus of N(0,1))",
        "config": {"workload": f"chunked gated delta rule fwd+bwd, per-channel decay, B={B} "
                               f"T={T} H={H} Dk=Dv={D}, chunk {C}, {dt} q/k/v, fp32 state",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": D,
                   "parallelism": "single GPU"},
        "timing": ("one HIP-graph replay of gdn_forward_train + gdn_backward_train per step "
                   "(check replays bitwise equal to the eager calls)") if use_graph
                  else "eager library calls",
        "eager": eager,
        "median_sync_ms": med_step,
        "median_sync_tokens_per_s": B * T / (med_step * 1e-3),
        "step_roofline": step_roofline(ms_step, B, T, H, C, D, in_bytes),
        "fwd_tokens_per_s": fwd_tps,
        "fwd_median_sync_ms": med_fwd,
        "fwd_roofline": step_roofline(ms_fwd, B, T, H, C, D, in_bytes, backward=False) if ms_fwd else None,
        "fwd_ms": ms_fwd,
        "fwd_timing": "HIP-graph replay of gdn_forward" if use_fgraph else "eager gdn_forward",
        "fwd_eager": fwd_eager,
        "fwd_kernels_us": fwd_kernels,
        "graph_replay": graph_res,
        "fwd_graph_replay": fwd_graph,
        "parity_ok": parity_ok,
        "parity_max_rel_err": par,
        "kernels": others,
        "roofline": roof,
        "per_head": head,
        "variants": variants,
        "qk_l2norm": l2,
        "safety_options": safety,
        "decode": decode,
        "cpu_baseline": cpu,
        "parity_checks": checks,
    }
    emit(line, checks)


if __name__ == "__main__":
    main()
