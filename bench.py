"""Benchmark of the SLoPe 2:4 sparse linear layer on one MI355X.

One step is one pass of the whole hot path over the four linears of an OPT-66B
transformer layer (QKV 9216->27648, O 9216->9216, FC1 9216->36864, FC2
36864->9216; T = 8192 tokens, adapter rank 72, bf16 with fp32 accumulation):

    prune_compress24 (magnitude 2:4 prune and compression of W, with W_s
    written as tile chunks, one pass) -> double_prune (straight into W_dp^T's
    tile chunks) -> spmm_fwd (+ fused adapter; also writes X's token
    chunks) -> spmm_bwd_dx (+ the adapter's dX term; also writes dY's token
    chunks) -> masked_wgrad -> lowrank_grads (dL, dR)

The three products run on the packed operands (the *_packed entry points);
the sparse operands' packing is part of the step, and the dense operands'
token chunks come out of the two sparse products (the *_packed_tokens entry
points), which stream those operands anyway; the separate packing pass
(slope_pack_tokens, bitwise the same chunks) can be timed with --profile-op.  A `decode` object adds the
few-token forward (slope_spmm_fwd_decode) at the workload's inference token
counts, as HBM bytes per second, and a `weight_update` object times the optimizer
step (AdamW on the compressed values fused with the double prune, writing both
GEMM operands' tile chunks, and AdamW on the adapter factors), also as HBM
bytes per second, and a `prune_nm` object times the general N:M prune
(slope_prune_nm at 2:8, 1:4 and 2:16) of the layer's dense weights.

The prune and compression run once per layer in training (the forward mask is
static); they are kept inside the timed step so the step covers every row of
the path.  The standalone prune24, compress24 and pack_sparse entry points
compute the same results in three passes (bitwise; tested) and can be timed
with --profile-op.  Inputs are synthetic (seeded Gaussian, see workloads/) and resident in
HBM before the timed region starts.

Prints one JSON line.  `value` is dense-equivalent TFLOP/s of the step's GEMMs
(3 x 2*T*N*K per linear plus the adapter's 2*T*r*(K+N) forward and 4*T*r*(K+N)
backward); `useful_tflops` counts only products with a kept weight (T*N*K per
sparse GEMM) plus the adapter's.  `roofline` reports the
kernel with the largest share of the step against the dense bf16 MFMA peak
(2.5 PFLOP/s) using useful flops.  `layer_roofline_frac` is the step's ideal
time (forward and dX at the 2:4-sparse MFMA peak, the weight gradient's dense
flops at the dense peak) over the measured step; `sparse_products_target`
gives the forward and dX products as fractions of the 2:4-sparse peak.
`graph` replays the same step from a HIP graph (context; `value` stays the
eager step). `configs` runs the GPT-2-small, BERT-Large and OPT-13B layers (and
OPT-13B's few-token forward at T = 16) through the same step, each against its
own ideal, eager and replayed from a graph (the small layers are bound by
launches); `dense_context` times the same twelve GEMMs as dense bf16 products
through torch (context only); `fp8` times the forward and dX products of the
8-bit (E4M3) variant on the same layer (quantizing and packing apart).  `cpu_baseline` times the CPU oracle on a
bounded slice of the same layer on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_DENSE_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_BF16_SPARSE_TFLOPS = 5000.0  # MI355X 2:4-sparse bf16 MFMA, dense-equivalent (published)
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E (published)
# the layer roofline basis: the sparse products' dense-equivalent flops at the
# 2:4-sparse bf16 MFMA rate, the weight gradient's computed dense flops at the
# dense rate (256 CUs x 2.4 GHz x 4096 / 8192 flop per clock and CU)
IDEAL_SPARSE_TFLOPS, IDEAL_DENSE_TFLOPS = 5033.0, 2516.6
METRIC = "2:4 sparse-GEMM TFLOP/s fwd+bwd(dX,dW) +LoRA, % MFMA peak, OPT-66B layer"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="opt_66b")
    ap.add_argument("--tokens", type=int, default=0, help="override T (tokens) of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the context legs (other configs, dense GEMMs, decode, update, N:M prune)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--profile-op", choices=OPS + ("prune24", "compress24", "pack_sparse", "pack_tokens",
                                              "adamw_double_prune", "prune_nm", "decode", "copy"),
                    default=None,
                    help="profiling mode: run only this op (after its inputs are prepared) --repeat times")
    ap.add_argument("--linear", default=None, help="profiling mode: only this linear of the layer (e.g. fc1)")
    ap.add_argument("--repeat", type=int, default=10)
    ap.add_argument("--copy-mib", type=int, default=1024, help="profiling mode 'copy': bytes of a plain device copy")
    return ap.parse_args()


class Linear:
    """Device buffers of one linear of the layer."""

    def __init__(self, name, K, N, T, r, seed, index):
        import numpy as np
        import torch
        from workloads import layer_inputs

        self.name, self.K, self.N, self.T, self.r = name, K, N, T, r
        d = layer_inputs(K, N, T, r, "bf16", seed=seed, index=index)
        dev = "cuda"

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        self.W, self.X, self.dY, self.L, self.R = (up(d[k]) for k in ("W", "X", "dY", "L", "R"))
        del d
        bf = torch.bfloat16
        self.mask = torch.empty((N, K), dtype=torch.uint8, device=dev)
        self.vs = torch.empty((N, K // 2), dtype=bf, device=dev)
        self.ms = torch.empty((N, (K // 4 + 7) // 8), dtype=torch.int32, device=dev)
        self.Y = torch.empty((T, N), dtype=bf, device=dev)
        self.dX = torch.empty((T, K), dtype=bf, device=dev)
        self.dW = torch.empty((N, K // 2), dtype=bf, device=dev)
        import sparse_gemm_02_amd as S
        self.ws = torch.empty(max(16, S.slope_lowrank_workspace_bytes(T, K, r, N)), dtype=torch.uint8, device=dev)
        # sparse operands as tile chunks (W_s for the forward, W_dp^T for dX)
        self.ps = torch.empty(S.slope_packed_sparse_bytes(N, K), dtype=torch.uint8, device=dev)
        self.pd = torch.empty(S.slope_packed_sparse_bytes(K, N), dtype=torch.uint8, device=dev)
        # adapter backward: the dX term's workspace (reduction over N, output over K)
        # and the adapter weight gradients
        self.ws_bwd = torch.empty(max(16, S.slope_lowrank_workspace_bytes(T, N, r, K)), dtype=torch.uint8,
                                  device=dev)
        self.ws_grads = torch.empty(max(16, S.slope_lowrank_grads_workspace_bytes(T, K, r, N)), dtype=torch.uint8,
                                    device=dev)
        self.dL = torch.empty((K, r), dtype=bf, device=dev)
        self.dR = torch.empty((r, N), dtype=bf, device=dev)
        # weight-gradient operands as transposed token chunks
        self.Xp = torch.empty(max(16, S.slope_packed_tokens_bytes(T, K)), dtype=torch.uint8, device=dev)
        self.dYp = torch.empty(max(16, S.slope_packed_tokens_bytes(T, N)), dtype=torch.uint8, device=dev)
        # the weight gradient's token-split partial sums (empty when its tiles fill the device)
        self.wsp = torch.empty(max(16, S.slope_wgrad_split_workspace_bytes(T, N, K)), dtype=torch.uint8, device=dev)

    def flops(self):
        T, N, K, r = self.T, self.N, self.K, self.r
        return {"spmm_fwd": 2 * T * N * K + 2 * T * r * (K + N), "spmm_bwd_dx": 2 * T * N * K + 2 * T * r * (K + N),
                "masked_wgrad": 2 * T * N * K, "lowrank_grads": 2 * T * r * (K + N)}

    def useful(self):
        T, N, K, r = self.T, self.N, self.K, self.r
        return {"spmm_fwd": T * N * K + 2 * T * r * (K + N), "spmm_bwd_dx": T * N * K + 2 * T * r * (K + N),
                "masked_wgrad": T * N * K, "lowrank_grads": 2 * T * r * (K + N)}


# the step's calls; the two sparse products also write X's and dY's token
# chunks (the weight gradient's operands), so no separate packing pass runs
OPS = ("prune_compress24", "double_prune", "spmm_fwd", "spmm_bwd_dx", "masked_wgrad", "lowrank_grads")


def pack_sparse(S, li):
    S.slope_pack_sparse(li.vs, li.ms, li.N, li.K, li.ps)


def prune_compress(S, li):
    S.slope_prune_compress24(li.W, li.vs, li.ms, packed=li.ps)


def double_prune(S, li):
    S.slope_double_prune_packed(li.vs, li.ms, li.N, li.K, li.pd)


def pack(S, li):
    S.slope_pack_tokens(li.X, li.Xp)
    S.slope_pack_tokens(li.dY, li.dYp)


def wgrad(S, li):
    S.slope_masked_wgrad_packed(li.dYp, li.Xp, li.T, li.N, li.K, li.ms, li.dW, split_workspace=li.wsp)


def bwd_dx(S, li):
    S.slope_spmm_bwd_dx_packed(li.dY, li.pd, li.K, li.dX, L=li.L, R=li.R, workspace=li.ws_bwd)


def fwd_tokens(S, li):
    S.slope_spmm_fwd_packed_tokens(li.X, li.ps, li.N, li.Y, li.Xp, L=li.L, R=li.R, workspace=li.ws)


def bwd_dx_tokens(S, li):
    S.slope_spmm_bwd_dx_packed_tokens(li.dY, li.pd, li.K, li.dX, li.dYp, L=li.L, R=li.R, workspace=li.ws_bwd)


def lowrank_grads(S, li):
    # X . L and dY . R^T come from the forward's and the dX product's workspaces
    S.slope_lowrank_grads_packed(li.X, li.dY, li.Xp, li.dYp, li.L, li.R, li.ws_grads, li.dL, li.dR,
                                 fwd_workspace=li.ws, bwd_workspace=li.ws_bwd)


def step(lins, S, ev=None):
    """One pass of the hot path over every linear; optional per-op events."""
    for li in lins:
        calls = (
            ("prune_compress24", lambda: prune_compress(S, li)),
            ("double_prune", lambda: double_prune(S, li)),
            ("spmm_fwd", lambda: fwd_tokens(S, li)),
            ("spmm_bwd_dx", lambda: bwd_dx_tokens(S, li)),
            ("masked_wgrad", lambda: wgrad(S, li)),
            ("lowrank_grads", lambda: lowrank_grads(S, li)),
        )
        for op, fn in calls:
            if ev is not None:
                a, b = ev.pair()
                a.record()
                fn()
                b.record()
                ev.add(li.name, op, a, b)
            else:
                fn()


class Events:
    def __init__(self, torch):
        self.torch = torch
        self.rec = []

    def pair(self):
        E = self.torch.cuda.Event
        return E(enable_timing=True), E(enable_timing=True)

    def add(self, lin, op, a, b):
        self.rec.append((lin, op, a, b))

    def totals(self):
        out = {}
        for lin, op, a, b in self.rec:
            out.setdefault((lin, op), []).append(a.elapsed_time(b))
        return out


def cpu_baseline(workload, budget_s):
    """The CPU oracle on a bounded slice of the layer: for each linear in turn, the
    first 256 output rows (N' = 256) and 256 tokens (T' = 256), running prune24,
    compress24, double_prune (of the slice), forward with adapter, dX and dW, and
    the adapter's backward.
    Repeats over the linears until the budget is spent; rate in dense-equivalent
    TFLOP/s of the slice's GEMMs (the same count as the GPU `value`)."""
    import numpy as np

    import oracle
    from workloads import layer_inputs

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    Tn, Nn = 256, 256
    samples = []
    for i, lin in enumerate(workload.linears):
        d = layer_inputs(lin.K, Nn, Tn, workload.r, "bf16", seed=0, index=100 + i)
        samples.append((lin, d))
    flops, spent, runs = 0.0, 0.0, 0
    t_start = time.perf_counter()
    while spent < budget_s:
        for lin, d in samples:
            K = lin.K
            t0 = time.perf_counter()
            mask, _ = oracle.prune24(d["W"])
            vs, ms, _ = oracle.compress24(d["W"], mask)
            vdp, mdp, _ = oracle.double_prune(vs, ms, Nn, K)
            oracle.spmm_fwd(d["X"], vs, ms, K, d["L"], d["R"])
            oracle.spmm_bwd_dx(d["dY"], vdp, mdp, Nn)
            oracle.masked_wgrad(d["dY"], d["X"], ms, K)
            oracle.lowrank_bwd(d["X"], d["dY"], d["L"], d["R"])
            spent += time.perf_counter() - t0
            flops += 3 * 2 * Tn * Nn * K + 6 * Tn * workload.r * (K + Nn)
            runs += 1
            if spent >= budget_s:
                break
        if time.perf_counter() - t_start > 4 * budget_s:
            break
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{runs} linear slices of N'={Nn} output rows x T'={Tn} tokens (full K) of the "
                      f"{workload.name} layer, whole path (prune, compress, double prune, fwd+adapter, dX, dW, adapter gradients), "
                      f"{spent:.1f} s of CPU work, numpy fp64 with {threads} BLAS threads on {os.cpu_count()} host cores"}


def profile_mode(args, wl, T):
    """Run one op alone (for rocprofv3 counters), or a plain device copy of known size."""
    import torch

    import sparse_gemm_02_amd as S
    if args.profile_op == "copy":
        # a plain device copy of known size: the counters' calibration, and the
        # box's own copy rate (n bytes read, n written) as context for HBM fractions
        n = args.copy_mib * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        b.copy_(a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.repeat):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.repeat
        print(json.dumps({"profile": "copy", "bytes": n, "repeat": args.repeat, "ms": round(ms, 4),
                          "tbs": round(2 * n / (ms * 1e-3) / 1e12, 3)}), flush=True)
        return
    sel = [(i, l) for i, l in enumerate(wl.linears) if args.linear in (None, l.name)]
    lins = [Linear(l.name, l.K, l.N, T, wl.r, seed=0, index=i) for i, l in sel]
    for li in lins:  # prerequisites of every op
        S.slope_prune24(li.W, li.mask)
        prune_compress(S, li)
        double_prune(S, li)
        pack(S, li)
        S.slope_spmm_fwd_packed(li.X, li.ps, li.N, li.Y, L=li.L, R=li.R, workspace=li.ws)
        bwd_dx(S, li)
        wgrad(S, li)
        if args.profile_op == "prune_nm":
            li.Wnm = torch.empty_like(li.W)
        if args.profile_op == "adamw_double_prune":
            li.opt_m = torch.zeros(li.vs.numel(), device="cuda")
            li.opt_v = torch.zeros(li.vs.numel(), device="cuda")
    torch.cuda.synchronize()
    op = args.profile_op
    if op == "decode":   # the few-token forward at the workload's inference token counts
        print(f"[profile] decode {decode_pass(lins, wl, S, torch, reps=args.repeat)}", flush=True)
        return
    for _ in range(args.repeat):
        for li in lins:
            if op == "prune_compress24":
                prune_compress(S, li)
            elif op == "prune24":
                S.slope_prune24(li.W, li.mask)
            elif op == "prune_nm":
                S.slope_prune_nm(li.W, 2, 8, li.mask, li.Wnm)
            elif op == "compress24":
                S.slope_compress24(li.W, li.mask, li.vs, li.ms)
            elif op == "double_prune":
                double_prune(S, li)
            elif op == "pack_sparse":
                pack_sparse(S, li)
            elif op == "spmm_fwd":
                fwd_tokens(S, li)
            elif op == "spmm_bwd_dx":
                bwd_dx_tokens(S, li)
            elif op == "lowrank_grads":
                lowrank_grads(S, li)
            elif op == "pack_tokens":
                pack(S, li)
            elif op == "masked_wgrad":
                wgrad(S, li)
            elif op == "adamw_double_prune":
                S.slope_adamw_double_prune_packed(li.vs, li.ms, li.dW, li.opt_m, li.opt_v, li.N, li.K, li.ps,
                                                  li.pd, 1, lr=1e-4)
    torch.cuda.synchronize()
    print(f"[profile] {op} x {args.repeat} on {[l.name for l in lins]} T={T}", flush=True)


def decode_pass(lins, wl, S, torch, reps=20):
    """The few-token forward (slope_spmm_fwd_decode, adapter on) over the layer's
    linears at each of the workload's inference token counts, on the packed
    weights the step already holds.  HBM bound: reported as algorithmic bytes
    (compressed weight 1.125 B per weight, X, Y, L, R) per second."""
    out = {}
    for T in wl.decode_T:
        calls, nbytes = [], 0
        for li in lins:
            X = torch.randn((T, li.K), device="cuda").to(torch.bfloat16)
            Y = torch.empty((T, li.N), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(max(16, S.slope_decode_workspace_bytes(T, li.K, li.r, li.N)), dtype=torch.uint8,
                             device="cuda")
            calls.append((li, X, Y, ws))
            nbytes += 1.125 * li.N * li.K + 2 * T * (li.K + li.N) + 2 * li.r * (li.K + li.N)
        run = lambda: [S.slope_spmm_fwd_decode(X, li.ps, li.N, Y, ws, L=li.L, R=li.R) for li, X, Y, ws in calls]
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"T={T}"] = {"us_per_layer": round(ms * 1e3, 1), "bytes": int(nbytes), "gbs": round(gbs, 1),
                         "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        del calls
    return out


def prune_nm_pass(lins, S, torch, patterns=((2, 8), (1, 4), (2, 16)), reps=5):
    """General N:M magnitude pruning (slope_prune_nm, mask and W_s written) of
    the layer's dense weights, timed apart from the step (it runs once, at
    initialisation, in place of the 2:4 prune).  HBM bound: 5 B per weight
    (the weight read, one mask byte and W_s written)."""
    big = max(lins, key=lambda li: li.W.numel())
    mask = torch.empty(big.W.numel(), dtype=torch.uint8, device="cuda")
    ws = torch.empty(big.W.numel(), dtype=big.W.dtype, device="cuda")
    nbytes = sum(5 * li.W.numel() for li in lins)
    out = {}
    for n, m in patterns:
        calls = [(li, mask[:li.W.numel()].view(li.W.shape), ws[:li.W.numel()].view(li.W.shape)) for li in lins]
        run = lambda: [S.slope_prune_nm(li.W, n, m, mk, w) for li, mk, w in calls]
        run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"{n}:{m}"] = {"ms_per_layer": round(ms, 4), "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del mask, ws
    return out


def update_pass(lins, S, torch, reps=10):
    """The weight update of a training step, timed apart from the GEMM step:
    AdamW on the compressed values fused with the double prune of the updated
    weight, both GEMM operands written as tile chunks
    (slope_adamw_double_prune_packed) on every linear, plus AdamW on the
    adapter factors L and R (slope_adamw), with fp32 moments.  HBM bound:
    algorithmic bytes are 13.25 B per weight (values, gradient and metadata
    read; values and moments read and written; W_s's packed values and
    W_dp^T's tile chunks written) and 22 B per adapter element."""
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    state, nbytes = [], 0
    for li in lins:
        n = li.vs.numel()
        m = torch.randn(n, device="cuda") * 1e-3
        v = torch.rand(n, device="cuda") * 1e-6
        aL = [torch.zeros(li.L.numel(), device="cuda") for _ in range(2)]
        aR = [torch.zeros(li.R.numel(), device="cuda") for _ in range(2)]
        state.append((li, m, v, aL, aR))
        nbytes += 13.25 * li.N * li.K + 22 * (li.L.numel() + li.R.numel())
    k = [0]

    def run():
        k[0] += 1
        for li, m, v, aL, aR in state:
            S.slope_adamw_double_prune_packed(li.vs, li.ms, li.dW, m, v, li.N, li.K, li.ps, li.pd, k[0], **hp)
            S.slope_adamw(li.L, li.dL, aL[0], aL[1], k[0], **hp)
            S.slope_adamw(li.R, li.dR, aR[0], aR[1], k[0], **hp)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = nbytes / (ms * 1e-3) / 1e9
    del state
    return {"ms_per_layer": round(ms, 4), "bytes": int(nbytes), "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "what": "AdamW on the compressed values fused with the double prune, writing both operands' "
                    "tile chunks (four linears) + AdamW on the adapter factors; fp32 moments"}


PEAK_FP8_SPARSE_TFLOPS = 10000.0   # MI355X 2:4-sparse fp8 MFMA, dense-equivalent (twice the 5.0 PFLOP/s dense fp8)


def fp8_pass(lins, S, torch, reps=10):
    """The 8-bit (E4M3) variant of the sparse products on the same layer: X and
    dY quantized per tensor (slope_quantize_e4m3), W_s and the double-pruned
    W_dp^T turned into E4M3 tile chunks (slope_pack_sparse_e4m3), then the
    forward and dX products (slope_spmm_e4m3_packed, bf16 outputs).  The
    products are reported as dense-equivalent TFLOP/s against the 2:4-sparse
    fp8 peak; quantizing and packing are timed apart (HBM bound)."""
    st = []
    for li in lins:
        vdp = torch.empty((li.K, li.N // 2), dtype=torch.bfloat16, device="cuda")
        mdp = torch.empty((li.K, (li.N // 4 + 7) // 8), dtype=torch.int32, device="cuda")
        S.slope_double_prune(li.vs, li.ms, li.N, li.K, vdp, mdp)
        o = dict(li=li, vdp=vdp, mdp=mdp,
                 xq=torch.empty((li.T, li.K), dtype=torch.uint8, device="cuda"),
                 dyq=torch.empty((li.T, li.N), dtype=torch.uint8, device="cuda"),
                 pw=torch.empty(S.slope_packed_sparse_e4m3_bytes(li.N, li.K), dtype=torch.uint8, device="cuda"),
                 pdp=torch.empty(S.slope_packed_sparse_e4m3_bytes(li.K, li.N), dtype=torch.uint8, device="cuda"),
                 sc=torch.empty(4, dtype=torch.float32, device="cuda"))
        st.append(o)

    def prep():
        for o in st:
            li, sc = o["li"], o["sc"]
            S.slope_quantize_e4m3(li.X, sc[0:1], o["xq"])
            S.slope_quantize_e4m3(li.dY, sc[1:2], o["dyq"])
            S.slope_pack_sparse_e4m3(li.vs, li.ms, li.N, li.K, sc[2:3], o["pw"])
            S.slope_pack_sparse_e4m3(o["vdp"], o["mdp"], li.K, li.N, sc[3:4], o["pdp"])

    def fwd():
        for o in st:
            li, sc = o["li"], o["sc"]
            S.slope_spmm_e4m3_packed(o["xq"], sc[0:1], o["pw"], sc[2:3], li.N, li.Y)

    def dx():
        for o in st:
            li, sc = o["li"], o["sc"]
            S.slope_spmm_e4m3_packed(o["dyq"], sc[1:2], o["pdp"], sc[3:4], li.K, li.dX)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_prep, t_fwd, t_dx = timed(prep), timed(fwd), timed(dx)
    flops = sum(2 * li.T * li.N * li.K for li in lins)
    # algorithmic bytes: each activation read twice (amax, then codes) and its
    # codes written (5 B per element); each compressed weight's values read
    # twice, its metadata read and its chunks written (2.75 B per dense weight)
    prep_bytes = sum(5 * li.T * (li.K + li.N) + 2 * 2.75 * li.N * li.K for li in lins)
    out = {"what": "E4M3 (OCP fp8) operands, per-tensor amax scales, bf16 outputs; the 2:4 pattern of the bf16 layer",
           "quantize_and_pack": {"ms_per_step": round(t_prep, 4),
                                 "gbs": round(prep_bytes / (t_prep * 1e-3) / 1e9, 1)}}
    for k, t in (("spmm_fwd", t_fwd), ("spmm_bwd_dx", t_dx)):
        de = flops / (t * 1e-3) / 1e12
        out[k] = {"ms_per_step": round(t, 4), "dense_equiv_tflops": round(de, 2),
                  "frac_fp8_sparse_peak": round(de / PEAK_FP8_SPARSE_TFLOPS, 4),
                  "speedup_vs_bf16": None}
    del st
    torch.cuda.empty_cache()
    return out


def measured_traffic(op):
    """HBM bytes per launch (fetched + written) of `op`'s kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when the kernel source has
    changed since the counters were taken (or none were taken)."""
    import hashlib
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[op]
        src = open(os.path.join(ROOT, t["kernel_source"]), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != t["source_sha256_16"]:
        return None
    return {"fetch_bytes_per_launch": t["fetch_bytes_per_launch"], "write_bytes_per_launch": t["write_bytes_per_launch"],
            "bytes_per_launch": t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"],
            "source": "profiles/traffic.json (rocprofv3 FETCH_SIZE x2.0, WRITE_SIZE x1.0 by copy calibration)"}


def ideal_step_ms(wl, T):
    """Ideal time of one layer step on the layer roofline basis: forward and dX
    at the 2:4-sparse MFMA rate (dense-equivalent 2*T*N*K each), the weight
    gradient at the dense rate (2*T*N*K computed); adapter and pruning excluded."""
    f = sum(2 * T * l.N * l.K for l in wl.linears)
    return (2 * f / (IDEAL_SPARSE_TFLOPS * 1e12) + f / (IDEAL_DENSE_TFLOPS * 1e12)) * 1e3


def time_steps(lins, S, torch, steps, warmup):
    """ms per whole step (no per-op events), after `warmup` untimed steps."""
    for _ in range(warmup):
        step(lins, S)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step(lins, S)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_steps_graph(lins, S, torch, steps, warmup):
    """ms per whole step replayed from a HIP graph (torch.cuda.CUDAGraph over
    the same library calls): eager warm-up steps first (every kernel attribute
    set, every plan made outside the capture), one step captured, `warmup`
    replays untimed, `steps` replays timed.  The library records no memset and
    allocates nothing, so a step captures as it runs."""
    for _ in range(max(1, warmup)):
        step(lins, S)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(lins, S)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(lins, S)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) / steps


def configs_pass(args, S, torch, WORKLOADS, steps=5, warmup=2):
    """The other training configurations (GPT-2-small, BERT-Large, OPT-13B) through
    the same step, each against its own layer roofline, and OPT-13B's few-token
    forward at T = 16 (HBM bound) against its compressed-weight bytes."""
    out = {}
    for name in ("gpt2_small", "bert_large", "opt_13b"):
        wl = WORKLOADS[name]
        lins = [Linear(l.name, l.K, l.N, wl.T, wl.r, seed=0, index=i) for i, l in enumerate(wl.linears)]
        ms = time_steps(lins, S, torch, steps, warmup)
        ms_g = time_steps_graph(lins, S, torch, steps, warmup)
        flops = sum(sum(l.flops().values()) for l in lins)
        ideal = ideal_step_ms(wl, wl.T)
        out[name] = {"tokens": wl.T, "adapter_rank": wl.r, "ms_per_step": round(ms, 4),
                     "dense_equiv_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "ideal_step_ms": round(ideal, 4), "layer_roofline_frac": round(ideal / ms, 4),
                     "ms_per_step_graph": round(ms_g, 4), "layer_roofline_frac_graph": round(ideal / ms_g, 4)}
        if wl.decode_T:
            for T, v in decode_pass(lins, wl, S, torch).items():
                ideal_us = v["bytes"] / (PEAK_HBM_GBS * 1e9) * 1e6
                out[f"{name}_decode_{T}"] = dict(v, ideal_us=round(ideal_us, 1))
        del lins
        torch.cuda.empty_cache()
        print(f"[bench] config {name} done", file=sys.stderr, flush=True)
    return out


def dense_context(lins, torch, reps=5):
    """Context only: the same twelve GEMMs as dense bf16 products through
    torch (hipBLASLt): Y = X W^T, dX = dY W, dW = dY^T X on the dense weights,
    fp32 accumulation, timed with events.  The analogue of the pages' sparse vs
    dense timing; not a target."""
    out, tot = {}, {"fwd": 0.0, "dx": 0.0, "dw": 0.0}
    for li in lins:
        Y = torch.empty((li.T, li.N), dtype=torch.bfloat16, device="cuda")
        dX = torch.empty((li.T, li.K), dtype=torch.bfloat16, device="cuda")
        dW = torch.empty((li.N, li.K), dtype=torch.bfloat16, device="cuda")
        calls = {"fwd": lambda: torch.mm(li.X, li.W.t(), out=Y), "dx": lambda: torch.mm(li.dY, li.W, out=dX),
                 "dw": lambda: torch.mm(li.dY.t(), li.X, out=dW)}
        for k, fn in calls.items():
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            tot[k] += a.elapsed_time(b) / reps
        del Y, dX, dW
    flops = sum(2 * li.T * li.N * li.K for li in lins)
    for k, v in tot.items():
        out[k] = {"ms_per_step": round(v, 4), "tflops": round(flops / (v * 1e-3) / 1e12, 2)}
    out["total_ms"] = round(sum(tot.values()), 4)
    out["what"] = "torch.mm bf16 (hipBLASLt) on the dense weights, the same 12 GEMMs; context, not a target"
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the 2:4 layer kernels are "
              "measured on a single MI355X; multi-GPU sharding is a design note, not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_gemm_02_amd as S
    from workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    T = args.tokens or wl.T
    torch.cuda.set_device(0)
    S.library()
    if args.profile_op:
        profile_mode(args, wl, T)
        return
    t_in = time.perf_counter()
    lins = [Linear(l.name, l.K, l.N, T, wl.r, seed=0, index=i) for i, l in enumerate(wl.linears)]
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_in:.1f}s: {args.workload} T={T} r={wl.r}",
          file=sys.stderr, flush=True)

    # timed region: whole steps, no per-op events
    ms_step = time_steps(lins, S, torch, args.steps, args.warmup)

    # the same steps again with an event pair around every call (per-op durations)
    ev = Events(torch)
    for _ in range(args.steps):
        step(lins, S, ev)
    torch.cuda.synchronize()
    per = ev.totals()

    dense_flops = sum(sum(l.flops().values()) for l in lins)
    useful_flops = sum(sum(l.useful().values()) for l in lins)
    value = dense_flops / (ms_step * 1e-3) / 1e12
    useful = useful_flops / (ms_step * 1e-3) / 1e12

    # per-op summary over the linears
    ops = {}
    for op in OPS:
        t = sum(sum(per[(l.name, op)]) / len(per[(l.name, op)]) for l in lins)
        ops[op] = {"ms_per_step": t}
    for op in ("spmm_fwd", "spmm_bwd_dx", "masked_wgrad", "lowrank_grads"):
        uf = sum(l.useful()[op] for l in lins)
        df = sum(l.flops()[op] for l in lins)
        t = ops[op]["ms_per_step"] * 1e-3
        ops[op].update(useful_tflops=uf / t / 1e12, dense_equiv_tflops=df / t / 1e12,
                       frac_dense_peak_useful=uf / t / 1e12 / PEAK_BF16_DENSE_TFLOPS)
        if op in ("spmm_fwd", "spmm_bwd_dx"):
            # the sparse products against the dense bf16 MFMA peak (dense-equivalent
            # flops, what a dense GEMM of the same shape would need) and against the
            # 2:4-sparse MFMA peak
            ops[op].update(frac_dense_peak_dense_equiv=df / t / 1e12 / PEAK_BF16_DENSE_TFLOPS,
                           frac_sparse_peak=df / t / 1e12 / PEAK_BF16_SPARSE_TFLOPS)
    # algorithmic HBM bytes per weight for the pruning ops
    # (prune_compress24: W read, values + metadata + W_s's tile chunks written)
    hbm = {"prune_compress24": lambda l: 4.25 * l.N * l.K, "double_prune": lambda l: 2.25 * l.N * l.K}
    for op, f in hbm.items():
        by = sum(f(l) for l in lins)
        ops[op]["gbs"] = by / (ops[op]["ms_per_step"] * 1e-3) / 1e9
        ops[op]["frac_hbm_peak"] = ops[op]["gbs"] / PEAK_HBM_GBS

    # dominant kernel: the weight-gradient GEMM (its call is the GEMM kernel plus,
    # where the tiles end in a partly filled round of blocks, a small kernel
    # adding that round's token ranges: a few microseconds of the call; the two
    # sparse products also launch the adapter's small kernels, so their call
    # time is not one kernel's)
    dom = "masked_wgrad"
    launches = [(l, sum(per[(l.name, dom)]) / len(per[(l.name, dom)])) for l in lins]
    achieved = sum(l.useful()[dom] for l, _ in launches) / (sum(t for _, t in launches) * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_DENSE_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_DENSE_TFLOPS, 4),
                "traffic": measured_traffic(dom),
                "flops_counted": "useful (T*N*K per launch: products with a kept weight / kept output)",
                "kernels": "wgrad_direct_kernel (+ wgrad_tail_reduce_kernel for the last round's token ranges)",
                "avg_launch_ms": {l.name: round(t, 4) for l, t in launches}}

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{wl.name} layer: " + ", ".join(f"{l.name} {l.K}->{l.N}" for l in wl.linears)
                      + f"; T={T} tokens; adapter rank {wl.r}; whole path per step",
                      "tokens": T, "adapter_rank": wl.r},
           "value_kind": "dense-equivalent TFLOP/s (2*T*N*K per GEMM)",
           "useful_tflops": round(useful, 2),
           "frac_dense_peak_useful": round(useful / PEAK_BF16_DENSE_TFLOPS, 4),
           "ideal_step_ms": round(ideal_step_ms(wl, T), 3),
           "layer_roofline_frac": round(ideal_step_ms(wl, T) / ms_step, 4),
           "ideal_basis": "fwd and dX dense-equivalent flops at the 2:4-sparse MFMA peak (5.03 PFLOP/s), dW's computed "
                          "dense flops at the dense peak (2.52 PFLOP/s); adapter and pruning excluded",
           "sparse_products_target": {
               "what": "sparse fwd and dX, dense-equivalent TFLOP/s over the 2:4-sparse bf16 MFMA peak (5.0 PFLOP/s); "
                       "target >= 0.5",
               "spmm_fwd": round(ops["spmm_fwd"]["frac_sparse_peak"], 4),
               "spmm_bwd_dx": round(ops["spmm_bwd_dx"]["frac_sparse_peak"], 4)},
           "ops": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in ops.items()},
           "roofline": roofline}
    if not args.no_extras:
        ms_graph = time_steps_graph(lins, S, torch, args.steps, args.warmup)
        out["graph"] = {"ms_per_step": round(ms_graph, 4),
                        "what": "the same step replayed from a HIP graph (torch.cuda.CUDAGraph over the library's "
                                "calls); context: value is the eager step"}
        if wl.decode_T:
            out["decode"] = decode_pass(lins, wl, S, torch)
        out["weight_update"] = update_pass(lins, S, torch)
        out["prune_nm"] = prune_nm_pass(lins, S, torch)
        out["dense_context"] = dense_context(lins, torch)
        out["fp8"] = fp8_pass(lins, S, torch)
        for k in ("spmm_fwd", "spmm_bwd_dx"):
            out["fp8"][k]["speedup_vs_bf16"] = round(ops[k]["ms_per_step"] / out["fp8"][k]["ms_per_step"], 3)
    # free the layer before the other configs and the CPU leg
    del lins
    torch.cuda.empty_cache()
    if not args.no_extras and not args.tokens and args.workload == "opt_66b":
        out["configs"] = configs_pass(args, S, torch, WORKLOADS)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
