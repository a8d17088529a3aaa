"""Benchmark of the multi-probe SPSA step on one MI355X.

Default workload: the OPT-30B-shaped decoder (48 layers, d = 7168, 56 heads,
FFN 28672, vocabulary 50272, bf16 random-init weights, 59.94 GB held in place
in HBM), batch 8 x seq 2048 Zipf(1.1) tokens, causal-LM loss, one SPSA pair
per step (N = 1, +-eps) in place: perturb +eps, L+, perturb -2 eps, L-,
perturb +eps, then the fused update -- the in-place, inference-mode OPT-30B
training step of the ZOO blog ("backprop의 메모리 세금": batch 8, sequence
2048, about 60 GB).  Other workloads: --workload mlp | lsq | gpt | opt1.3b.

Prints one JSON line: probe-evals/s of the whole step, the dominant kernel's
roofline (live HIP-event timing of its launches, and only its, over the timed
region), a per-kernel table from a second instrumented pass, the step's own
perturb / update passes in GB/s, the same passes on a 1.3e9-element buffer
(the OPT-1.3B-shaped count), and the CPU oracle timed on a bounded sample.
Every timed loss must be finite, else the run fails.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SPSA probe-evals/sec per model + perturb/update HBM GB/s (frac. of peak)"
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3
BF16_PEAK_TFLOPS = 2500.0
# VALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz non-packed 32-bit lane operations per second
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
# VALU instructions per generated Gaussian (Philox4x32-10 quarter plus half a
# Box-Muller pair): the perturb_bf16 loop issues 237 per 8 elements including
# its fma, conversions and address arithmetic
C_Z = 29.6
# HBM bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE /
# WRITE_SIZE, scaled by the same counters on a plain copy of known size
# (factors 2.00 / 1.00); see profiles/.  Keyed by the kernel revision they were
# taken on -- set to None when that kernel changes.
TRAFFIC = {
    "sgemm:mlp:r5": 2 * 8486.5 * 1024 + 10240 * 1024,
    # the OPT-30B shape's four layer GEMMs (QKV, O, up, down) with the decoder's
    # epilogues (store, residual, ReLU, residual), mean per launch: FETCH_SIZE x 2
    # + WRITE_SIZE summed over one of each, divided by four
    "gemm_bf16:opt30b:r9": (2 * (3.8064 + 1.3169 + 4.9894 + 4.9289) + (0.6565 + 0.2189 + 0.8760 + 0.2189))
                           * 2**30 / 4,
}
KERNEL_REV = {"mlp": "sgemm:mlp:r5", "lsq": None, "opt30b": "gemm_bf16:opt30b:r9"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="opt30b", choices=["mlp", "lsq", "gpt", "opt1.3b", "opt30b"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-passes", action="store_true", help="skip the perturb/update pass measurement")
    p.add_argument("--precond", action="store_true",
                   help="1.5-SPSA: one clean evaluation per step and probe-space preconditioning")
    p.add_argument("--curv-floor", type=float, default=1.0, help="1.5-SPSA curvature floor")
    p.add_argument("--split", default=None, metavar="P1,PS",
                   help="MLP: split-perturbation (FedSPZO) steps with P1 theta_1 directions and PS theta_2 "
                        "directions per branch instead of SPSA steps")
    p.add_argument("--dust", default=None, metavar="K1,K2",
                   help="MLP: Dust steps (activation noise) with K1 hidden-layer and K2 head draws")
    p.add_argument("--mode", default=None, choices=["inplace", "fused", "copies"],
                   help="step mode (default: copies for the GPT-small shape, in place for the OPT shapes, "
                        "fused for the fp32 models)")
    p.add_argument("--dirs", default="gauss", choices=["gauss", "q8"],
                   help="direction distribution: Gaussian, or 8-bit packed (in-place decoder workloads)")
    p.add_argument("--gemm", default=None, metavar="M,N,K",
                   help="instead of a step: time one stored-weight bf16 GEMM C = A W^T of this shape "
                        "(--steps calls after --warmup), for kernel measurements")
    p.add_argument("--gemm-epi", type=int, default=0, choices=[0, 1, 2, 3],
                   help="the --gemm epilogue: 0 store, 1 GELU, 2 ReLU, 3 residual (C += product)")
    p.add_argument("--attention", default=None, metavar="B,S,H,DH",
                   help="instead of a step: time the decoders' causal attention kernel on a bf16 QKV of this "
                        "shape (--steps calls after --warmup), for kernel measurements")
    return p.parse_args()


def build_mlp(torch, zo, inputs):
    import numpy as np
    B, D, H, C = 256, 1024, 4096, 10
    inp = inputs.mlp_inputs(0, batch=B, d_in=D, hidden=H, classes=C)
    desc = zo.make_desc(zo.ZO_MODEL_MLP, batch=B, d_in=D, hidden=H, classes=C)
    layout, total = zo.param_layout(desc)
    arena = np.zeros(total, np.float32)
    for name, off, shape in layout:
        arena[off:off + int(np.prod(shape))] = inp[name].ravel()
    model = zo.Model(desc, torch.from_numpy(arena).cuda())
    x = torch.from_numpy(inp["X"]).cuda()
    lab = torch.from_numpy(inp["labels"]).cuda()
    batch = zo.make_batch(x=x, labels=lab, batch=B)
    info = {
        "workload": "2-layer MLP classifier fp32 1024->4096(GELU)->10, batch 256, cross-entropy; "
                    "N=16 probes, eps=1e-3, lr=1e-3; perturbed-tile (fused) mode",
        "probes": 16, "eps": 1e-3, "lr": 1e-3, "mode": "fused", "batch": B, "hidden": H,
        "params": int(total),
        # algorithmic flops of one evaluation: X W1^T and H W2^T
        "flops_per_eval": 2.0 * B * D * H + 2.0 * B * H * C,
        # the dominant kernel forms X Z_i^T for each probe direction (fp32
        # through six bf16 MFMA products) and generates Z_i (and W2's part)
        "split_bf16": {"direction_flops": 2.0 * B * D * H, "gaussians": H * D + C * H, "w1_gaussians": H * D,
                       "w2_gaussians": C * H},
        "dtype": "f32", "kernel": "gemm_f32", "peak_tflops": BF16_PEAK_TFLOPS,
        "oracle_desc": {"kind": "mlp", "batch": B, "d_in": D, "hidden": H, "classes": C},
        "oracle_batch": {"X": inp["X"], "labels": inp["labels"]}, "arena": arena,
    }
    return model, batch, (x, lab), info


def build_lsq(torch, zo, inputs):
    import numpy as np
    n, D, O = 512, 256, 256
    inp = inputs.lsq_inputs(0, n=n, d_in=D, d_out=O)
    desc = zo.make_desc(zo.ZO_MODEL_LSQ, batch=n, d_in=D, d_out=O)
    _, total = zo.param_layout(desc)
    arena = inp["W"].ravel().copy()
    model = zo.Model(desc, torch.from_numpy(arena).cuda())
    x = torch.from_numpy(inp["X"]).cuda()
    y = torch.from_numpy(inp["Y"]).cuda()
    batch = zo.make_batch(x=x, y=y, batch=n)
    info = {
        "workload": "least squares fp32 W 256x256, X 512x256, MSE/2; N=4 probes, eps=1e-3, lr=1e-2; fused mode",
        "probes": 4, "eps": 1e-3, "lr": 1e-2, "mode": "fused", "batch": n, "params": int(total),
        "flops_per_eval": 2.0 * n * D * O, "dtype": "f32", "kernel": "gemm_f32", "peak_tflops": FP32_PEAK_TFLOPS,
        "oracle_desc": {"kind": "lsq", "n": n, "d_in": D, "d_out": O},
        "oracle_batch": {"X": inp["X"], "Y": inp["Y"]}, "arena": arena,
    }
    return model, batch, (x, y), info


DECODERS = {
    # name: layers, d, heads, ffn, vocab, batch, seq, act, probes, lr
    # lr (the configs give none for the decoders): sized so that one step's
    # weight change stays about 1e-3 of the weights' norm,
    # ||dW|| / ||W|| ~ lr ||grad L|| / (0.02 sqrt(N)) with ||grad L|| ~ 10 at
    # initialisation (the measured spread of g_i), i.e. lr ~ 2e-6 sqrt(N)
    "gpt": (12, 768, 12, 3072, 32000, 8, 512, "gelu", 32, 1e-5),
    "opt1.3b": (24, 2048, 32, 8192, 50272, 8, 2048, "relu", 1, 1e-6),
    "opt30b": (48, 7168, 56, 28672, 50272, 8, 2048, "relu", 1, 1e-6),
}


def build_decoder(torch, zo, inputs, name, dirs="gauss"):
    L, D, H, F, V, B, S, act, N, lr = DECODERS[name]
    desc = zo.make_desc(zo.ZO_MODEL_DECODER, batch=B, seq=S, layers=L, d_model=D, heads=H, ffn=F, vocab=V,
                        max_seq=S, act=zo.ZO_ACT_GELU if act == "gelu" else zo.ZO_ACT_RELU,
                        dirs=zo.ZO_DIRS_Q8 if dirs == "q8" else zo.ZO_DIRS_GAUSS)
    layout, total = zo.param_layout(desc)
    arena = torch.empty(total, dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    for pname, off, shape in layout:
        n = 1
        for x in shape:
            n *= x
        view = arena[off:off + n]
        if pname.endswith("_g"):
            view.fill_(1.0)
        elif pname.endswith("_b"):
            view.zero_()
        else:
            view.normal_(0.0, 0.02, generator=gen)
    model = zo.Model(desc, arena)
    tok = torch.from_numpy(inputs.zipf_tokens(0, B, S, V)).cuda()
    batch = zo.make_batch(tokens=tok, batch=B, seq=S)
    M = B * S
    # default mode: in place for the large shapes (the memory the pages
    # save), copies for the GPT-small shape (its 64 evaluations of 4096 rows
    # run 8 side by side; 2 GB of copies)
    mode = "copies" if name == "gpt" else "inplace"
    gemm_flops = L * (2.0 * M * D * 3 * D + 2.0 * M * D * D + 2 * 2.0 * M * D * F)
    attn_flops = L * 2.0 * B * H * S * S * (D // H)  # causal half of 4 B H S^2 dh
    head_flops = 2.0 * M * D * V
    info = {
        "workload": f"decoder {name}: {L} layers, d={D}, {H} heads, FFN {F}, vocab {V}, bf16 "
                    f"({total * 2 / 1e9:.2f} GB of weights); batch {B} x seq {S} "
                    f"Zipf(1.1) tokens; N={N} probes, eps=1e-3, lr={lr:g}; " + (
                        "copies mode (D(W +- eps z_i) written to arena copies, evaluated side by side)"
                        if mode == "copies" else "in-place mode"),
        "probes": N, "eps": 1e-3, "lr": lr, "mode": mode, "batch": B, "params": int(total),
        "flops_per_eval": gemm_flops + attn_flops + head_flops, "gemm_flops_per_eval": gemm_flops,
        "head_flops_per_eval": head_flops, "attn_flops_per_eval": attn_flops,
        # per layer GEMM (timing sub-families gemm_bf16.<name>), all layers
        "gemm_parts_flops_per_eval": {"qkv": L * 2.0 * M * D * 3 * D, "o": L * 2.0 * M * D * D,
                                      "up": L * 2.0 * M * D * F, "down": L * 2.0 * M * F * D},
        "dtype": "bf16", "kernel": "gemm_bf16", "peak_tflops": BF16_PEAK_TFLOPS,
        "decoder_shape": {"layers": L, "d": D, "heads": H, "ffn": F, "vocab": V, "act": act, "batch": B, "seq": S},
    }
    return model, batch, (tok,), info


def valu_fields(fam, gaussians, seconds):
    """The Gaussian passes are VALU-bound.  The perturbation loop's count of
    c_z instructions per Gaussian prices it against the VALU peak; the update
    loops share their loads, stores and addressing between N directions, so
    for them the line gives the instructions per Gaussian the measured rate
    would leave at the VALU peak."""
    rate = gaussians / seconds
    if fam == "perturb":
        return {"frac_valu_peak_generation": round(rate * C_Z / VALU_PEAK_LANE_OPS, 4), "c_z": C_Z}
    return {"valu_instr_per_gaussian_at_peak": round(VALU_PEAK_LANE_OPS / rate, 2)}


def measure_passes(torch, zo):
    """Perturb and update passes over an OPT-1.3B-sized parameter count, with
    Gaussian and with 8-bit packed directions; the update also at N = 32."""
    n = 1_315_311_616
    out = {}
    for name, dtype, tdt, esz in (("bf16", zo.ZO_BF16, torch.bfloat16, 2), ("f32", zo.ZO_F32, torch.float32, 4)):
        w = torch.zeros(n, dtype=tdt, device="cuda")
        g = torch.ones(32, dtype=torch.float64, device="cuda")
        # plain copy of the same size: the HBM reference for these passes
        c = torch.empty_like(w)
        c.copy_(w)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for r in range(5):
            c.copy_(w)
        ev1.record()
        torch.cuda.synchronize()
        tc = ev0.elapsed_time(ev1) / 5 * 1e-3
        out[f"copy_{name}"] = {"GB/s": round(2.0 * n * esz / tc / 1e9, 1), "ms": round(tc * 1e3, 4),
                               "elements": n, "kind": "torch copy_, reference"}
        del c
        for dirs, suffix in ((zo.ZO_DIRS_GAUSS, ""), (zo.ZO_DIRS_Q8, "_q8")):
            zo.perturb_buffer(w, n, 0, 1, 0, 1e-3, dtype, dirs=dirs)
            zo.update_buffer(w, n, 0, 1, 1, g, 1e-3, dtype, dirs=dirs)
            torch.cuda.synchronize()
            zo.timing_reset()
            zo.timing_enable(True)
            for r in range(5):
                zo.perturb_buffer(w, n, 0, 1, r, 1e-3, dtype, dirs=dirs)
                zo.update_buffer(w, n, 0, 1, 1, g, 1e-3, dtype, dirs=dirs)
            torch.cuda.synchronize()
            zo.timing_enable(False)
            for fam in ("perturb", "update"):
                ms, k = zo.timing_query(fam)
                t = ms / k * 1e-3
                gbs = 2.0 * n * esz / t / 1e9
                out[f"{fam}_{name}{suffix}"] = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                                                "frac_copy": round(gbs / out[f"copy_{name}"]["GB/s"], 4),
                                                "ms": round(t * 1e3, 4), "elements": n, "probes": 1}
                if dirs == zo.ZO_DIRS_GAUSS:
                    out[f"{fam}_{name}{suffix}"].update(valu_fields(fam, n, t))
            # many probes: the update regenerates N directions per element
            zo.timing_reset()
            zo.timing_enable(True)
            for r in range(2):
                zo.update_buffer(w, n, 0, 1, 32, g, 1e-9, dtype, dirs=dirs)
            torch.cuda.synchronize()
            zo.timing_enable(False)
            ms, k = zo.timing_query("update")
            t = ms / k * 1e-3
            out[f"update_{name}{suffix}_N32"] = {"directions_per_s": round(32 * n / t, 1), "ms": round(t * 1e3, 3),
                                                 "elements": n, "probes": 32}
            if dirs == zo.ZO_DIRS_GAUSS:
                out[f"update_{name}{suffix}_N32"].update(valu_fields("update", 32 * n, t))
            zo.timing_reset()
        del w
        torch.cuda.empty_cache()
    return out


def _oracle_probe_worker(job):
    """One host core: single-probe oracle steps of the workload for a fixed
    time; returns (steps, seconds)."""
    desc, arena, batch, eps, lr, seed0, seconds = job
    from threadpoolctl import threadpool_limits

    from oracle import oracle
    a = oracle.Arena(desc, arena.copy())
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < seconds:
            oracle.spsa_step(a, batch, seed=seed0 + reps, n_probes=1, eps=eps, lr=lr, mode="fused")
            reps += 1
        return reps, time.perf_counter() - t0


def cpu_baseline_probe_parallel(info, seconds=8.0):
    """Probes are independent: one single-threaded oracle process per host
    core (at most 16), each evaluating its own probe's pair and update."""
    import multiprocessing
    procs = max(1, min(16, os.cpu_count() or 1))
    jobs = [(info["oracle_desc"], info["arena"], info["oracle_batch"], info["eps"], info["lr"], 1000 * i, seconds)
            for i in range(procs)]
    with multiprocessing.get_context("spawn").Pool(procs) as pool:
        res = pool.map(_oracle_probe_worker, jobs)
    rate = sum(2 * r / t for r, t in res)
    return {"value": round(rate, 3), "unit": "probe-evals/s", "cores": procs, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{procs} processes x {seconds:.0f} s of single-probe oracle steps "
                      f"({sum(r for r, _ in res)} steps in all)"}


def gemm_only(torch, zo, shape, steps, warmup, epi=0):
    """One layer GEMM of the decoders, C = epi(A W^T) in bf16 (fp32 accumulate;
    epilogue 0 plain store, 1 GELU, 2 ReLU, 3 residual), through the C ABI's
    debug entry; prints its time and rate."""
    M, N, K = shape
    g = torch.Generator(device="cuda").manual_seed(0)
    A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
    W = (torch.randn(N, K, device="cuda", generator=g) * 0.05).to(torch.bfloat16).view(torch.int16)
    C = torch.zeros(M * N, dtype=torch.int16, device="cuda")
    for _ in range(max(warmup, 1)):
        zo.debug_gemm_bf16(A, W, C, M, N, K, epi)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        zo.debug_gemm_bf16(A, W, C, M, N, K, epi)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    print(json.dumps({"gemm_bf16": {"M": M, "N": N, "K": K, "epi": epi}, "calls": steps, "ms": round(ms, 4),
                      "TFLOP/s": round(tflops, 1), "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}),
          flush=True)


def attention_only(torch, zo, shape, steps, warmup):
    """The decoders' causal attention softmax(Q K^T / sqrt(dh)) V on a bf16
    QKV buffer [B S][3 H dh] of N(0,1) values, through the C ABI's debug entry;
    prints its time and rate (causal flops 2 B H S^2 dh)."""
    B, S, H, dh = shape
    g = torch.Generator(device="cuda").manual_seed(0)
    qkv = torch.randn(B * S, 3 * H * dh, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
    out = torch.zeros(B * S * H * dh, dtype=torch.int16, device="cuda")
    for _ in range(max(warmup, 1)):
        zo.debug_attention(qkv, out, B, S, H, dh)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        zo.debug_attention(qkv, out, B, S, H, dh)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = 2.0 * B * H * S * S * dh / (ms * 1e-3) / 1e12
    print(json.dumps({"attention": {"B": B, "S": S, "H": H, "dh": dh}, "calls": steps, "ms": round(ms, 4),
                      "TFLOP/s": round(tflops, 1), "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}),
          flush=True)


def cpu_baseline_variant(info, split=None, dust=None, seconds=12.0):
    """The oracle's split-perturbation or Dust step on the same workload,
    single-threaded, with smaller populations, counted in the bench line's
    unit (split: f2-evaluations 4 p1 ps; Dust: draws k1 + k2)."""
    from threadpoolctl import threadpool_limits

    from oracle import oracle
    arena = oracle.Arena(info["oracle_desc"], info["arena"].copy())
    if split:
        p1, ps = 2, min(split[1], 2)
        run = lambda r: oracle.fedspzo_step(arena, info["oracle_batch"], seed=r, p1=p1, ps=ps, eps=info["eps"],
                                            lr=info["lr"])
        per, what = 4 * p1 * ps, f"split-perturbation step(s) with p1={p1}, ps={ps}"
    else:
        k1, k2 = 4, 16
        run = lambda r: oracle.dust_step(arena, info["oracle_batch"], seed=r, k1=k1, sigma1=0.05, k2=k2,
                                         sigma2=0.05, lr=info["lr"])
        per, what = k1 + k2, f"Dust step(s) with k1={k1}, k2={k2}"
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < seconds:
            run(reps)
            reps += 1
        t = time.perf_counter() - t0
    counted = "f2-evaluations (4 p1 ps per step)" if split else "draws (k1 + k2 per step)"
    return {"value": round(per * reps / t, 3), "unit": "probe-evals/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{reps} oracle {what} of the same workload, single-threaded, {t:.1f} s; counts {counted}"}


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decoder(info):
    """The oracle's decoder forward is far too slow for a whole evaluation
    (OPT-30B shape: about 1e15 flops per evaluation in fp64 numpy), so its
    cost is extrapolated: one forward on one sequence of S' tokens with 1 and
    with 2 layers (full width and vocabulary, constant weights; the fastest of
    three runs each) gives the
    per-layer and the embedding + LM-head times, scaled linearly to L layers
    and B x S tokens.  The causal attention's S^2 term is scaled linearly too,
    which favours the CPU; the small products of S' tokens run below the
    CPU's large-matrix rate, which disfavours it."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import oracle
    sh = info["decoder_shape"]
    s_small = 16 if sh["d"] >= 4096 else 64
    tokens = (np.arange(s_small, dtype=np.int64) * 7919 % sh["vocab"])[None, :]
    times = []
    with threadpool_limits(limits=1):
        for layers in (1, 2):
            desc = {"kind": "decoder", "layers": layers, "d": sh["d"], "heads": sh["heads"], "ffn": sh["ffn"],
                    "vocab": sh["vocab"], "max_seq": s_small, "act": sh["act"]}
            params = {name: np.full(shape, 0.01 if not name.endswith("_g") else 1.0)
                      for name, shape in oracle.param_shapes(desc)}
            best = float("inf")
            for _ in range(3):  # the first call also pays one-time costs; keep the fastest
                t0 = time.perf_counter()
                oracle.decoder_loss(desc, params, tokens)
                best = min(best, time.perf_counter() - t0)
            times.append(best)
            del params
    per_layer = max(times[1] - times[0], 0.0)
    rest = max(times[0] - per_layer, 0.0)
    scale = sh["batch"] * sh["seq"] / s_small
    t_eval = scale * (sh["layers"] * per_layer + rest)
    return {"value": float(f"{1.0 / t_eval:.4g}"), "unit": "probe-evals/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(), "extrapolated": True,
            "sample": f"extrapolated (forward evaluations only): one forward on 1 x {s_small} tokens with 1 and 2 "
                      f"layers ({times[0]:.2f} s, {times[1]:.2f} s), scaled to {sh['layers']} layers and "
                      f"{sh['batch']} x {sh['seq']} tokens = {t_eval:.0f} s per evaluation, single-threaded"}


def cpu_baseline(info):
    """The oracle as it stands, single-threaded, on a bounded sample: one
    fused-mode step of the same workload with fewer probes."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import oracle
    probes = 2 if info["oracle_desc"]["kind"] == "mlp" else 4
    arena = oracle.Arena(info["oracle_desc"], info["arena"].copy())
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.spsa_step(arena, info["oracle_batch"], seed=reps, n_probes=probes, eps=info["eps"],
                             lr=info["lr"], mode="fused")
            reps += 1
            if time.perf_counter() - t0 > 12.0:
                break
        t = time.perf_counter() - t0
    evals = 2 * probes * reps
    return {"value": round(evals / t, 3), "unit": "probe-evals/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{reps} oracle SPSA step(s) of the same workload with N={probes} probes "
                      f"({evals} evaluations + update), single-threaded, {t:.1f} s",
            "probe_parallel": cpu_baseline_probe_parallel(info)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "across GPUs the step would shard by probes (each GPU evaluates its own probes, "
              "one all-gather of the scalars g_i, every replica runs the same update)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from zeroth_order_backprop_amd import inputs, zo
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.gemm:
        gemm_only(torch, zo, [int(x) for x in args.gemm.split(",")], args.steps, args.warmup, args.gemm_epi)
        return
    if args.attention:
        attention_only(torch, zo, [int(x) for x in args.attention.split(",")], args.steps, args.warmup)
        return
    if args.dirs != "gauss" and args.workload not in DECODERS:
        print("bench.py: 8-bit directions apply in place or in copies; use a decoder workload (the fp32 ones run fused)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload in DECODERS:
        model, batch, keep, info = build_decoder(torch, zo, inputs, args.workload, args.dirs)
    else:
        model, batch, keep, info = (build_mlp if args.workload == "mlp" else build_lsq)(torch, zo, inputs)
    if args.mode:
        if args.mode == "copies" and args.workload not in DECODERS:
            print("bench.py: copies steps are for the decoder workloads", file=sys.stderr)
            sys.exit(2)
        info["mode"] = args.mode
        info["workload"] = info["workload"].rsplit(";", 1)[0] + {
            "inplace": "; in-place mode", "fused": "; perturbed-tile (fused) mode",
            "copies": "; copies mode (D(W +- eps z_i) written to arena copies, evaluated side by side)"}[args.mode]
    N = info["probes"]
    pc = 1 if args.precond else 0
    split = None
    dust = None
    if args.dust:
        if args.workload != "mlp" or args.precond or args.split:
            print("bench.py: --dust applies to the MLP workload alone", file=sys.stderr)
            sys.exit(2)
        dust = tuple(int(x) for x in args.dust.split(","))
        info["kernel"] = "dust"
    if args.split:
        if args.workload != "mlp" or args.precond:
            print("bench.py: --split applies to the MLP workload, without --precond", file=sys.stderr)
            sys.exit(2)
        split = tuple(int(x) for x in args.split.split(","))
    if dust:
        evals_per_step = 1 + dust[0] + dust[1]          # clean + hidden draws + head draws
        probe_evals_per_step = dust[0] + dust[1]        # the population members
    else:
        evals_per_step = 4 * split[0] * split[1] if split else 2 * N + pc
        probe_evals_per_step = evals_per_step if split else 2 * N
    # every step (warm-up, timed, instrumented) writes its losses and scalars
    # into its own row, so that all of them can be checked for finiteness
    # afterwards without adding work to the timed region
    instr_steps = min(args.steps, 3) if "decoder_shape" in info and info["params"] > 10**10 else args.steps
    total_steps = args.warmup + args.steps + instr_steps
    n_loss = evals_per_step * info["batch"] if dust else evals_per_step
    n_g = max(N, split[0] if split else 0)
    losses_all = torch.zeros(total_steps, n_loss, dtype=torch.float64, device="cuda")
    g_all = torch.zeros(total_steps, n_g, dtype=torch.float64, device="cuda")
    g2 = torch.zeros(2 * split[0] * split[1] if split else 1, dtype=torch.float64, device="cuda")
    mode = {"fused": zo.ZO_MODE_FUSED, "copies": zo.ZO_MODE_COPIES}.get(info["mode"], zo.ZO_MODE_INPLACE)

    def step(seed):
        losses, g = losses_all[seed], g_all[seed]
        if dust:
            model.step_dust(batch, seed, dust[0], dust[1], 0.05, 0.05, info["lr"], losses)
        elif split:
            model.step_split(batch, seed, split[0], split[1], info["eps"], info["lr"], losses, g, g2)
        else:
            model.step(batch, seed, N, info["eps"], info["lr"], mode, losses, g, precond=pc,
                       curv_floor=args.curv_floor)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    # timed region: exactly K steps; HIP events bracket only the dominant
    # kernel's launches (on the library's stream) for the roofline
    zo.timing_reset()
    zo.timing_select(info["kernel"])
    zo.timing_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]  # after each step, for percentiles
    torch.cuda.synchronize()
    start.record()
    for t in range(args.steps):
        step(args.warmup + t)
        marks[t].record()
    stop.record()
    torch.cuda.synchronize()
    zo.timing_enable(False)
    total_ms = start.elapsed_time(stop)
    per_step = np.array([start.elapsed_time(marks[0])] +
                        [marks[t - 1].elapsed_time(marks[t]) for t in range(1, args.steps)])
    ms_step = total_ms / args.steps
    evals_per_s = probe_evals_per_step * args.steps / (total_ms * 1e-3)
    k_ms, k_n = zo.timing_query(info["kernel"])
    k_avg_s = k_ms / k_n * 1e-3
    # then the same number of steps again with events around every launch,
    # for the per-kernel table
    zo.timing_reset()
    zo.timing_select(None)
    zo.timing_enable(True)
    i0 = torch.cuda.Event(enable_timing=True)
    i1 = torch.cuda.Event(enable_timing=True)
    i0.record()
    for t in range(instr_steps):
        step(args.warmup + args.steps + t)
    i1.record()
    torch.cuda.synchronize()
    zo.timing_enable(False)
    ms_step_instr = i0.elapsed_time(i1) / instr_steps
    # a non-finite loss would make the update write nothing (and the step
    # lighter than the method's): fail rather than report such a run
    all_losses = losses_all.cpu().numpy()
    all_g = g_all.cpu().numpy()
    if not (np.isfinite(all_losses).all() and np.isfinite(all_g).all()):
        bad = [int(t) for t in range(total_steps) if not np.isfinite(all_losses[t]).all()]
        print(f"bench.py: non-finite losses or scalars at steps {bad}: the run is not a valid measurement",
              file=sys.stderr)
        sys.exit(3)
    extra = {}
    bound, peak, unit = "mfma", info["peak_tflops"], "TFLOP/s"
    if dust:
        # hidden-layer draws and output errors: each regenerates k1 x M x hidden
        # Gaussians (c_z VALU instructions each) -- priced against the VALU peak
        gauss = 2.0 * dust[0] * info["batch"] * info["hidden"] * args.steps / k_n
        flops_per_launch = gauss * C_Z / 1e0
        bound, peak, unit = "alu", VALU_PEAK_LANE_OPS / 1e12, "T lane-op/s"
        extra = {"gaussians_per_s": round(gauss / k_avg_s, 1), "c_z": C_Z}
    elif info["kernel"] == "gemm_bf16":
        # layer GEMMs of all evaluations: algorithmic flops / summed launch time
        flops_per_launch = evals_per_step * info["gemm_flops_per_eval"] * args.steps / k_n
    elif "split_bf16" in info:
        # one launch forms the N direction products X Z_i^T (the +- evaluations
        # of a probe share one, by the first layer's linearity): the method's
        # fp32 work is 2 M K H flops per direction, priced against the fp32
        # peak.  The kernel computes each fp32 product as six bf16 MFMA
        # products; that emulation rate against the bf16 peak is reported
        # beside it, with the generation of every direction element it uses.
        sp = info["split_bf16"]
        dirs_per_launch = split[0] * args.steps / k_n if split else N
        flops_per_launch = dirs_per_launch * sp["direction_flops"]
        bound, peak, unit = "mfma", FP32_PEAK_TFLOPS, "TFLOP/s"
        # split perturbation: each theta_1 direction's launch also draws 2 ps theta_2 directions
        gauss = dirs_per_launch * (sp["gaussians"] if not split else sp["w1_gaussians"] + 2 * split[1] * sp["w2_gaussians"])
        six = 6 * flops_per_launch / k_avg_s / 1e12
        extra = {"split_bf16_tflops": round(six, 2), "split_bf16_frac_of_bf16_peak": round(six / BF16_PEAK_TFLOPS, 4),
                 "gaussians_per_s": round(gauss / k_avg_s, 1),
                 "valu_frac_generation": round(gauss * C_Z / k_avg_s / VALU_PEAK_LANE_OPS, 4),
                 "c_z": C_Z}
    else:
        flops_per_launch = 2 * N * info["flops_per_eval"]
    achieved = flops_per_launch / k_avg_s / 1e12
    kernels = {}
    fwd_ms = 0.0  # per step, summed over the kernels that evaluate (all but perturb and update)
    for fam in ("gemm_f32", "gemm_f32_base", "dust", "gemm_bf16", "lm_head", "attention", "layernorm", "embed", "reduce", "update",
                "perturb"):
        ms, n = zo.timing_query(fam)
        if n and fam not in ("perturb", "update"):
            fwd_ms += ms / instr_steps
        if n:
            kernels[fam] = {"avg_us": round(ms / n * 1e3, 2), "launches_per_step": n / instr_steps,
                            "ms_per_step": round(ms / instr_steps, 3)}
    # the step's own perturbation and update passes over the whole arena
    # (2 P b bytes each: one read and one write of every parameter)
    step_passes = {}
    arena_bytes = info["params"] * (2 if info["dtype"] == "bf16" else 4)
    for fam in ("perturb", "update"):
        if fam in kernels:
            # a copies-mode perturbation reads the arena once and writes 2P copies:
            # per step (launches + 2N) arena sizes
            per_launch = (2.0 * arena_bytes if not (fam == "perturb" and info["mode"] == "copies") else
                          (kernels[fam]["launches_per_step"] + 2 * N) * arena_bytes / kernels[fam]["launches_per_step"])
            gbs = per_launch / (kernels[fam]["avg_us"] * 1e-6) / 1e9
            step_passes[fam] = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                                "avg_us": kernels[fam]["avg_us"], "bytes": int(per_launch),
                                **(valu_fields(fam, info["params"] * (1 if fam == "perturb" else N),
                                               kernels[fam]["avg_us"] * 1e-6)
                                   if args.dirs == "gauss" and info["mode"] != "copies" else {}),
                                **({"probes": N} if fam == "update" else {}),
                                **({"note": "arena resident in the last-level cache (not an HBM figure)"}
                                   if arena_bytes < 256e6 else {})}
    # forward-only rate: the evaluations of a step over the summed time of the
    # kernels that evaluate (everything but the perturbation and update passes)
    rates = {"step_evals_per_s": round(evals_per_s, 2),
             "forward_only_evals_per_s": round(probe_evals_per_step / (fwd_ms * 1e-3), 2) if fwd_ms else None,
             "probe_pairs_per_s": None if (split or dust) else round(evals_per_s / 2, 2),
             "ms_per_step_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)]}
    if "lm_head" in kernels:
        t = kernels["lm_head"]["ms_per_step"] * 1e-3
        kernels["lm_head"]["TFLOP/s"] = round(evals_per_step * info["head_flops_per_eval"] / t / 1e12, 1)
    if "attention" in kernels:
        t = kernels["attention"]["ms_per_step"] * 1e-3
        kernels["attention"]["TFLOP/s"] = round(evals_per_step * info["attn_flops_per_eval"] / t / 1e12, 1)
    if "gemm_bf16" in kernels and "gemm_parts_flops_per_eval" in info:
        # each layer GEMM on its own: algorithmic flops over its launches' time
        parts = {}
        for part, fl in info["gemm_parts_flops_per_eval"].items():
            ms, n = zo.timing_query(f"gemm_bf16.{part}")
            if n:
                tflops = evals_per_step * fl * instr_steps / (ms * 1e-3) / 1e12
                parts[part] = {"avg_us": round(ms / n * 1e3, 2), "launches_per_step": n / instr_steps,
                               "TFLOP/s": round(tflops, 1), "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}
        kernels["gemm_bf16"]["parts"] = parts
    zo.timing_reset()
    timed = all_losses[args.warmup:args.warmup + args.steps]
    line = {
        "metric": METRIC, "value": round(evals_per_s, 2), "unit": "probe-evals/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_instrumented": round(ms_step_instr, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": info["dtype"],
        "data": "synthetic (seeded N(0,1) inputs, random-init weights; no dataset)",
        "config": {"workload": info["workload"], "probes": N, "batch": info["batch"], "params": info["params"],
                   "mode": info["mode"], "parallelism": "none (1 GPU)",
                   **({"variant": "1.5-SPSA", "evals_per_step": evals_per_step, "curv_floor": args.curv_floor}
                      if pc else {}),
                   **({"directions": "8-bit packed (256-level quantised Gaussian)"} if args.dirs == "q8" else {}),
                   **({"variant": "split perturbation (FedSPZO), activation reuse", "p1": split[0], "ps": split[1],
                       "p2": 2 * split[0] * split[1], "evals_per_step": evals_per_step} if split else {}),
                   **({"variant": "Dust (activation noise, per-token rewards)", "k1": dust[0], "k2": dust[1],
                       "sigma": 0.05, "evals_per_step": evals_per_step, "unit_note": "value counts draws (k1 + k2)"}
                      if dust else {})},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": None if (split or dust or args.dirs != "gauss" or args.mode in ("fused", "copies"))
                     else TRAFFIC.get(KERNEL_REV.get(args.workload) or "", None),
                     "kernel": ((f"gemm_f32 direction-product GEMM (split-bf16 MFMA), "
                                 f"{evals_per_step if split else 2 * N} evaluations per step"
                                 if "split_bf16" in info else
                                 f"{info['kernel']} fused perturbed-tile GEMM, {2 * N} evaluations per launch")
                                if info["kernel"] == "gemm_f32" else
                                "dust hidden-layer draws and output errors (Gaussian generation, GELU, logits)"
                                if dust else "gemm_bf16 layer GEMMs (QKV, O, up, down)"),
                     "avg_launch_us": round(k_avg_s * 1e6, 2), **extra},
        "rates": rates,
        "kernels": kernels,
        "step_passes": step_passes,
        "losses": {"first_timed_step_mean": float(timed[0].mean()), "last_timed_step_mean": float(timed[-1].mean()),
                   "all_finite": True, "steps_checked": total_steps},
    }
    if not args.no_passes:
        line["perturb_update"] = measure_passes(torch, zo)
    if not args.no_cpu_baseline and "oracle_desc" in info:
        line["cpu_baseline"] = cpu_baseline_variant(info, split, dust) if (split or dust) else cpu_baseline(info)
    elif not args.no_cpu_baseline and "decoder_shape" in info:
        line["cpu_baseline"] = cpu_baseline_decoder(info)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
