"""Benchmark of the activation-sparse (TwELL) FFN forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

A step is one twell_ffn_fwd over one batch of synthetic tokens (the up-projection GEMM
with the fused ReLU + TwELL epilogue, the overflow bookkeeping, and the sparse down
projection), enqueued as its three stages with a HIP event after the GEMM so that the
GEMM's own duration is measured on the stream it runs on. Inputs are resident in HBM
before timing starts. Prints one JSON line.

Baselines measured in the same run: a dense bf16 FFN (torch, hipBLASLt) on the same GPU
and shapes, and the CPU oracle on the host cores (a bounded sample of the workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 MFMA / packed VALU
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3"])
    ap.add_argument("--T", type=int, default=None, help="override token count (c3: 1, 8 or 64)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--ovf-cap", type=int, default=64)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--legs", default="pack,c3,c4,c5,gated,decode_graph",
                    help="extra workloads measured after the headline (comma list, or 'none')")
    return ap.parse_args()


def cpu_baseline(g, w, T_sample: int, min_seconds: float = 10.0) -> dict:
    """Time the oracle forward (fp64 numpy) on the first T_sample tokens, repeated until
    about min_seconds of CPU work has been done."""
    import numpy as np
    from oracle import twell_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    dt = g["dtype"]
    x = orc.widen(g["x"][:T_sample], dt)
    w1t = orc.widen(g["w1t"], dt)
    w2 = orc.widen(g["w2"], dt)
    b1 = g["b1"].astype(np.float64)
    reps, t_total = 0, 0.0
    while t_total < min_seconds and reps < 50:
        t0 = time.perf_counter()
        z, h, y = orc.ffn_fwd(x, w1t, b1, w2)
        orc.twell_pack(h, w.tile_w, w.slots, T_sample)
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": T_sample * reps / t_total, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "nproc": os.cpu_count(), "affinity_cpus": _affinity(),
            "cpu_model": _cpu_model(),
            "sample": f"{T_sample} tokens of the {w.name} workload x {reps} repetitions "
                      f"(fp64 numpy forward + TwELL pack, {t_total:.1f} s; 'cores' is the BLAS "
                      f"thread count numpy used)"}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _affinity():
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return None


def counter_traffic(workload: str):
    """HBM bytes per launch of the up GEMM from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each divided by what the counter reads per byte of a plain
    device copy), or None if the summary is missing, is for another workload, or was taken
    on a different version of the GEMM source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "k_up_twell_c2_counters.json")
    src = os.path.join(ROOT, "activation_sparse_transformer_up_amd", "csrc", "gemm.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha256") != sha or rec.get("workload") != workload:
        return None
    fetch = rec["fetch_kib_per_dispatch"] * 1024 / rec["copy_fetch_per_byte"]
    write = rec["write_kib_per_dispatch"] * 1024 / rec["copy_write_per_byte"]
    return fetch + write


def warm(fn, steps: int, min_seconds: float = 0.5):
    """W untimed steps, continued until at least min_seconds have passed: the GPU's clocks
    take several milliseconds of sustained load to settle, and kernels timed before that
    read up to 20 % slow."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < steps or time.perf_counter() - t0 < min_seconds:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _up(arr, dt, dev):
    import numpy as np
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def _time(fn, steps, warmup):
    import torch
    warm(fn, warmup, min_seconds=0.2)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def leg_c3(steps, warmup):
    """Decode-shaped layer, T in {1, 8, 64}, weights cold: three copies of (w1t, w2) are
    rotated so the 235 MB of weights of a step are not resident in the 256 MB MALL."""
    import numpy as np
    import torch
    import activation_sparse_transformer_up_amd as tw
    import synth
    w = synth.C3
    dev = torch.device("cuda:0")
    g = synth.generate(w)
    copies = [(_up(g["w1t"], "bf16", dev), _up(g["w2"], "bf16", dev)) for _ in range(3)]
    b1 = _up(g["b1"], "f32", dev)
    out = {}
    for T in (1, 8, 64):
        x = _up(g["x"][:T], "bf16", dev)
        hs = [tw.TwellMatrix(T, w.f, w.tile_w, w.slots, 4, torch.float32, dev) for _ in range(3)]
        y = torch.empty((T, w.d), device=dev)
        it = [0]

        def fwd():
            i = it[0] % 3
            it[0] += 1
            w1, w2_ = copies[i]
            tw.twell_ffn_fwd(x, w1, b1, w2_, w.tile_w, w.slots, 4, h=hs[i], y=y)

        def down():
            i = it[0] % 3
            it[0] += 1
            tw.twell_fwd_down(hs[i], copies[i][1], y=y)

        def gemm():
            i = it[0] % 3
            it[0] += 1
            tw.twell_up_gemm(x, copies[i][0], b1, hs[i])

        bb = b1.to(torch.bfloat16)

        def dense():
            i = it[0] % 3
            it[0] += 1
            w1, w2_ = copies[i]
            torch.relu(torch.addmm(bb, x, w1.t())) @ w2_

        ms = _time(fwd, steps * 4, warmup)
        # the gather walks the row lists of the staged path (the fused decode forward leaves none)
        for i in range(3):
            tw.twell_up_gemm(x, copies[i][0], b1, hs[i])
            tw.twell_up_finish(x, copies[i][0], b1, hs[i])
        ms_down = _time(down, steps * 4, warmup)
        ms_gemm = _time(gemm, steps * 4, warmup)
        ms_dense = _time(dense, steps * 4, warmup)
        # algorithmic bytes of the gather: unique W2 rows touched + y + the compact lists
        cnt = hs[0].counts.clamp(max=w.slots)
        nnz = int(cnt.sum().item())
        ci = hs[0].col_idx.cpu().numpy()
        uniq = len(np.unique(ci[ci >= 0]))
        gbytes = uniq * w.d * 2 + T * w.d * 4 + nnz * 8 + T * w.n_tiles * 4
        ubytes = w.f * w.d * 2 + T * w.d * 2 + T * w.n_tiles * (4 + 8 * w.slots)
        out[f"T{T}"] = {
            "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms, "dense_ms": ms_dense,
            "speedup_vs_dense": ms_dense / ms, "nnz_per_token": nnz / T, "unique_w2_rows": uniq,
            "gather": {"ms": ms_down, "algorithmic_bytes": gbytes,
                       "GB_per_s": gbytes / (ms_down * 1e-3) / 1e9,
                       "frac_hbm_peak": gbytes / (ms_down * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "up_gemm": {"ms": ms_gemm, "algorithmic_bytes": ubytes,
                        "GB_per_s": ubytes / (ms_gemm * 1e-3) / 1e9,
                        "frac_hbm_peak": ubytes / (ms_gemm * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "cold_weights": "3 rotated copies of w1t+w2 (705 MB)"}
    return out


def leg_c4(steps, warmup):
    """N:M pruning of the zero-bias layer's activations and the packed down projection."""
    import torch
    import activation_sparse_transformer_up_amd as tw
    import synth
    w = synth.C4
    dev = torch.device("cuda:0")
    g = synth.generate(w)
    x, w1t, w2 = _up(g["x"], "bf16", dev), _up(g["w1t"], "bf16", dev), _up(g["w2"], "bf16", dev)
    b1 = _up(g["b1"], "f32", dev)
    h = tw.ffn_up_relu_dense(x, w1t, b1, torch.bfloat16)
    T, f, d = w.T, w.f, w.d
    out = {"dense_down_ms": _time(lambda: h @ w2, steps, warmup)}
    out["up_relu_dense_ms"] = _time(lambda: tw.ffn_up_relu_dense(x, w1t, b1, torch.bfloat16, out=h), steps, warmup)
    out["up_relu_dense_frac_mfma_peak"] = 2.0 * T * d * f / (out["up_relu_dense_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    for n, m in w.nm:
        vals, idx = tw.nm_prune(h, n, m)
        ms_p = _time(lambda: tw.nm_prune(h, n, m), steps, warmup)
        y = torch.empty((T, d), device=dev)
        ms_d = _time(lambda: tw.nm_ffn_down(vals, idx, n, m, w2, y=y), steps, warmup)
        pbytes = T * f * 2 + T * (f // m) * n * 3
        # the same pruning inside the up GEMM's epilogue (the dense h never reaches HBM)
        fv, fi = tw.ffn_up_relu_nm(x, w1t, b1, n, m)
        ms_f = _time(lambda: tw.ffn_up_relu_nm(x, w1t, b1, n, m, vals=fv, idx=fi), steps, warmup)
        up_flop = 2.0 * T * d * f
        out[f"{n}:{m}"] = {
            "prune_ms": ms_p, "prune_GB_per_s": pbytes / (ms_p * 1e-3) / 1e9,
            "prune_frac_hbm_peak": pbytes / (ms_p * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "fused_up_nm_ms": ms_f, "unfused_up_nm_ms": out["up_relu_dense_ms"] + ms_p,
            "fused_vs_unfused": (out["up_relu_dense_ms"] + ms_p) / ms_f,
            "fused_up_nm_frac_mfma_peak": up_flop / (ms_f * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "nm_down_ms": ms_d, "nm_down_TFLOPs": 2.0 * T * f * d / (ms_d * 1e-3) / 1e12,
            "nm_down_vs_dense_down": out["dense_down_ms"] / ms_d}
    return out


def leg_pack(steps, warmup):
    """Standalone TwELL pack of a dense ReLU output at c2 (HBM-bound), and the unfused forward
    (dense ReLU GEMM to HBM, pack, gather) beside the fused one: what the GEMM epilogue saves."""
    import torch
    import activation_sparse_transformer_up_amd as tw
    import synth
    w = synth.C2
    dev = torch.device("cuda:0")
    g = synth.generate(w)
    x, w1t, w2 = _up(g["x"], "bf16", dev), _up(g["w1t"], "bf16", dev), _up(g["w2"], "bf16", dev)
    b1 = _up(g["b1"], "f32", dev)
    T, f, d = w.T, w.f, w.d
    n_t = f // w.tile_w
    cap = 64
    out = {}
    for name, dt in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
        h = tw.ffn_up_relu_dense(x, w1t, b1, dt)
        m = tw.twell_pack(h, w.tile_w, w.slots, cap)
        ms = _time(lambda: tw.twell_pack(h, w.tile_w, w.slots, cap, out=m), steps, warmup)
        eb = h.element_size()
        nbytes = T * f * eb + T * n_t * 4 + T * n_t * w.slots * (4 + eb)
        out[f"pack_{name}"] = {"ms": ms, "algorithmic_bytes": nbytes,
                               "GB_per_s": nbytes / (ms * 1e-3) / 1e9,
                               "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del h, m
    hb = torch.empty((T, f), dtype=torch.bfloat16, device=dev)
    mb = tw.TwellMatrix(T, f, w.tile_w, w.slots, cap, torch.bfloat16, dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)

    def unfused():
        tw.ffn_up_relu_dense(x, w1t, b1, torch.bfloat16, out=hb)
        tw.twell_pack(hb, w.tile_w, w.slots, cap, out=mb)
        tw.twell_down(mb, w2, y=y)
    mf = tw.TwellMatrix(T, f, w.tile_w, w.slots, cap, torch.float32, dev)
    out["unfused_fwd_ms"] = _time(unfused, steps, warmup)
    out["fused_fwd_ms"] = _time(lambda: tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=mf, y=y),
                                steps, warmup)
    out["unfused"] = "ffn_up_relu_dense (bf16 h to HBM) + twell_pack + twell_down"
    return out


def leg_gated(steps, warmup):
    """The gated layer y = (ReLU(x Wg + bg) * (x Wu)) W2 at c2 and at c3's decode sizes: the
    TwELL path (gate GEMM + TwELL, up dot products over the active units, down gather)
    against the dense bf16 layer (three GEMMs). The up stage's own time is the difference
    from the plain forward on the same gate; at decode its algorithmic bytes are the unique
    up rows read."""
    import torch
    import activation_sparse_transformer_up_amd as tw
    import synth
    dev = torch.device("cuda:0")
    out = {}
    for w, Ts in ((synth.C2, (synth.C2.T,)), (synth.C3, (1, 8, 64))):
        g = synth.generate(w)
        x_all = _up(g["x"], "bf16", dev)
        wgt, w2 = _up(g["w1t"], "bf16", dev), _up(g["w2"], "bf16", dev)
        wut = _up(synth.up_weights(w), "bf16", dev)
        bg = _up(g["b1"], "f32", dev)
        bgb = bg.to(torch.bfloat16)
        for T in Ts:
            x = x_all[:T].contiguous()
            h = tw.TwellMatrix(T, w.f, w.tile_w, w.slots, 16, torch.float32, dev)
            y = torch.empty((T, w.d), dtype=torch.float32, device=dev)
            ws = torch.empty((max(tw.twell_gate_up_workspace_bytes(T, w.d, w.f, h), 16),), dtype=torch.uint8,
                             device=dev)
            ms = _time(lambda: tw.twell_gated_ffn_fwd(x, wgt, bg, wut, w2, w.tile_w, w.slots, 16, h=h, y=y,
                                                      workspace=ws), steps, warmup)
            ms_plain = _time(lambda: tw.twell_ffn_fwd(x, wgt, bg, w2, w.tile_w, w.slots, 16, h=h, y=y),
                             steps, warmup)

            def dense():
                return (torch.relu(torch.addmm(bgb, x, wgt.t())) * (x @ wut.t())) @ w2
            dms = _time(dense, steps, warmup)
            rec = {"ms": ms, "dense_ms": dms, "speedup_vs_dense": dms / ms,
                   "up_stage_ms": ms - ms_plain}
            if T <= 64:
                # the fused inference path: gate GEMM, then one kernel over the active units
                hi = tw.TwellMatrix(T, w.f, w.tile_w, w.slots, 0, torch.float32, dev)
                ms_inf = _time(lambda: tw.twell_gated_ffn_infer(x, wgt, bg, wut, w2, w.tile_w, w.slots, h=hi, y=y),
                               steps, warmup)
                ms_gate = _time(lambda: tw.twell_up_gemm(x, wgt, bg, hi), steps, warmup)
                rec.update({"fused_infer_ms": ms_inf, "fused_speedup_vs_dense": dms / ms_inf,
                            "fused_vs_staged": ms / ms_inf, "gate_gemm_ms": ms_gate,
                            "fused_kernel_ms": ms_inf - ms_gate})
                del hi
            if w is synth.C3:
                cols = h.col_idx.clamp(min=0).view(-1)
                act = torch.zeros(w.f, dtype=torch.bool, device=dev)
                act[cols[(h.col_idx.view(-1) >= 0)]] = True
                uniq = int(act.sum().item())
                nbytes = uniq * w.d * 2
                rec["up_stage_unique_rows"] = uniq
                if rec["up_stage_ms"] > 0:
                    rec["up_stage_frac_hbm_peak"] = nbytes / (rec["up_stage_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS
            out[f"{'c2' if w is synth.C2 else 'c3'}_T{T}"] = rec
            del h, y
        del x_all, wgt, w2, wut
        torch.cuda.empty_cache()
    return out


def leg_decode_graph(steps, warmup):
    """A decode loop over 4 layers of c3's shape (per-layer densities 0.5 / 1 / 2 / 3 %),
    eager and captured in a HIP graph, beside the dense bf16 layers run the same way; T = 1
    and 8 tokens. Between layers each token is normalised to unit RMS (torch, fp32 -> bf16),
    the stand-in for the rest of a transformer block, the same for both paths."""
    import torch
    import activation_sparse_transformer_up_amd as tw
    import synth
    dev = torch.device("cuda:0")
    w = synth.C3
    out = {}
    x_bits, layers = synth.decode_layers(4, 64)
    L = [(_up(a["w1t"], "bf16", dev), _up(a["b1"], "f32", dev), _up(a["w2"], "bf16", dev)) for a in layers]
    x_all = _up(x_bits, "bf16", dev)

    def norm(y, out):
        yf = y.float()
        out.copy_(yf * torch.rsqrt(yf.square().mean(dim=1, keepdim=True)))
        return out

    # per-layer slot counts: each layer's row-maximum histogram on a 64-token calibration batch,
    # the smallest stash with no row beyond S (twell_choose_slots, capacity 0)
    hc = [tw.TwellMatrix(64, w.f, w.tile_w, w.slots, 4, torch.float32, dev) for _ in L]
    xc = x_all
    for (w1t, b1, w2), h in zip(L, hc):
        yc, _ = tw.twell_ffn_fwd(xc, w1t, b1, w2, w.tile_w, w.slots, 4, h=h, y_dtype=torch.bfloat16)
        xc = norm(yc, torch.empty_like(yc))
    slots_cal = [tw.twell_choose_slots(tw.twell_row_max_histogram(h).cpu().numpy(), w.tile_w, 64, w.f, 0)[0]
                 for h in hc]
    del hc
    out["per_layer_slots"] = slots_cal
    for T, per_layer in ((1, False), (8, False), (1, True), (8, True)):
        x0 = x_all[:T].contiguous()
        sl = slots_cal if per_layer else [w.slots] * len(L)
        hs = [tw.TwellMatrix(T, w.f, w.tile_w, S, 4, torch.float32, dev) for S in sl]
        ys = [torch.empty((T, w.d), dtype=torch.bfloat16, device=dev) for _ in L]
        xs = [torch.empty((T, w.d), dtype=torch.bfloat16, device=dev) for _ in L]

        def run():
            x = x0
            for l, ((w1t, b1, w2), h, y) in enumerate(zip(L, hs, ys)):
                tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, h.slots, 4, h=h, y=y, y_dtype=torch.bfloat16)
                x = norm(y, xs[l])

        def dense():
            x = x0
            for l, (w1t, b1, w2) in enumerate(L):
                x = norm(torch.relu(torch.addmm(b1.to(torch.bfloat16), x, w1t.t())) @ w2, xs[l])
            return x
        eager_ms = _time(run, steps, warmup)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        graph_ms = _time(graph.replay, steps, warmup)
        dense_ms = _time(dense, steps, warmup)
        dens = [float((hh.counts.clamp(max=w.slots).sum() / (T * w.f)).item()) for hh in hs]
        stash = sum(tw.twell_stash_bytes(T, w.f, w.tile_w, hh.slots, int(hh.ovf_n.item())) for hh in hs)
        out[f"T{T}" + ("_per_layer_S" if per_layer else "")] = {
            "layers": len(L), "slots": sl, "layer_density": dens, "eager_ms": eager_ms, "graph_ms": graph_ms,
            "graph_speedup": eager_ms / graph_ms, "dense_eager_ms": dense_ms,
            "speedup_vs_dense": dense_ms / graph_ms, "stash_bytes": stash,
            "tokens_per_s": T / (graph_ms * 1e-3)}
        del hs, ys, graph
    return out


def leg_c5(steps, warmup):
    """Training step (forward + backward with the L1 term) vs the dense bf16 FFN's
    forward + backward through autograd (the same six GEMMs a dense layer needs).

    Two flows of the hybrid format ("Formato Híbrido para Treinamento"):
      twell : the forward's TwELL (W=128, S=8) is the stash, the backward workspace sized for
              the whole entry capacity (no host round trip; the headline ms_fwd_bwd);
      rowell: after the forward, the row-nonzero histogram goes to the host, which picks the
              compact row-ELL width of this step (twell_choose_row_ell_width) and the exact
              entry count; the TwELL is converted into the row-ELL stash and freed, and the
              backward runs on the row-ELL with a workspace sized for the step's entries.
    Peak memory: device bytes allocated during one step above what was allocated before it
    (inputs and weights), outputs included (y, dx, dW1, dW2, db1; the dense layer's autograd
    keeps bf16 gradients, ours are fp32)."""
    import numpy as np
    import torch
    import activation_sparse_transformer_up_amd as tw
    import synth
    w = synth.C5
    dev = torch.device("cuda:0")
    g = synth.generate(w)
    x, w1t, w2, dy = (_up(g[k], "bf16", dev) for k in ("x", "w1t", "w2", "dy"))
    b1 = _up(g["b1"], "f32", dev)
    T, f, d = w.T, w.f, w.d
    cap, cap_ell = 1024, 1024
    h = tw.TwellMatrix(T, f, w.tile_w, w.slots, cap, torch.float32, dev)
    y = torch.empty((T, d), device=dev)
    ws = torch.empty((tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype),), dtype=torch.uint8, device=dev)
    ws_capacity_bytes = ws.numel()

    def step():
        tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=h, y=y)
        tw.twell_ffn_bwd(x, w1t, w2, h, dy, w.l1_coef, workspace=ws)

    ms = _time(step, steps, warmup)
    ms_fwd = _time(lambda: tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=h, y=y), steps, warmup)
    # the up GEMM with its TwELL epilogue alone (the forward's first stage), against bf16 peak
    ms_up = _time(lambda: tw.twell_up_gemm(x, w1t, b1, h), steps, warmup)
    up_frac = 2.0 * T * d * f / (ms_up * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=h, y=y)
    ovf = int(h.ovf_n.item())
    dens = float(h.counts.sum().item()) / (T * f)
    # Activation memory kept for the backward: counts, slots (int32 index + fp32 value) and the
    # fp32 backup rows, against a dense h; per slot count from the row-maximum histogram, and
    # the slot count twell_choose_slots picks.
    dense_bf16 = T * f * 2
    hist_dev = tw.twell_row_max_histogram(h)
    ms_hist = _time(lambda: tw.twell_row_max_histogram(h, hist_dev), steps, warmup)
    hist = hist_dev.cpu().numpy()
    per_s = {}
    for S in (4, 6, 8, 12, 16, 24, 32):
        n_ovf = int(hist[S + 1:].sum())
        b = tw.twell_stash_bytes(T, f, w.tile_w, S, n_ovf)
        per_s[str(S)] = {"overflow_rows": n_ovf, "bytes": b, "frac_of_dense_bf16": b / dense_bf16}
    best, best_bytes = tw.twell_choose_slots(hist, w.tile_w, T, f, cap)
    stash = tw.twell_stash_bytes(T, f, w.tile_w, w.slots, ovf)
    # the compact row-ELL of this step
    nnz_hist = tw.twell_row_nnz_histogram(h).cpu().numpy()
    nnz = int((nnz_hist * np.arange(len(nnz_hist))).sum())
    width, ell_bytes = tw.twell_choose_row_ell_width(nnz_hist, T, f, cap_ell)
    ws_entries_bytes = tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype, nnz=nnz)
    mem = {"dense_h_bf16_bytes": dense_bf16, "dense_h_fp32_bytes": 2 * dense_bf16,
           "stash_bytes": stash, "stash_frac_of_dense_bf16": stash / dense_bf16,
           "per_slots": per_s, "chosen_slots": best, "chosen_stash_bytes": best_bytes,
           "chosen_frac_of_dense_bf16": best_bytes / dense_bf16, "cap": cap,
           "row_max_histogram_ms": ms_hist, "stored_entries": nnz,
           "row_ell_width": width, "row_ell_stash_bytes": ell_bytes,
           "row_ell_frac_of_dense_bf16": ell_bytes / dense_bf16, "row_ell_cap": cap_ell,
           "bwd_workspace_capacity_bytes": ws_capacity_bytes, "bwd_workspace_entries_bytes": ws_entries_bytes}
    del ws, h, y
    torch.cuda.empty_cache()

    def step_twell_entries():
        hh = tw.TwellMatrix(T, f, w.tile_w, w.slots, cap, torch.float32, dev)
        yy, _ = tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=hh)
        hist_h = tw.twell_row_nnz_histogram(hh).cpu().numpy()
        n = int((hist_h * np.arange(len(hist_h))).sum())
        wsb = torch.empty((tw.twell_ffn_bwd_workspace_bytes(T, d, f, hh, x.dtype, nnz=n),), dtype=torch.uint8,
                          device=dev)
        return yy, tw.twell_ffn_bwd(x, w1t, w2, hh, dy, w.l1_coef, workspace=wsb)

    def step_rowell():
        hh = tw.TwellMatrix(T, f, w.tile_w, w.slots, cap, torch.float32, dev)
        yy, _ = tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=hh)
        hist_h = tw.twell_row_nnz_histogram(hh).cpu().numpy()
        N, _ = tw.twell_choose_row_ell_width(hist_h, T, f, cap_ell)
        n = int((hist_h * np.arange(len(hist_h))).sum())
        e = tw.twell_to_row_ell(hh, N, cap_ell)
        del hh                                   # the stash is the row-ELL from here on
        wsb = torch.empty((tw.twell_ffn_bwd_workspace_bytes(T, d, f, e, x.dtype, nnz=n),), dtype=torch.uint8,
                          device=dev)
        return yy, tw.twell_ffn_bwd(x, w1t, w2, e, dy, w.l1_coef, workspace=wsb)

    def peak_of(fn):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        out = fn()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        del out
        torch.cuda.empty_cache()
        return peak

    ms_twell_entries = _time(step_twell_entries, steps, warmup)
    ms_rowell = _time(step_rowell, steps, warmup)
    peak_twell = peak_of(step_twell_entries)
    peak_rowell = peak_of(step_rowell)
    xd = x.clone().requires_grad_(True)
    w1d = w1t.clone().requires_grad_(True)
    w2d = w2.clone().requires_grad_(True)
    bd = b1.to(torch.bfloat16).requires_grad_(True)

    def dense_step():
        hh = torch.relu(torch.addmm(bd, xd, w1d.t()))
        yy = hh @ w2d
        loss = (yy * dy).sum() + w.l1_coef * hh.float().sum()
        loss.backward()
        grads = (xd.grad, w1d.grad, w2d.grad, bd.grad)
        xd.grad = w1d.grad = w2d.grad = bd.grad = None
        return yy, grads

    ms_dense = _time(dense_step, steps, warmup)
    peak_dense = peak_of(dense_step)
    # the outputs each flow allocates: ours fp32 y, dx, dW1, dW2, db1; the dense layer bf16
    out_ours = 4 * (2 * T * d + 2 * f * d + f)
    out_dense = 2 * (2 * T * d + 2 * f * d + f)
    mem.update({"peak_step_bytes_twell_stash": peak_twell, "peak_step_bytes_row_ell_stash": peak_rowell,
                "peak_step_bytes_dense": peak_dense,
                "peak_row_ell_vs_dense": peak_rowell / peak_dense, "peak_twell_vs_dense": peak_twell / peak_dense,
                "outputs_bytes_ours_fp32": out_ours, "outputs_bytes_dense_bf16": out_dense,
                "peak_minus_outputs_row_ell": peak_rowell - out_ours, "peak_minus_outputs_twell": peak_twell - out_ours,
                "peak_minus_outputs_dense": peak_dense - out_dense,
                "peak_minus_outputs_row_ell_vs_dense": (peak_rowell - out_ours) / max(1, peak_dense - out_dense)})
    del xd, w1d, w2d, bd, x, w1t, w2, dy, b1
    torch.cuda.empty_cache()
    # hot tokens (every 1024th token's x scaled by 4, so those rows overflow) at S = 8 and 16
    variants = {f"hot1024_S{S}": c5_variant(w.with_(slots=S, hot_every=1024), cap, steps, warmup)
                for S in (8, 16)}
    achieved = 2.0 * T * d * f / (ms_up * 1e-3) / 1e12
    return {"tokens_per_s": T / (ms * 1e-3), "ms_fwd_bwd": ms, "ms_fwd": ms_fwd, "ms_bwd": ms - ms_fwd,
            "dense_ms_fwd_bwd": ms_dense, "speedup_vs_dense": ms_dense / ms, "density": dens,
            "ms_fwd_bwd_entry_workspace": ms_twell_entries, "ms_fwd_bwd_row_ell": ms_rowell,
            "up_gemm_ms": ms_up, "up_gemm_frac_mfma_peak": up_frac,
            "roofline": {"kernel": "k_up_twell (up GEMM + fused ReLU/TwELL epilogue)", "bound": "mfma",
                         "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                         "per_launch_flop": 2.0 * T * d * f, "avg_launch_ms": ms_up},
            "overflow_rows": ovf, "slots": w.slots, "tile_w": w.tile_w, "activation_memory": mem,
            "variants": variants}


def c5_variant(w, cap, steps, warmup):
    """Forward + backward time of one c5 variant (hot tokens, slot count)."""
    import torch
    import activation_sparse_transformer_up_amd as tw
    import synth
    dev = torch.device("cuda:0")
    g = synth.generate(w)
    x, w1t, w2, dy = (_up(g[k], "bf16", dev) for k in ("x", "w1t", "w2", "dy"))
    b1 = _up(g["b1"], "f32", dev)
    T, f, d = w.T, w.f, w.d
    h = tw.TwellMatrix(T, f, w.tile_w, w.slots, cap, torch.float32, dev)
    y = torch.empty((T, d), device=dev)
    ws = torch.empty((tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype),), dtype=torch.uint8, device=dev)

    def step():
        tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=h, y=y)
        tw.twell_ffn_bwd(x, w1t, w2, h, dy, w.l1_coef, workspace=ws)

    ms = _time(step, steps, warmup)
    ms_fwd = _time(lambda: tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, cap, h=h, y=y), steps, warmup)
    return {"slots": w.slots, "hot_every": w.hot_every, "ms_fwd_bwd": ms, "ms_fwd": ms_fwd,
            "tokens_per_s": T / (ms * 1e-3), "overflow_rows": int(h.ovf_n.item()),
            "capacity_ok": tw.twell_sync_status(h) == 0}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import activation_sparse_transformer_up_amd as tw
    import synth

    if a.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")      # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "dispatches": 3}))
        return

    w = synth.WORKLOADS[a.workload]
    T = a.T or w.T
    g = synth.generate(w, T=T)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(arr, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)

    x, w1t, w2 = up(g["x"], w.dtype), up(g["w1t"], w.dtype), up(g["w2"], w.dtype)
    b1 = up(g["b1"], "f32")
    d, f = w.d, w.f
    h = tw.TwellMatrix(T, f, w.tile_w, w.slots, a.ovf_cap, torch.float32, dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    t0, t1 = E(), E()

    # The timed step: one twell_ffn_fwd (up GEMM + fused TwELL epilogue, finish, gather).
    def fwd():
        tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, w.slots, a.ovf_cap, h=h, y=y)
    warm(fwd, a.warmup)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(a.steps):
        fwd()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / a.steps

    # The same work as its three public stages with a HIP event after the GEMM, for the
    # GEMM's own launch time (the events sit on the stream the kernels run on). The extra
    # event in the middle of every step makes this loop slightly slower than the one above.
    def staged(ev=None):
        tw.twell_up_gemm(x, w1t, b1, h)
        if ev is not None:
            ev.record()
        tw.twell_up_finish(x, w1t, b1, h)
        tw.twell_fwd_down(h, w2, y=y)

    warm(staged, a.warmup)
    starts = [E() for _ in range(a.steps)]
    gemm_end = [E() for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0.record()
    for i in range(a.steps):
        starts[i].record()
        staged(gemm_end[i])
    t1.record()
    torch.cuda.synchronize()
    ms_staged = t0.elapsed_time(t1) / a.steps
    gemm_ms = sum(s.elapsed_time(e) for s, e in zip(starts, gemm_end)) / a.steps
    nnz = int(h.counts.clamp(max=w.slots).sum().item())
    ovf_n = int(h.ovf_n.item())

    flops_up = 2.0 * T * d * f
    name = w.name.replace(f"_T{w.T}_", f"_T{T}_")
    traffic = counter_traffic(name)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = flops_up / (gemm_ms * 1e-3) / 1e12
    roof = {"kernel": "k_up_twell (up GEMM + fused ReLU/TwELL epilogue)", "bound": "mfma",
            "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
            "traffic": traffic, "per_launch_flop": flops_up, "avg_launch_ms": gemm_ms}
    if T <= 64:
        # decode sizes: the up stage streams W1 once (plus x and the TwELL it writes)
        n_t = f // w.tile_w
        ubytes = f * d * (2 if w.dtype == "bf16" else 4) + T * d * 2 + T * n_t * (4 + 8 * w.slots)
        gbs = ubytes / (gemm_ms * 1e-3) / 1e9
        roof = {"kernel": "up stage at decode sizes (W1 stream or decode tile GEMM, then the TwELL pack)",
                "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "traffic": traffic, "per_launch_bytes": ubytes, "avg_launch_ms": gemm_ms}
    out = {
        "metric": "FFN tokens/sec at 1% density (TwELL forward), speedup vs dense bf16, % MFMA peak",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded generator, random-init weights)",
        "config": {"workload": name, "T": T, "d_model": d, "d_ff": f, "tile_w": w.tile_w,
                   "slots": w.slots, "bias": w.bias, "seed": w.seed, "parallelism": "single GPU"},
        "roofline": roof,
        "measured_density": nnz / (T * f), "ovf_rows": ovf_n, "ms_per_step_staged": ms_staged,
    }

    if not a.no_dense:
        xb, w1b, w2b = x, w1t, w2
        bb = b1.to(x.dtype)

        def dense():
            return torch.relu(torch.addmm(bb, xb, w1b.t())) @ w2b
        warm(dense, a.warmup)
        t0.record()
        for _ in range(a.steps):
            dense()
        t1.record()
        torch.cuda.synchronize()
        dms = t0.elapsed_time(t1) / a.steps
        out["dense_baseline"] = {"value": T / (dms * 1e-3), "unit": "tokens/s", "ms_per_step": dms,
                                 "impl": f"torch relu(addmm) @ w2 in {w.dtype} (hipBLASLt)"}
        out["speedup_vs_dense"] = dms / ms

    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(g, w, T_sample=min(T, 4096))
    legs = [] if a.legs in ("", "none") else a.legs.split(",")
    if legs:
        del x, w1t, w2, h, y
        torch.cuda.empty_cache()
        out["legs"] = {}
        for leg in legs:
            fn = {"c3": leg_c3, "c4": leg_c4, "c5": leg_c5, "pack": leg_pack, "gated": leg_gated,
                  "decode_graph": leg_decode_graph}.get(leg)
            if fn is None:
                continue
            try:
                out["legs"][leg] = fn(max(5, a.steps // 5), max(2, a.warmup // 2))
            except Exception as e:        # a failing extra leg must not hide the headline
                out["legs"][leg] = {"error": f"{type(e).__name__}: {e}"}
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
