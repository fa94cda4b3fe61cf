"""Benchmark of the MoE decode layer on one MI355X.

One step = moe_layer_forward over one batch of token rows (router GEMV,
top-k + compaction, gate+up+SiLU, down, blend) with every input already in
HBM.  Steps rotate over several copies of the expert weights and a pool of
token batches, so each step's selected experts are cold in the 256 MB
Infinity Cache and every step routes differently.

Prints ONE JSON line: tokens/s of the workload, µs/step, the roofline of the
dominant kernel (gate+up GEMV: algorithmic bytes per launch / its measured
duration from HIP events recorded around it in every timed step), and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer µs/step & tokens/s at N=1..256; achieved HBM GB/s vs 8 TB/s peak"
PEAK_HBM_GBPS = 8000.0
POOL_B = 2 << 30  # the cold-read probe's pool, 8x the 256 MB Infinity Cache
PEAK_MFMA_BF16_TFLOPS = 2500.0  # dense bf16 MFMA (the expert MFMA path's type)

# HBM bytes per gate+up launch from two rocprofv3 --pmc runs (FETCH_SIZE x 2.000, WRITE_SIZE
# x 1.000, the factors a 1 GiB device copy reads), with the hash of the expert-kernel sources
# they were taken on: reported only while the sources still hash to it.
TRAFFIC = {
    ("qwen3_30b_a3b", 4): {
        "sources_sha256": "9d02e78d71a0bdf14fbd8bda82a5135a5d371cada877336f3a2d9fcd5c9dacfb",
        "bytes": 177228161,
        "profile": "profiles/expert_gemv_qwen3_30b_a3b_n4_hbm_counters.md",
    },
    ("verify_mxfp4", 256): {
        "sources_sha256": "9d02e78d71a0bdf14fbd8bda82a5135a5d371cada877336f3a2d9fcd5c9dacfb",
        "bytes": 1833345669,
        "profile": "profiles/expert_mfma_verify_mxfp4_n256_hbm_counters.md",
    },
}


def expert_sources_sha256() -> str:
    """sha256 over the expert-pass kernel sources (headers and experts*.hip, sorted by name)."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "mixture_experts_decode_wave_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "experts*.hip")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the stream it runs on)."""

    def __init__(self, n: int):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.ev = (C.c_void_p * n)()
        for i in range(n):
            h = C.c_void_p()
            rc = self.hip.hipEventCreate(C.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev[i] = h

    def group(self, i: int):
        """Address of handles i, i+1, ... (the hipEvent_t* the library takes)."""
        return C.c_void_p(C.addressof(self.ev) + i * C.sizeof(C.c_void_p))

    def ms(self, a: int, b: int) -> float:
        out = C.c_float()
        rc = self.hip.hipEventElapsedTime(C.byref(out), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return out.value


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="verify_mxfp4")
    p.add_argument("--rows", type=int, default=256, help="token rows N of one step")
    p.add_argument("--copies", type=int, default=0,
                   help="weight copies rotated over (0: 8, or 2 when a copy exceeds 4 GB)")
    p.add_argument("--batches", type=int, default=64, help="token batches rotated over")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU work budget of the oracle baseline (0 = skip); at least one "
                        "step runs")
    p.add_argument("--cpu-rows-1thread", type=int, default=4,
                   help="rows of each oracle step on one host thread (at most N)")
    p.add_argument("--pre-norms", action="store_true",
                   help="run the layer with its router pre-norm and pre-expert RMSNorm "
                        "(moe_layer_forward_norm)")
    p.add_argument("--hash-vocab", type=int, default=0,
                   help="hash routing over a synthetic token table of this many tokens "
                        "(moe_layer_forward_hash; 0 = top-k routing)")
    p.add_argument("--read-probe-mib", type=int, default=1024,
                   help="after the steps, time the library's streaming-read probe kernel over "
                        "a buffer of this many MiB, 10 launches (the practical read ceiling, "
                        "as context; 0 = skip)")
    p.add_argument("--read-probe-sizes", default="",
                   help="comma-separated MiB sizes: time the streaming-read probe on cold "
                        "slices of a 2 GiB pool at each size (the read ceiling of a step that "
                        "moves that many bytes, as context; empty = skip)")
    p.add_argument("--no-matched-probe", dest="matched_probe", action="store_false",
                   help="skip the streaming-read probe at the step's own expert bytes")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="before the steps, copy a buffer of this many MiB 3 times (a plain "
                        "copy kernel of known size, to scale HBM counters by; 0 = none)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_decode_wave_amd as mw
    import moe_synth as ms
    from mixture_experts_decode_wave_amd.layer import device_layer

    mw.lib()
    torch.cuda.set_device(0)
    spec = ms.SPECS[args.workload]
    n = args.rows
    dev = "cuda"

    base = ms.make_layer(spec, seed=0, device=dev)
    layers = [device_layer(base, max_n=n)]
    copies = args.copies or (8 if spec.num_experts * ms.expert_bytes(spec) <= (4 << 30) else 2)
    for c in range(1, copies):
        li = ms.LayerInputs(spec, base.x, base.router, base.bias,
                            *[ms.Matrix(m.w.clone(), None if m.s is None else m.s.clone())
                              for m in (base.gate, base.up, base.down)],
                            *[None if m is None else ms.Matrix(m.w.clone(),
                                                               None if m.s is None else m.s.clone())
                              for m in (base.sh_gate, base.sh_up, base.sh_down)],
                            sgate=base.sgate, seed=0)
        dl = device_layer(li, max_n=n)
        dl.ws = layers[0].ws
        layers.append(dl)
    def batch(b):  # n rows: as many fresh 256-row draws as it takes
        parts, j = [], 0
        while sum(p.shape[0] for p in parts) < n:
            parts.append(ms.fresh_x(base, 100 + 1000 * j + b))
            j += 1
        return torch.cat(parts, 0)[:n].contiguous()

    xs = [batch(b) for b in range(args.batches)]
    adt = xs[0].dtype
    out = torch.empty(n, spec.hidden, dtype=adt, device=dev)
    logits = torch.empty(n, spec.router_width, dtype=torch.float32, device=dev)
    K, W = args.steps, args.warmup
    idx_log = torch.empty(K, n, spec.top_k, dtype=torch.int32, device=dev)
    w_buf = torch.empty(n, spec.top_k, dtype=torch.float32, device=dev)
    idx_tmp = torch.empty(n, spec.top_k, dtype=torch.int32, device=dev)
    NE = mw.MOE_LAYER_EVENTS
    ev = HipEvents(NE * K)

    norms = ms.make_norms(spec, 0, dev) if args.pre_norms else None
    if args.hash_vocab and args.pre_norms:
        print("--hash-vocab and --pre-norms are separate entry points", file=sys.stderr)
        sys.exit(2)
    htab = ms.make_hash_table(spec, args.hash_vocab, 0, dev) if args.hash_vocab else None
    htok = ([ms.make_token_ids(n, args.hash_vocab, b, dev) for b in range(args.batches)]
            if args.hash_vocab else None)
    x_index = {id(x): b for b, x in enumerate(xs)}

    def run(dl, x, strm, idx_out, evp=None):
        if htab is not None:
            mw.moe_layer_forward_hash(dl.cfg, x, htok[x_index[id(x)]], htab, dl.li.router,
                                      dl.tables, dl.shared, out, dl.ws, logits=logits,
                                      topk_idx=idx_out, topk_w=w_buf, stream=strm,
                                      stage_events=evp)
        elif norms is None:
            mw.moe_layer_forward(dl.cfg, x, dl.li.router, dl.li.bias, dl.tables, dl.shared, out,
                                 dl.ws, logits=logits, topk_idx=idx_out, topk_w=w_buf,
                                 stream=strm, stage_events=evp)
        else:
            mw.moe_layer_forward_norm(dl.cfg, x, norms[0], norms[1], ms.NORM_EPS, dl.li.router,
                                      dl.li.bias, dl.tables, dl.shared, out, dl.ws,
                                      logits=logits, topk_idx=idx_out, topk_w=w_buf,
                                      stream=strm, stage_events=evp)

    def step(i, strm, idx_out, evp=None):
        run(layers[i % len(layers)], xs[i % len(xs)], strm, idx_out, evp)

    stream = torch.cuda.current_stream()
    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(W):
        step(i, stream, idx_tmp)
    torch.cuda.synchronize()

    # The timed region: K steps captured into one HIP graph and replayed once
    # (decode steps run from graphs; per-launch host cost is out of the loop).
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(K):
            step(W + i, side, idx_log[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    # The same K steps launched on the stream with start / stop events of every
    # stage's kernels (events of graph-launched kernels cannot be timed).
    te0 = time.perf_counter()
    for i in range(K):
        step(W + i, stream, idx_tmp, ev.group(NE * i))
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - te0) * 1e6 / K
    stage = np.array([[ev.ms(NE * i + 2 * s, NE * i + 2 * s + 1) for s in range(NE // 2)]
                      for i in range(K)]) * 1e3  # us
    gu_us = stage[:, 1]
    # whole step: first stage kernel start to last stage kernel end
    step_us = np.array([ev.ms(NE * i, NE * i + NE - 1) for i in range(K)]) * 1e3

    # Warm steps, as context: one weight copy and one token batch, so the
    # experts a step picks stay in the 256 MB Infinity Cache between steps.
    warm = torch.cuda.CUDAGraph()
    kw = min(K, 50)
    with torch.cuda.graph(warm, stream=side):
        for i in range(kw):
            run(layers[0], xs[0], side, idx_tmp)
    warm.replay()
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    warm.replay()
    torch.cuda.synchronize()
    warm_us = (time.perf_counter() - tw0) * 1e6 / kw

    # the box's practical streaming-read ceiling, as context: a read-only
    # kernel over a buffer far larger than the 256 MB Infinity Cache
    read_ceiling = None
    if args.read_probe_mib > 0:
        rb = args.read_probe_mib << 20
        buf = torch.zeros(rb, dtype=torch.uint8, device=dev)
        sink = torch.zeros(2048 * 256, dtype=torch.int32, device=dev)
        pev = HipEvents(20)
        mw.probe_stream_read(buf, sink, 2048, stream=stream)
        for i in range(10):
            mw.probe_stream_read(buf, sink, 2048, stream=stream, ev0=pev.ev[2 * i],
                                 ev1=pev.ev[2 * i + 1])
        torch.cuda.synchronize()
        p_us = float(np.mean([pev.ms(2 * i, 2 * i + 1) for i in range(10)]) * 1e3)
        read_ceiling = {"kernel": "stream_read_kernel", "bytes": rb, "launch_us": round(p_us, 2),
                        "GBps": round(rb / (p_us * 1e-6) / 1e9, 1),
                        "frac_of_peak": round(rb / (p_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        del buf, sink
    # the same probe at a step's own size: each launch reads a slice of a
    # 2 GiB pool that the launches before it have not touched, so nothing is
    # left in the 256 MB Infinity Cache (the median of the launches)
    pool = sink = None
    off = [0]  # runs on over every size, so a slice was last read >= 256 MB of reads ago

    def cold_read_us(sb, grid):
        nonlocal pool, sink
        if pool is None:
            pool = torch.zeros(POOL_B, dtype=torch.uint8, device=dev)
            sink = torch.zeros(8192 * 256, dtype=torch.int32, device=dev)
        if sb > POOL_B:  # a sweep of the whole pool, scaled
            return cold_read_us(POOL_B, grid) * sb / POOL_B
        sb = (sb + 15) // 16 * 16
        reps = max(4, min(16, POOL_B // sb - 1))  # slices over 1 GiB are re-read: still cold
        pev = HipEvents(2 * reps)
        for i in range(reps + 1):  # the first launch untimed
            if off[0] + sb > POOL_B:
                off[0] = 0
            sl = pool[off[0]:off[0] + sb]
            if i == 0:
                mw.probe_stream_read(sl, sink, grid, stream=stream)
            else:
                mw.probe_stream_read(sl, sink, grid, stream=stream, ev0=pev.ev[2 * i - 2],
                                     ev1=pev.ev[2 * i - 1])
            off[0] += sb
        torch.cuda.synchronize()
        return float(np.median([pev.ms(2 * i, 2 * i + 1) for i in range(reps)]) * 1e3)

    read_by_size = None
    if args.read_probe_sizes:
        read_by_size = []
        for mib in [int(v) for v in args.read_probe_sizes.split(",") if v]:
            sb = mib << 20
            us = cold_read_us(sb, 2048)
            read_by_size.append({"MiB": mib, "launch_us": round(us, 2),
                                 "GBps": round(sb / (us * 1e-6) / 1e9, 1),
                                 "frac_of_peak": round(sb / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)})

    # algorithmic bytes from each step's actual routing
    idx = idx_log.cpu().numpy().reshape(K, -1)
    # experts whose weights the step streams (zero-computation experts have none)
    distinct = np.array([len(np.unique(r[r < spec.num_experts])) for r in idx])
    gu_expert = ms.gate_up_bytes(spec)
    dn_expert = ms.expert_bytes(spec) - gu_expert
    sh = spec.shared_inter
    gu_sh = ms.gate_up_bytes(spec, sh) if sh else 0
    dn_sh = (ms.expert_bytes(spec, sh) - gu_sh) if sh else 0
    asz = 4 if spec.act_dtype == "f32" else 2
    act_sz = 4 if spec.expert_dtype == "f32" else 2  # act is bf16 unless the experts are fp32
    x_bytes = n * spec.hidden * asz
    gu_bytes = (distinct * gu_expert + gu_sh + x_bytes
                + (n * spec.top_k * spec.inter + n * sh) * act_sz)
    step_bytes = (spec.router_width * spec.hidden * asz + x_bytes + distinct * (gu_expert + dn_expert)
                  + gu_sh + dn_sh + n * spec.hidden * asz)
    gu_achieved = float(np.mean(gu_bytes) / (np.mean(gu_us) * 1e-6) / 1e9)
    # algorithmic flops of the gate+up launch (two products per route, and the
    # shared expert's on every row): past the MFMA ridge, the bound is MFMA
    gu_flops = 2.0 * 2 * spec.inter * spec.hidden * n * spec.top_k + 2.0 * 2 * sh * spec.hidden * n
    ridge = PEAK_MFMA_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    mfma_bound = gu_flops / float(np.mean(gu_bytes)) > ridge
    step_gbps = float(np.mean(step_bytes) / (ms_per_step * 1e-3) / 1e9)
    expert_us = stage[:, 1] + stage[:, 2]
    expert_frac = float(np.mean(distinct * (gu_expert + dn_expert) + gu_sh + dn_sh)
                        / (np.mean(expert_us) * 1e-6) / 1e9 / PEAK_HBM_GBPS)

    # the probe at this step's own expert bytes: one cold read of the gate+up
    # weights and one of the down weights (the best of four grids each), the
    # time a plain read of the same bytes takes on this GPU; the expert passes
    # also read x and the act, write act and y, and run the blend
    matched = None
    if args.matched_probe:
        gu_w = int(np.mean(distinct * gu_expert + gu_sh))
        dn_w = int(np.mean(distinct * dn_expert + dn_sh))
        grids = (256, 512, 1024, 2048, 4096, 8192)
        gu_p = min(cold_read_us(gu_w, g) for g in grids)
        dn_p = min(cold_read_us(dn_w, g) for g in grids)
        matched = {"gate_up_weight_bytes": gu_w, "down_weight_bytes": dn_w,
                   "probe_us": round(gu_p + dn_p, 2), "gate_up_probe_us": round(gu_p, 2),
                   "down_probe_us": round(dn_p, 2),
                   "expert_us": round(float(np.mean(expert_us)), 2),
                   "probe_over_expert": round((gu_p + dn_p) / float(np.mean(expert_us)), 4),
                   "probe_frac_of_peak": round((gu_w + dn_w) / ((gu_p + dn_p) * 1e-6) / 1e9
                                               / PEAK_HBM_GBPS, 4)}
    del pool, sink

    # fp64 oracle on the host cores, bounded sample of the same workload
    cpu = cpu1 = None
    if args.cpu_seconds > 0 and htab is None:
        import oracle
        li_cpu = ms.to_device(base, "cpu")
        xs_cpu = [x.cpu() for x in xs]
        threads = oracle.max_threads()
        cpu_norms = None if norms is None else (norms[0].cpu(), norms[1].cpu(), ms.NORM_EPS)
        done, tc0 = 0, time.perf_counter()
        while True:
            oracle.layer_forward(li_cpu, n, nthreads=threads, x=xs_cpu[done % len(xs_cpu)],
                                 norms=cpu_norms)
            done += 1
            if time.perf_counter() - tc0 >= args.cpu_seconds:
                break
        tc = time.perf_counter() - tc0
        cpu = {"value": round(n * done / tc, 3), "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{done} full layer steps of {n} rows (fp64 C oracle, each selected "
                         f"expert decoded once, OpenMP over the output elements of each "
                         f"product; {tc:.1f} s)"}
        # and on one host thread, a quarter of the budget, over steps of the
        # first n1 rows of each batch (a whole step of many rows would take
        # minutes on one thread)
        n1 = max(1, min(n, args.cpu_rows_1thread))
        done1, tc0 = 0, time.perf_counter()
        while True:
            oracle.layer_forward(li_cpu, n1, nthreads=1, x=xs_cpu[done1 % len(xs_cpu)],
                                 norms=cpu_norms)
            done1 += 1
            if time.perf_counter() - tc0 >= args.cpu_seconds / 4:
                break
        tc1 = time.perf_counter() - tc0
        cpu1 = {"value": round(n1 * done1 / tc1, 3), "unit": "tokens/s", "cores": 1,
                "kind": "oracle",
                "sample": f"{done1} layer steps of {n1} rows (the first {n1} of a batch) on "
                          f"one thread ({tc1:.1f} s)"}

    tr = TRAFFIC.get((spec.name, n))
    traffic = tr["bytes"] if tr and tr["sources_sha256"] == expert_sources_sha256() else None

    res = {
        "metric": METRIC,
        "value": round(n / (ms_per_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.act_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}-shaped MoE decode layer, N={n} token rows "
                               f"(h{spec.hidden}, E{spec.num_experts}, top-{spec.top_k} "
                               f"{spec.scoring}, I{spec.inter}, {spec.expert_dtype} experts"
                               + (f", shared {sh}" if sh else "")
                               + (", gated shared" if spec.shared_gate else "")
                               + (f", {spec.zero_experts} zero experts"
                                  if spec.zero_experts else "")
                               + (", router pre-norm and pre-expert RMSNorm"
                                  if args.pre_norms else "")
                               + (f", hash routing over {args.hash_vocab} tokens"
                                  if args.hash_vocab else "") + ")",
                   "rows": n, "weight_copies": len(layers), "token_batches": len(xs)},
        "roofline": ({"bound": "hbm", "kernel": "expert_gemv gate+up",
                      "achieved": round(gu_achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(gu_achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                      "bytes_per_launch": int(np.mean(gu_bytes)),
                      "launch_us": round(float(np.mean(gu_us)), 3)} if not mfma_bound else
                     {"bound": "mfma", "kernel": "expert gate+up (grouped MFMA)",
                      "achieved": round(gu_flops / (np.mean(gu_us) * 1e-6) / 1e12, 2),
                      "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(gu_flops / (np.mean(gu_us) * 1e-6) / 1e12
                                    / PEAK_MFMA_BF16_TFLOPS, 4),
                      "traffic": traffic, "flops_per_launch": gu_flops,
                      "bytes_per_launch": int(np.mean(gu_bytes)),
                      "launch_us": round(float(np.mean(gu_us)), 3)}),
        "stages_us": {k: round(float(v), 3) for k, v in
                      zip(("route", "gate_up", "down_blend"), stage.mean(0))},
        "eager_us_per_step": round(eager_us, 2),
        "eager_step_us": {"p10": round(float(np.percentile(step_us, 10)), 2),
                          "median": round(float(np.median(step_us)), 2),
                          "p90": round(float(np.percentile(step_us, 90)), 2)},
        "warm_us_per_step": round(warm_us, 2),
        "expert_stream_frac": round(expert_frac, 4),
        "step_GBps": round(step_gbps, 1),
        "distinct_experts_per_step": round(float(distinct.mean()), 2),
        "read_ceiling": read_ceiling,
        "read_ceiling_by_size": read_by_size,
        "expert_stream_matched_probe": matched,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
