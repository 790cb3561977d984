"""Benchmark of the spectral MoE gate/up decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one bitsmoe_moe_gateup call: z = Phi^T x for the batch, then every
routed expert's bit-plane apply and the SiLU * mul epilogue.  Inputs are
seeded synthetic layers (see synth/) resident in HBM before timing starts.
To keep the 256 MB Infinity Cache from serving the data, the step rotates
over C device copies of the layer (C * layer bytes >= 1 GiB) and over NB
pre-generated batches.  Steps are replayed from HIP graphs (captured through
torch) and timed with HIP events on the launch stream.

Prints one JSON line (rank 0, N = 1).  The CPU baseline is the float64
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/token + % HBM roofline, spectral MoE gate/up layer, Qwen3-30B-A3B shape, batch 1"
HBM_PEAK_GBS = 8000.0
KERNEL_ONE_TOKEN = ("k_gateup_one (z, every routed expert's coefficients, expert apply and "
                    "SiLU*mul in one launch)")
KERNEL_ONE_LAUNCH = "k_gateup_fused (z, expert apply and SiLU*mul in one launch)"


def kernel_batched(T):
    """The launches of one batched step, timed together (the route grouping
    runs as one more work-group of the projection launch)."""
    proj = "k_proj_gemm" if T >= 64 else "k_proj_mfma" if T >= 16 else "k_proj_rows"
    return proj + " + k_group_coef + k_gateup_grouped (timed together)"

# HBM bytes per launch from FETCH_SIZE + WRITE_SIZE counter runs, scaled by
# the same counters on a plain copy of known size, with the hash of the
# kernel sources they were taken on: reported only while the sources still
# hash the same (None once a kernel has changed since).
TRAFFIC = {
    "qwen3_30b_a3b_t1": (28583154, "476f46c709b5bff4"),
    "qwen3_30b_a3b_t32": (111021641, "476f46c709b5bff4"),
    "mixtral_8x7b_t1": (149256251, "476f46c709b5bff4"),
    "mixtral_8x7b_t8": (352212659, "476f46c709b5bff4"),
    "deepseek_moe_16b_t512": (602235068, "476f46c709b5bff4"),
}


def kernel_source_hash():
    """First 16 hex digits of the SHA-256 of the library's sources (csrc/,
    in name order)."""
    import hashlib
    d = os.path.join(ROOT, "spectral_expert_gemv_amd", "csrc")
    hs = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")):
            hs.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                hs.update(f.read())
    return hs.hexdigest()[:16]


def traffic_for(workload):
    t = TRAFFIC.get(workload)
    return t[0] if t and t[1] == kernel_source_hash() else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="qwen3_30b_a3b_t1")
    ap.add_argument("--copies", type=int, default=0, help="layer copies rotated (0: auto)")
    ap.add_argument("--batches", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the bench, copy a tensor of this many MiB 4 times "
                         "(reference dispatches for HBM byte counters)")
    return ap.parse_args()


def layer_bytes_per_expert(bits, dout):
    """Algorithmic bytes of one expert of one linear type (E vector).

    bit planes (dout_pad * sum b / 8) + fp16 values of 16-bit columns +
    10 bytes of metadata per stored column (u16 k, fp16 s, fp16 m, fp32 a);
    dout_pad = dout rounded up to the 32-row segment.  Padding slots of the
    packed format are not counted.
    """
    dout_pad = (dout + 31) // 32 * 32
    b = bits.astype(np.int64)
    q = np.where((b >= 1) & (b <= 8), b, 0).sum(axis=1)
    n16 = (b == 16).sum(axis=1)
    nnz = (b > 0).sum(axis=1)
    return dout_pad * q // 8 + 2 * dout_pad * n16 + 10 * nnz


def step_bytes(spec, per_e_g, per_e_u, ids):
    distinct = np.unique(ids)
    T, k = ids.shape
    phi = 2 * spec.r * spec.din * 2
    experts = int(per_e_g[distinct].sum() + per_e_u[distinct].sum())
    xh = T * spec.din * 2 + T * k * spec.dout * 4 + T * k * 4
    return phi + experts + xh, phi, experts


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layer, batches, seconds):
    """The plain C oracle (oracle/ref_decode.c) on the host cores: z = Phi^T x,
    every routed expert's codes read back from its bit planes, the ordered
    k sums and SiLU*mul, all in float64, from blobs written by the oracle's
    own packer.  A token sample sized to ~`seconds` of work is timed with 1
    thread and with every core the process may use, 3 runs each (median)."""
    from oracle import build_ref, fmt, ref_c
    if not os.path.exists(ref_c.LIB_PATH):
        build_ref.build()
    spec = layer.spec
    blobs = [np.frombuffer(fmt.pack(layer.p[p], layer.a[p], layer.bits[p]), np.uint8)
             for p in ("gate", "up")]
    phi_t = np.ascontiguousarray(np.concatenate([np.asarray(layer.phi["gate"], np.float16).T,
                                                 np.asarray(layer.phi["up"], np.float16).T]))
    x = np.concatenate([b[0] for b in batches])
    ids = np.concatenate([b[1] for b in batches])
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():   # the host's share for this job
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))

    def run(n, threads):
        t0 = time.perf_counter()
        ref_c.gateup(blobs[0], blobs[1], phi_t, x[:n], ids[:n], spec.E, spec.dout, spec.r,
                     threads=threads)
        return time.perf_counter() - t0

    t1 = run(1, 1)
    # 3 single-thread and 3 all-core runs of n tokens within ~seconds
    n = int(max(1, min(len(x), seconds / (3.0 * t1 * (1.0 + 1.0 / cores)))))
    one = sorted(run(n, 1) for _ in range(3))[1]
    allc = sorted(run(n, cores) for _ in range(3))[1]
    return {"value": round(allc / n * 1e6, 1), "unit": "µs/token", "cores": int(cores),
            "kind": "oracle", "tokens_per_s": round(n / allc, 2),
            "one_core": {"value": round(one / n * 1e6, 1), "unit": "µs/token", "cores": 1},
            "cpu_model": _cpu_model(),
            "sample": "%d token(s) of the same workload (routed experts decoded from the "
                      "packed planes each time) through the plain C float64 oracle "
                      "(gcc -O2, OpenMP over tokens and pairs); median of 3 runs on %d "
                      "threads and of 3 on 1 thread" % (n, cores)}


def bench_pack(args):
    """Device packer on one projection of a full layer: p and a resident in
    HBM, widths on the host; each call returns with the blob complete (it
    synchronizes), so the wall time of the call is the measure."""
    import time

    import torch
    import synth
    from oracle import fmt
    from spectral_expert_gemv_amd import bitsmoe

    name = args.workload[len("pack_"):]
    spec = synth.LAYERS[name]
    L = synth.make_layer(spec)
    dev = torch.device("cuda:0")
    p, a, bits = L.p["gate"], L.a["gate"], L.bits["gate"]
    pd = torch.from_numpy(np.ascontiguousarray(p)).to(dev)
    ad = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    n = bitsmoe.pack_size(spec.E, spec.dout, spec.r, bits)
    out = torch.empty(n, dtype=torch.uint8, device=dev)
    ws = torch.empty(bitsmoe.pack_device_workspace_size(spec.E, spec.dout, spec.r, bits),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    K, W = max(1, args.steps), args.warmup
    for _ in range(W):
        bitsmoe.pack_device(pd, ad, bits, out=out, ws=ws, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        bitsmoe.pack_device(pd, ad, bits, out=out, ws=ws, stream=stream)
    ms = (time.perf_counter() - t0) * 1e3 / K
    stored = int((bits > 0).sum())
    alg = stored * spec.dout * 4 + bits.size * 4 + n     # read stored p and a, write the blob
    gbs = alg / (ms * 1e-3) / 1e9
    res = {
        "metric": "device_pack_ms", "value": round(ms, 4), "unit": "ms/projection",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "E": spec.E, "dout": spec.dout, "r": spec.r,
                   "stored_columns": stored, "blob_bytes": n,
                   "inputs": "fp32 p and a in HBM, widths on the host"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": alg,
                     "note": "whole call (planning, copies, pack and checksum kernels, "
                             "host fold of the checksum) over the algorithmic bytes"},
    }
    if not args.no_cpu:
        # the oracle packer on a sample of experts, scaled to the layer
        ne = 4
        t0 = time.perf_counter()
        fmt.pack(p[:ne], a[:ne], bits[:ne])
        el = time.perf_counter() - t0
        t0 = time.perf_counter()
        bitsmoe.pack(p, a, bits)
        host_ms = (time.perf_counter() - t0) * 1e3
        res["cpu_baseline"] = {"value": round(el * 1e3 * spec.E / ne, 1), "unit": "ms/projection",
                               "cores": 1, "kind": "oracle",
                               "sample": "numpy oracle packer on %d of %d experts (%.2f s), "
                                         "scaled to the layer" % (ne, spec.E, el),
                               "host_library_packer_ms": round(host_ms, 1)}
    print(json.dumps(res, ensure_ascii=False), flush=True)


def bench_fqcm(args):
    """FQCM inputs and the allocation for one projection of a full layer:
    eps of every column, beta from 512 calibration tokens (z = Phi^T x on
    the device, the workload's routing, uniform weights) and the Lagrangian
    allocation under the synthetic layer's own bit total.  p, a, x resident
    in HBM; each part timed with events on its stream (the allocation
    synchronizes once per bisection step, so its wall time is used)."""
    import time

    import torch
    import synth
    from oracle import fqcm
    from spectral_expert_gemv_amd import bitsmoe

    name = args.workload[len("fqcm_"):]
    spec = synth.LAYERS[name]
    L = synth.make_layer(spec)
    dev = torch.device("cuda:0")
    P, a, bits = L.p["gate"], L.a["gate"], L.bits["gate"]
    pd = torch.from_numpy(np.ascontiguousarray(P)).to(dev)
    ad = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    wl = [w for w in synth.WORKLOADS.values() if w.layer.name == name and w.T > 1]
    wl = wl[0] if wl else synth.workload(name + "_t1")
    xs, idss = [], []
    while sum(x.shape[0] for x in xs) < 512:
        x, ids = synth.make_batch(wl, L, step=len(xs))
        xs.append(x)
        idss.append(ids)
    x = np.concatenate(xs)[:512]
    ids = np.concatenate(idss)[:512].astype(np.int32)
    T = x.shape[0]
    phi_t = torch.from_numpy(np.ascontiguousarray(np.asarray(L.phi["gate"], np.float16).T)).to(dev)
    z = torch.empty((T, spec.r), dtype=torch.float32, device=dev)
    bitsmoe.spectral_proj(phi_t, torch.from_numpy(x).to(dev), z)
    idd = torch.from_numpy(ids).to(dev)
    g = torch.full(ids.shape, 1.0 / ids.shape[1], dtype=torch.float32, device=dev)
    eps = torch.empty((spec.E, spec.r, 8), dtype=torch.float64, device=dev)
    beta = torch.empty((spec.E, spec.r), dtype=torch.float64, device=dev)
    budget = int(bits.astype(np.int64).sum()) * spec.dout
    stream = torch.cuda.Stream(device=dev)
    K, W = max(1, args.steps), args.warmup

    def timed(fn):
        for _ in range(W):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(K):
                fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    ms_eps = timed(lambda: bitsmoe.fqcm_distortion(pd, eps=eps, stream=stream))
    ms_beta = timed(lambda: bitsmoe.fqcm_beta(z, idd, g, spec.E, beta=beta, stream=stream))
    out_bits = torch.empty((spec.E, spec.r), dtype=torch.uint8, device=dev)
    for _ in range(W):
        bitsmoe.fqcm_allocate(ad, beta, eps, spec.dout, budget, bits=out_bits, stream=stream)
    t0 = time.perf_counter()
    for _ in range(K):
        res = bitsmoe.fqcm_allocate(ad, beta, eps, spec.dout, budget, bits=out_bits,
                                    stream=stream)
    ms_alloc = (time.perf_counter() - t0) * 1e3 / K
    ncol = spec.E * spec.r
    eps_bytes = ncol * spec.dout * 4 + ncol * 8 * 8
    gbs = eps_bytes / (ms_eps * 1e-3) / 1e9
    total = ms_eps + ms_beta + ms_alloc
    out = {
        "metric": "fqcm_allocation_ms", "value": round(total, 4), "unit": "ms/projection",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(total, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": args.workload, "E": spec.E, "dout": spec.dout, "r": spec.r,
                   "calibration_tokens": T, "budget_bits": budget,
                   "bits_used": int(res[2]), "lambda": res[1], "lp_gap": res[3]},
        "parts_ms": {"distortion": round(ms_eps, 4), "beta": round(ms_beta, 4),
                     "allocate": round(ms_alloc, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": eps_bytes, "kernel": "k_fqcm_eps",
                     "launch_us_avg": round(ms_eps * 1e3, 2)},
    }
    if not args.no_cpu:
        # the oracle on a sample: eps of 512 columns, then the allocation
        # over the whole layer from the device inputs' shapes (seeded values)
        ne = 512
        flat = P.reshape(-1, spec.dout)
        t0 = time.perf_counter()
        fqcm.distortion(flat[:ne])
        el_eps = (time.perf_counter() - t0) * ncol / ne
        t0 = time.perf_counter()
        fqcm.beta(z.cpu().numpy()[:64], ids[:64], np.full((64, ids.shape[1]), 1.0 / ids.shape[1],
                                                          np.float32), spec.E)
        el_beta = (time.perf_counter() - t0) * T / 64
        # the exact allocation's dynamic program costs columns x budget units,
        # i.e. grows with the square of the columns: a 2048-column sample with
        # the same bits per column, scaled by (ncol / 2048)^2
        na = 2048
        a_s = np.asarray(a).reshape(-1)[:na]
        b_s = beta.cpu().numpy().reshape(-1)[:na]
        e_s = eps.cpu().numpy().reshape(-1, 8)[:na]
        t0 = time.perf_counter()
        fqcm.allocate(a_s, b_s, e_s, spec.dout, budget * len(a_s) // ncol)
        el_alloc = (time.perf_counter() - t0) * (ncol / len(a_s)) ** 2
        out["cpu_baseline"] = {
            "value": round((el_eps + el_beta + el_alloc) * 1e3, 1), "unit": "ms/projection",
            "cores": 1, "kind": "oracle",
            "sample": "numpy oracle: distortion of %d columns scaled to %d, beta of 64 tokens "
                      "scaled to %d, the exact allocation of %d columns (same bits per column) "
                      "scaled by the square of the column ratio" % (ne, ncol, T, len(a_s))}
    print(json.dumps(out, ensure_ascii=False), flush=True)


def bench_down(args):
    """Down projection + routing-weighted combine for the tokens of a
    gate/up workload (down_<workload>): the layer's down blob and Phi_down
    rotated over enough copies that >= 1 GiB is touched between two uses of
    one copy, h (the gate/up output shape) resident; K back-to-back calls
    timed with events on the launch stream."""
    import time

    import torch
    import synth
    from oracle import path
    from oracle.quantize import quantize_expert
    from spectral_expert_gemv_amd import bitsmoe

    wl = synth.workload(args.workload[len("down_"):])
    spec = wl.layer
    L = synth.make_layer(spec)
    D = synth.make_down(L)
    rd = D.phi.shape[1]
    dev = torch.device("cuda:0")
    blob = bitsmoe.pack(D.p, D.a, D.bits)
    phi16 = np.asarray(D.phi, np.float16)
    phit = np.ascontiguousarray(phi16.T)
    per_e = layer_bytes_per_expert(D.bits, spec.din)
    NB = max(1, args.batches)
    host = []
    for i in range(NB):
        _, ids = synth.make_batch(wl, L, step=i)
        g = synth.make_gates(wl, L, step=i)
        h = (np.random.default_rng(1000 + i).standard_normal((wl.T, spec.k, spec.dout)) * 0.3
             ).astype(np.float32)
        host.append((h, ids.astype(np.int32), g))
    T, k = host[0][1].shape
    alg = [rd * spec.dout * 2 + int(per_e[np.unique(ids)].sum()) + h.nbytes + ids.nbytes +
           g.nbytes + T * spec.din * 4 for h, ids, g in host]
    C = args.copies or max(2, min(64, math.ceil((1 << 30) / (blob.nbytes + phit.nbytes))))
    copies = [(torch.from_numpy(blob).to(dev), torch.from_numpy(phit).to(dev)) for _ in range(C)]
    dbat = [tuple(torch.from_numpy(a).to(dev) for a in b) for b in host]
    out = torch.empty((T, spec.din), dtype=torch.float32, device=dev)
    ws = torch.empty(bitsmoe.moe_down_workspace_size(T, k, spec.E, spec.dout, spec.din, rd),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step(i):
        bl, ph = copies[i % C]
        h, ids, g = dbat[i % NB]
        bitsmoe.moe_down(bl, ph, h, ids, g, spec.E, spec.din, rd, out=out, ws=ws, stream=stream)

    K, W = args.steps, args.warmup
    with torch.cuda.stream(stream):
        for i in range(W):
            step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(K):
            step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    avg = sum(alg[i % NB] for i in range(K)) / K
    gbs = avg / (ms * 1e-3) / 1e9
    res = {
        "metric": "down_combine_us_per_token", "value": round(ms * 1e3 / T, 4),
        "unit": "µs/token", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "E": spec.E, "din": spec.din, "dout": spec.dout,
                   "r_down": rd, "top_k": spec.k, "tokens": T, "layer_copies": C,
                   "inputs": "fp32 h (rounded to fp16), fp16 Phi_down, packed down directions"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": round(avg),
                     "note": "one call = fp16 cast, projection, expert apply, combine"},
    }
    if not args.no_cpu:
        h, ids, g = host[0]
        t0 = time.perf_counter()
        phat = np.zeros((spec.E, rd, spec.din))
        for e in np.unique(ids):
            phat[e] = quantize_expert(D.p[e], D.bits[e])["phat"]
        path.moe_down(phi16, D.a, phat, D.bits, h, ids, g)
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(el * 1e6 / T, 1), "unit": "µs/token", "cores": 1,
                               "kind": "oracle",
                               "sample": "one batch of %d token(s) through the float64 oracle "
                                         "(dequantize routed experts, z per pair, expert "
                                         "products, combine): %.2f s" % (T, el)}
    print(json.dumps(res, ensure_ascii=False), flush=True)


def bench_ssd(args):
    """Shared-basis decomposition of one linear type at a layer's full size
    (ssd_<layer>): a seeded Gaussian dense stack W (E x dout x din float32)
    resident in HBM, r = din; one call (it synchronizes once per Jacobi
    sweep) timed on the wall clock."""
    import time

    import torch
    import synth
    from oracle import ssd as ossd
    from spectral_expert_gemv_amd import bitsmoe

    spec = synth.LAYERS[args.workload[len("ssd_"):]]
    E, dout, din = spec.E, spec.dout, spec.din
    rng = np.random.default_rng(2024)
    W = rng.standard_normal((E, dout, din), dtype=np.float32)
    dev = torch.device("cuda:0")
    Wd = torch.from_numpy(W).to(dev)
    ws = torch.empty(bitsmoe.ssd_workspace_size(E, dout, din, din), dtype=torch.uint8,
                     device=dev)
    K = max(1, min(args.steps, 3))
    if args.warmup:
        bitsmoe.ssd(Wd, din, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        phi, a, p, s2, sweeps = bitsmoe.ssd(Wd, din, ws=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    # float64 flops: Gram matrix and projection (2 x 2 E dout din^2) and the
    # rotations (per round 9 din^2: two 2 x 2 rotations of every element of
    # G, 6 flops, and one of every element of V, 3 flops; din - 1 rounds a
    # sweep)
    flop = 2 * 2.0 * E * dout * din * din + sweeps * (din - 1) * 9.0 * din * din
    tfs = flop / (ms * 1e-3) / 1e12
    res = {
        "metric": "ssd_ms", "value": round(ms, 2), "unit": "ms/projection", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 2),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": args.workload, "E": E, "dout": dout, "din": din, "r": din,
                   "jacobi_sweeps": sweeps, "inputs": "seeded N(0,1) dense W, float32"},
        "roofline": {"bound": "alu", "achieved": round(tfs, 3), "peak": 78.6,
                     "unit": "TFLOP/s", "frac": round(tfs / 78.6, 5), "traffic": None,
                     "flop": flop,
                     "note": "whole call over the float64 flops of the Gram matrix, the "
                             "projection and the Jacobi rotations, against the fp64 vector "
                             "peak"},
    }
    if not args.no_cpu:
        ne = max(1, min(E, 16))
        t0 = time.perf_counter()
        ossd.ssd(W[:ne].astype(np.float64))
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(el * 1e3 * E / ne, 1), "unit": "ms/projection",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or None,
                               "kind": "oracle",
                               "sample": "numpy SVD (LAPACK) of %d of %d experts' stack, "
                                         "%.2f s, scaled linearly in E" % (ne, E, el)}
    print(json.dumps(res, ensure_ascii=False), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.workload.startswith("pack_"):
        return bench_pack(args)
    if args.workload.startswith("fqcm_"):
        return bench_fqcm(args)
    if args.workload.startswith("down_"):
        return bench_down(args)
    if args.workload.startswith("ssd_"):
        return bench_ssd(args)
    import torch
    import synth
    from spectral_expert_gemv_amd import bitsmoe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = synth.workload(args.workload)
    spec = wl.layer
    L = synth.make_layer(spec)
    blob_g = bitsmoe.pack(L.p["gate"], L.a["gate"], L.bits["gate"])
    blob_u = bitsmoe.pack(L.p["up"], L.a["up"], L.bits["up"])
    phi_t = np.ascontiguousarray(np.concatenate([np.asarray(L.phi["gate"], np.float16).T,
                                                 np.asarray(L.phi["up"], np.float16).T]))
    per_g = layer_bytes_per_expert(L.bits["gate"], spec.dout)
    per_u = layer_bytes_per_expert(L.bits["up"], spec.dout)
    host_batches = [synth.make_batch(wl, L, step=i) for i in range(args.batches)]
    sb = [step_bytes(spec, per_g, per_u, ids) for _, ids in host_batches]
    # enough copies that >= 1 GiB is touched between two uses of one copy
    C = args.copies or max(2, min(64, math.ceil((1 << 30) / min(s[0] for s in sb))))
    copies = []
    for _ in range(C):
        copies.append((torch.from_numpy(blob_g).to(dev), torch.from_numpy(blob_u).to(dev),
                       torch.from_numpy(phi_t).to(dev)))
    batches = [(torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev))
               for x, ids in host_batches]
    T, k = host_batches[0][1].shape
    ws_bytes = bitsmoe.moe_gateup_workspace_size(T, k, spec.E, spec.din, spec.dout, spec.r)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    bitsmoe.workspace_init(ws)
    h = torch.empty((T, k, spec.dout), dtype=torch.float32, device=dev)

    def step(i, stream):
        bg, bu, ph = copies[i % C]
        x, ids = batches[i % len(batches)]
        bitsmoe.moe_gateup(bg, bu, ph, x, ids, spec.E, spec.dout, spec.r, h, ws, stream=stream)

    stream = torch.cuda.Stream(device=dev)
    S = C * len(batches) // math.gcd(C, len(batches))
    S = min(S, 256)

    def make_graph(n, start):
        if n == 0:
            return None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for i in range(n):          # eager run once before capture
                step(start + i, stream)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                step(start + i, stream.cuda_stream)
        return g

    def run(nsteps, start, graph_full, graph_rem):
        if args.no_graph:
            with torch.cuda.stream(stream):
                for i in range(nsteps):
                    step(start + i, stream)
            return
        for _ in range(nsteps // S):
            graph_full.replay()
        if nsteps % S:
            graph_rem.replay()

    # W warm-up steps from index 0, then LOOPS timed loops of exactly K
    # steps, each continuing the rotation where the last one stopped (loop j
    # starts at W + j K), so no timed loop starts on copies just touched;
    # the value is the median loop.
    LOOPS = 5
    K, W = args.steps, args.warmup
    starts = [W + j * K for j in range(LOOPS)]
    g_full = None if args.no_graph else make_graph(S, 0)
    g_rems = [None if args.no_graph else make_graph(K % S, st) for st in starts]
    g_wrem = None if args.no_graph else make_graph(W % S, 0)
    with torch.cuda.stream(stream):
        run(W, 0, g_full, g_wrem)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    loop_ms = []
    for j in range(LOOPS):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            run(K, starts[j], g_full, g_rems[j])
            ev1.record(stream)
        torch.cuda.synchronize()
        loop_ms.append(ev0.elapsed_time(ev1))
    jm = sorted(range(LOOPS), key=lambda j: loop_ms[j])[LOOPS // 2]
    ms = loop_ms[jm]
    ms_per_step = ms / K
    us_per_token = ms_per_step * 1000.0 / T

    # algorithmic bytes averaged over the steps timed (step i uses batch i % NB)
    if args.no_graph:
        idx = [starts[jm] + i for i in range(K)]
    else:
        idx = list(range(S)) * (K // S) + [starts[jm] + i for i in range(K % S)]
    avg_bytes = sum(sb[i % len(sb)][0] for i in idx) / K
    achieved = avg_bytes / (ms_per_step * 1e-3) / 1e9

    # The timed region is back-to-back launches of the step's kernel(s) on
    # `stream`: its per-launch average is the event time over K steps.
    kern_us = ms_per_step * 1000.0
    kern_bytes = avg_bytes
    kern_gbs = achieved

    # warm (single copy, MALL-resident) reference number, labelled as such
    warm_us = None
    if not args.no_graph:
        g_warm = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            step(0, stream)
        stream.synchronize()
        with torch.cuda.graph(g_warm, stream=stream):
            for _ in range(64):
                step(0, stream.cuda_stream)
        with torch.cuda.stream(stream):
            g_warm.replay()
            stream.synchronize()
            ev0.record(stream)
            for _ in range(5):
                g_warm.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        warm_us = ev0.elapsed_time(ev1) * 1000.0 / (5 * 64) / T

    out = {
        "metric": METRIC, "value": round(us_per_token, 4), "unit": "µs/token",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "E": spec.E, "din": spec.din, "dout": spec.dout,
                   "r": spec.r, "top_k": spec.k, "tokens": T, "layer_copies": C,
                   "batches": len(batches), "graph_steps": S,
                   "inputs": "fp16 Phi and x, packed 0..16-bit directions, fp32 h"},
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "timed_loops_us_per_token": [round(m * 1000.0 / K / T, 4) for m in loop_ms],
        "warm_mall_us_per_token": None if warm_us is None else round(warm_us, 4),
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(wl.name), "kernel_source_hash": kernel_source_hash(),
                     "bytes_per_launch": round(kern_bytes),
                     "phi_bytes": sb[0][1],
                     "expert_bytes_avg": round(sum(s[2] for s in sb) / len(sb)),
                     "launch_us_avg": round(kern_us, 3),
                     "kernel": (KERNEL_ONE_TOKEN if T == 1 and spec.r <= 2048 else
                                KERNEL_ONE_LAUNCH if T <= 4 else kernel_batched(T))},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(L, host_batches, args.cpu_seconds)
    print(json.dumps(out, ensure_ascii=False), flush=True)
    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):          # elementwise kernel: reads n bytes, writes n bytes
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print("copy calibration: 4 copies of %d MiB" % args.copy_calib_mib, file=sys.stderr)


if __name__ == "__main__":
    main()
