"""Benchmark of the fused channelwise tensor-product convolution on one MI355X.

One step = one fused TP-conv forward over the large synthetic graph (20,000
nodes, 600,000 edges, in-degree 30, dst-sorted; features
128x0e+128x1o+128x2e, edge harmonics l <= 3, per-edge weights, output types
0e+1o+2e): gather, all 13 paths, per-edge weights and the segmented
sum-scatter in one kernel launch.  Inputs are resident in HBM before the
timed region.  The symmetric contraction (second client, 50,000 atoms) and
the other layout are timed in the same run and reported in their own
objects; the oracle is timed on a bounded sample on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout ir_mul|mul_ir]

Prints one JSON line.
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

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published
FP32_VALU_PEAK_TFLOPS = 78.6      # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz (a 16-lane derivation)
FP32_PUBLISHED_TFLOPS = 157.3     # MI355X published FP32 vector figure
FP32_MFMA_PEAK_TFLOPS = 157.3     # MI355X dense FP32 matrix, published
METRIC = "edges/sec + achieved HBM GB/s (fraction of peak) for fused equivariant TP-conv"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layout", default="ir_mul", choices=["ir_mul", "mul_ir"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the second layout and the symmetric contraction")
    p.add_argument("--with-backward", action="store_true",
                   help="time the backward on the same graph also under --no-extras")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for the HBM counter scale factor)")
    p.add_argument("--small-steps", type=int, default=200,
                   help="least number of timed calls of each small workload (fewer for counter runs)")
    p.add_argument("--no-eager", action="store_true",
                   help="skip the eager per-path PyTorch context of the medium graph (for counter runs)")
    return p.parse_args()


FWD_SOURCES = ("kernels/tp_conv_spec.hpp", "kernels/common.hpp", "codegen.cpp", "specs.txt",
               "tp_descriptor.cpp", "cg.cpp")
BWD_SOURCES = FWD_SOURCES + ("kernels/tp_conv_bwd.hpp",)


CODEGEN_SYMCON_MARK = b"// ---------------------------------------------------------------- symcon"


def kernel_source_hash(kind="fwd"):
    """Hash of everything the timed TP-conv kernels are generated from (of
    the generator, the part before its symmetric-contraction section), to
    tell whether stored hardware counters still describe them."""
    h = hashlib.sha256()
    base = os.path.join(ROOT, "segmented_polynomials_amd", "csrc")
    for rel in (FWD_SOURCES if kind == "fwd" else BWD_SOURCES):
        with open(os.path.join(base, rel), "rb") as f:
            data = f.read()
        if rel == "codegen.cpp":
            data = data.split(CODEGEN_SYMCON_MARK)[0]
        h.update(data)
    return h.hexdigest()[:16]


def stored_traffic(layout, kind="fwd"):
    """HBM bytes per call from the committed counter summary, or None if
    the summary is missing or was taken on different kernels."""
    name = "tp_conv" if kind == "fwd" else "tp_conv_bwd"
    path = os.path.join(ROOT, "profiles", f"{name}_large_graph_{layout}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    mh = re.search(r"kernel_source_hash:\s*(\w+)", text)
    mb = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not mh or not mb or mh.group(1) != kernel_source_hash(kind):
        return None
    return float(mb.group(1))


_T0 = time.perf_counter()


def note(what):
    """Progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {what} ({time.perf_counter() - _T0:.1f} s)", file=sys.stderr, flush=True)


def time_launches(torch, fn, steps, warmup):
    """Warm up, then time `steps` launches: total wall time bracketed by
    synchronisations, and per-launch HIP events on the launch stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(a.elapsed_time(b) for a, b in ev)   # ms
    return wall, per


def pattern_ceiling(torch, wl, h, x, sh, w, src, out, N, E, args):
    """Time the traffic replay of the conv on the large graph (same loads and
    stores as the fused kernel, trivial arithmetic): weight rows alone, with
    the output rows (plain and non-temporal stores), and the full traffic
    with the gathered source rows and harmonics.  None when the probe
    library is missing or the graph is not the uniform-degree one."""
    import ctypes
    path = os.path.join(ROOT, "segmented_polynomials_amd", "libsegpoly_bench.so")
    if not os.path.exists(path) or E != N * wl.degree:
        note("pattern ceiling skipped (probe library missing or non-uniform degree)")
        return None
    lib = ctypes.CDLL(path)
    fn = lib.segpoly_bench_traffic_replay
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int64,
                                                                          ctypes.c_int] + [ctypes.c_int64] * 4 + [
        ctypes.c_void_p]

    def run(mode, nt):
        stream = torch.cuda.current_stream().cuda_stream
        rc = fn(mode, nt, w.data_ptr(), x.data_ptr(), sh.data_ptr(), src.data_ptr(), out.data_ptr(), N,
                x.shape[0], wl.degree, h.weight_numel, h.dim_in1, h.dim_in2, h.dim_out, stream)
        if rc != 0:
            raise RuntimeError(f"traffic replay failed ({rc})")

    res = {"what": "the conv's loads and stores with trivial arithmetic, one wave per destination node"}
    steps = max(5, args.steps // 2)
    for key, mode, nt in (("weights_ms", 0, 0), ("weights_out_ms", 1, 0), ("weights_out_nt_ms", 1, 1),
                          ("full_ms", 2, 0), ("full_nt_ms", 2, 1)):
        _, per = time_launches(torch, lambda: run(mode, nt), steps, 2)
        res[key] = sum(per) / len(per)
    bytes_w = E * h.weight_numel * 4
    res["weights_GBps"] = bytes_w / (res["weights_ms"] * 1e-3) / 1e9
    note("pattern ceiling timed")
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU design is described, not built).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import segmented_polynomials_amd as sp
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[4]
    layout = args.layout
    t_create = time.perf_counter()
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=layout)
    create_ms = (time.perf_counter() - t_create) * 1e3
    fan_in = workloads.fan_in_from_irreps_out(h.irreps_out)
    inp = workloads.tp_inputs(wl, fan_in)
    N, E = inp["n_nodes"], inp["sh"].shape[0]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, sh, w = to(inp["x"]), to(inp["sh"]), to(inp["w"])
    src, dst = to(inp["src"]), to(inp["dst"])
    vec = to(inp["vec"])
    out = torch.empty((N, h.dim_out), dtype=torch.float32, device=dev)
    # keep only what the host-side baselines need (first destination nodes)
    sample_nodes, par_nodes = 1000, 4000
    par_e = par_nodes * wl.degree
    base_inp = dict(x=inp["x"], sh=inp["sh"][:par_e].copy(), w=inp["w"][:par_e].copy(),
                    src=inp["src"][:par_e].copy(), dst=inp["dst"][:par_e].copy(), n_nodes=par_nodes)
    del inp

    note("inputs ready")
    fwd = lambda: sp.tp_conv_fwd(h, x, sh, w, src, dst, n_nodes=N, out=out)
    wall, per = time_launches(torch, fwd, args.steps, args.warmup)
    note("forward timed")
    ms_per_step = wall * 1e3 / args.steps
    avg_kernel_ms = sum(per) / len(per)

    # algorithmic bytes per launch: every operand read or written once
    bytes_w = E * h.weight_numel * 4
    bytes_sh = E * h.dim_in2 * 4
    bytes_idx = 2 * E * 4
    bytes_x = N * h.dim_in1 * 4
    bytes_out = N * h.dim_out * 4
    alg_bytes = bytes_w + bytes_sh + bytes_idx + bytes_x + bytes_out
    alg_flops = E * (2 * h.mul * h.cg_nnz + h.mul * (h.dim_out // h.mul))
    achieved_gbps = alg_bytes / (avg_kernel_ms * 1e-3) / 1e9
    edges_per_s = E / (ms_per_step * 1e-3)
    traffic = stored_traffic(layout)

    result = {
        "metric": METRIC,
        "value": edges_per_s,
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "nodes": N, "edges": E, "in_degree": wl.degree,
                   "irreps_in1": wl.irreps_in1, "irreps_sh": wl.irreps_in2, "irreps_out": h.irreps_out,
                   "layout": layout, "index_dtype": "int32", "kernel": h.kernel_name},
        "hbm_GBps_algorithmic": achieved_gbps,
        "hbm_fraction_of_peak": achieved_gbps / HBM_PEAK_GBPS,
        "kernel_ms": {"mean": avg_kernel_ms, "min": per[0], "median": per[len(per) // 2]},
        "create_ms": create_ms,
        "roofline": {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "algorithmic_bytes_per_edge": alg_bytes / E,
                     "algorithmic_flops_per_launch": alg_flops},
    }

    if not args.no_extras:
        import gc
        # the other layout (same inputs reinterpreted: timing only)
        other = "mul_ir" if layout == "ir_mul" else "ir_mul"
        h2 = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=other)
        f2 = lambda: sp.tp_conv_fwd(h2, x, sh, w, src, dst, n_nodes=N, out=out)
        wall2, per2 = time_launches(torch, f2, args.steps, args.warmup)
        k2 = sum(per2) / len(per2)
        result[f"tp_conv_{other}"] = {"edges_per_s": E / (wall2 / args.steps), "kernel_ms": k2,
                                      "hbm_GBps_algorithmic": alg_bytes / (k2 * 1e-3) / 1e9,
                                      "hbm_fraction_of_peak": alg_bytes / (k2 * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                      "kernel": h2.kernel_name, "traffic": stored_traffic(other)}
    if not args.no_extras:
        # the harmonics computed in the kernel from the edge vectors, against
        # the two-call path (harmonics kernel, then the convolution)
        fv = lambda: sp.tp_conv_fwd_vec(h, x, vec, w, src, dst, n_nodes=N, out=out)
        wallv, perv = time_launches(torch, fv, args.steps, args.warmup)
        shbuf = torch.empty_like(sh)
        fs = lambda: sp.sh_fwd(vec, 3, out=shbuf)
        walls, pers = time_launches(torch, fs, args.steps, args.warmup)
        result["tp_conv_fused_sh"] = {"kernel_ms": sum(perv) / len(perv), "edges_per_s": E / (wallv / args.steps),
                                      "sh_kernel_ms": sum(pers) / len(pers),
                                      "two_call_ms": sum(pers) / len(pers) + avg_kernel_ms}
        del shbuf

        # one GPU's share of an eight-way destination split: the first eighth
        # of the destinations with their edges (dst-sorted: one contiguous
        # edge range) and the whole source table, as each GPU would run it
        # after the all-gather of x; algorithmic bytes count the source rows
        # its edges read once each
        n8 = N // 8
        e8 = int((dst < n8).sum().item())
        out8 = out[:n8]
        f8 = lambda: sp.tp_conv_fwd(h, x, sh[:e8], w[:e8], src[:e8], dst[:e8], n_nodes=n8, out=out8)
        wall8, per8 = time_launches(torch, f8, args.steps, args.warmup)
        k8 = sum(per8) / len(per8)
        rows8 = int(torch.unique(src[:e8]).numel())
        b8 = e8 * (h.weight_numel + h.dim_in2 + 2) * 4 + rows8 * h.dim_in1 * 4 + n8 * h.dim_out * 4
        result["shard_one_of_eight"] = {"what": "destinations [0, N/8) and their edges, whole source table",
                                        "nodes": n8, "edges": e8, "source_rows_read": rows8, "kernel_ms": k8,
                                        "edges_per_s": e8 / (wall8 / args.steps),
                                        "hbm_GBps_algorithmic": b8 / (k8 * 1e-3) / 1e9,
                                        "hbm_fraction_of_peak": b8 / (k8 * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        note("one-eighth shard timed")

        # practical ceiling: a plain device copy of the weight tensor (4 GB read + 4 GB written)
        wc = torch.empty_like(w)
        cwall, cper = time_launches(torch, lambda: wc.copy_(w), max(5, args.steps // 4), 2)
        cms = sum(cper) / len(cper)
        copy_gbps = 2 * w.numel() * 4 / (cms * 1e-3) / 1e9
        result["copy_ceiling"] = {"what": "device copy of the 3.99 GB weight tensor", "ms": cms,
                                  "GBps": copy_gbps, "frac_of_peak": copy_gbps / HBM_PEAK_GBPS}
        result["roofline"]["frac_of_copy"] = achieved_gbps / copy_gbps
        del wc

        # ceiling of the access pattern itself: the kernel's loads and stores
        # replayed with trivial arithmetic (libsegpoly_bench.so)
        rep = pattern_ceiling(torch, wl, h, x, sh, w, src, out, N, E, args)
        if rep is not None:
            result["pattern_ceiling"] = rep
            result["roofline"]["frac_of_pattern_ceiling"] = rep["full_ms"] / avg_kernel_ms

    if not args.no_extras or args.with_backward:
        del out
        other = "mul_ir" if layout == "ir_mul" else "ir_mul"
        hs = [h] if args.no_extras else [h, sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=other)]
        bw = backward(torch, sp, workloads, hs, x, sh, w, src, dst, N, E, args)
        result["tp_conv_bwd"] = bw[layout]
        if len(hs) > 1:
            result[f"tp_conv_bwd_{other}"] = bw[other]

    if not args.no_extras:
        import gc
        del x, sh, w, src, dst, vec
        gc.collect()
        torch.cuda.empty_cache()

        # symmetric contraction, 50,000 atoms
        s5 = workloads.WORKLOADS[5]
        hs = sp.symcon_create(s5.irreps_in, s5.irreps_out, 3, s5.num_elements, layout="ir_mul")
        k = {}
        for c in range(hs.num_couplings):
            i = hs.coupling_info(c)
            k[(i["degree"], i["out_block"])] = k.get((i["degree"], i["out_block"]), 0) + 1
        sfan = np.concatenate([np.full(hs.mul, k[(hs.coupling_info(c)["degree"], hs.coupling_info(c)["out_block"])])
                               for c in range(hs.num_couplings)])
        si = workloads.symcon_inputs(s5, sfan)
        sx, ssp, sw = to(si["x"]), to(si["species"]), to(si["w"])
        sout = torch.empty((s5.n_atoms, hs.dim_out), dtype=torch.float32, device=dev)
        fs = lambda: sp.symcon_fwd(hs, sx, ssp, sw, out=sout)
        wall3, per3 = time_launches(torch, fs, args.steps, args.warmup)
        k3 = sum(per3) / len(per3)
        A = s5.n_atoms
        s_bytes = A * hs.dim_in * 4 + A * hs.dim_out * 4 + A * 4 + s5.num_elements * hs.weight_numel * 4
        seg_out = sum(2 * hs.coupling_info(c)["l"] + 1 for c in range(hs.num_couplings))
        s_flops = A * hs.mul * (2 * hs.num_terms + hs.num_monomial_products + 2 * seg_out)
        result["symcon"] = {
            "workload": s5.name, "atoms_per_s": A / (wall3 / args.steps), "kernel_ms": k3,
            "kernel": "symcon_spec" if hs.specialized else "symcon_generic",
            "hbm": {"achieved": s_bytes / (k3 * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": s_bytes / (k3 * 1e-3) / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": s_bytes},
            "alu": {"achieved": s_flops / (k3 * 1e-3) / 1e12, "peak": FP32_PUBLISHED_TFLOPS, "unit": "TFLOP/s",
                    "frac": s_flops / (k3 * 1e-3) / 1e12 / FP32_PUBLISHED_TFLOPS, "algorithmic_flops": s_flops,
                    "peak_kind": "published MI355X FP32 vector figure; plain FP32 issues faster than a "
                                 "16-lane derivation (78.6 TFLOP/s) assumes: the counters show up to 0.36 "
                                 "wave64 VALU instructions per SIMD-cycle against its 0.25",
                    "frac_of_16_lane_derivation": s_flops / (k3 * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS},
        }
        # backward of the symmetric contraction on the same atoms
        sg = torch.from_numpy(workloads.output_gradient(s5.n_atoms, hs.dim_out, "f32", seed=59)).to(dev)
        sperm = torch.argsort(ssp, stable=True).to(ssp.dtype)
        sgx, sgw = torch.empty_like(sx), torch.empty_like(sw)
        sws = torch.empty(sp.symcon_bwd_workspace(hs, s5.n_atoms), dtype=torch.uint8, device=dev)
        fb = lambda: sp.symcon_bwd(hs, sx, ssp, sw, sg, sperm, workspace=sws, grad_x=sgx, grad_w=sgw)
        wall4, per4 = time_launches(torch, fb, args.steps, args.warmup)
        k4 = sum(per4) / len(per4)
        b_bytes = 2 * A * hs.dim_in * 4 + A * hs.dim_out * 4 + 2 * A * 4 + 2 * s5.num_elements * hs.weight_numel * 4
        result["symcon_bwd"] = {
            "atoms_per_s": A / (wall4 / args.steps), "ms_per_call": k4,
            "kernels": ["symcon_table_kernel", "symcon_bwd_kernel", "symcon_fold_kernel"],
            "hbm": {"achieved": b_bytes / (k4 * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": b_bytes / (k4 * 1e-3) / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": b_bytes}}
        del sx, ssp, sw, sout, sg, sperm, sgx, sgw, sws

    if not args.no_extras:
        note("convolution variants and symmetric contraction timed")
        result["other_workloads"] = other_workloads(torch, sp, workloads, dev, args)
        note("smaller workloads timed")
        result["linear"] = linear_layers(torch, sp, workloads, dev, args)
        note("linear layers timed")
        result["fctp"] = fc_product(torch, sp, workloads, dev, args)
        note("fully connected product timed")
        result["fctp_conv"] = fc_conv(torch, sp, workloads, dev, args)
        note("fully connected convolution timed")
        result["fctp_per_sample"] = fc_per_sample(torch, sp, workloads, dev, args)
        note("fully connected product with per-sample weights timed")

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"read": a.numel() * 4, "write": b.numel() * 4}
        del a, b

    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import tp as otp
        o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
        n_e = sample_nodes * wl.degree
        with threadpool_limits(1):
            t0 = time.perf_counter()
            o.conv(base_inp["x"], base_inp["sh"][:n_e], base_inp["w"][:n_e], base_inp["src"][:n_e],
                   base_inp["dst"][:n_e], sample_nodes, layout=layout)
            dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n_e / dt, "unit": "edges/s", "cores": 1, "kind": "oracle",
                                  "sample": f"first {sample_nodes} destination nodes of the same graph "
                                            f"({n_e} edges, all 13 paths), float64 NumPy, {dt:.1f} s",
                                  "host_cpu": _cpu_model(), "host_nproc": os.cpu_count()}
        note("oracle timed on one core")
        result["cpu_baseline_parallel"] = parallel_oracle(wl, base_inp, layout)
        note("oracle timed on all cores")
        if not args.no_extras:
            result["cpu_baseline_by_config"] = oracle_by_config(workloads)
            note("oracle timed on the other configurations")

    print(json.dumps(result), flush=True)


def _oracle_warm(_):
    """Start-up of a parallel-oracle worker: the imports, then a short wait
    so that every worker takes one of these tasks."""
    import threadpoolctl  # noqa: F401

    import oracle.symcon  # noqa: F401
    import oracle.tp  # noqa: F401
    time.sleep(0.5)
    return os.getpid()


_SYMCON_CACHE = {}


def _symcon_object(irreps):
    from oracle import symcon as osym
    if irreps not in _SYMCON_CACHE:
        _SYMCON_CACHE[irreps] = osym.SymmetricContraction(*irreps)
    return _SYMCON_CACHE[irreps]


def _symcon_prepare(irreps):
    """Build the oracle's contraction in a worker before the timed run (its
    basis construction is set-up, not evaluation), then wait so that every
    worker takes one of these tasks."""
    _symcon_object(irreps)
    time.sleep(0.5)
    return os.getpid()


def _symcon_chunk(a):
    """One worker of the parallel symmetric-contraction oracle run."""
    from threadpoolctl import threadpool_limits

    irreps, x, species, w, layout = a
    so = _symcon_object(irreps)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        so.eval(x, species, w, layout=layout)
        return time.perf_counter() - t0


def _oracle_chunk(a):
    """One worker of the parallel oracle run: the destinations [n0, n1)."""
    from threadpoolctl import threadpool_limits

    from oracle import tp as otp
    irreps, x, sh, w, src, dst, n0, n1, layout = a
    o = otp.ChannelwiseTP(*irreps)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        o.conv(x, sh, w, src, dst - n0, n1 - n0, layout=layout)
        return time.perf_counter() - t0


def parallel_oracle(wl, inp, layout):
    """The oracle as it stands, split by destination range over the host
    cores (at most 16 worker processes); wall time from handing out the
    chunks to the last result (worker start-up excluded)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np
    workers = max(1, min(16, os.cpu_count() or 1))
    n, deg = inp["n_nodes"], wl.degree
    bounds = np.linspace(0, n, workers + 1).astype(int)
    chunks = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        e0, e1 = a * deg, b * deg
        # each worker receives only the source rows its edges read (renumbered)
        rows, src_local = np.unique(inp["src"][e0:e1], return_inverse=True)
        chunks.append(((wl.irreps_in1, wl.irreps_in2, wl.irreps_out), inp["x"][rows], inp["sh"][e0:e1],
                       inp["w"][e0:e1], src_local, inp["dst"][e0:e1], int(a), int(b), layout))
    ex = cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))
    try:
        list(ex.map(_oracle_warm, range(workers), timeout=120))   # start the workers
        t0 = time.perf_counter()
        list(ex.map(_oracle_chunk, chunks, timeout=300))
        wall = time.perf_counter() - t0
    except Exception as err:   # a worker that cannot start must not cost the bench line
        ex.shutdown(wait=False, cancel_futures=True)
        return {"error": f"{type(err).__name__}: {err}"}
    ex.shutdown()
    e = n * deg
    return {"value": e / wall, "unit": "edges/s", "cores": workers, "kind": "oracle",
            "sample": f"first {n} destination nodes of the same graph ({e} edges) split by destination range "
                      f"over {workers} processes of one thread each, {wall:.1f} s"}


def _tp_dst_chunks(wl, inp, layout, parts):
    """Split a dst-sorted graph into `parts` destination ranges; each chunk
    carries only the source rows its edges read (renumbered)."""
    import numpy as np
    n, dst = inp["n_nodes"], inp["dst"]
    bounds = np.linspace(0, n, parts + 1).astype(int)
    chunks = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        e0, e1 = int(np.searchsorted(dst, a)), int(np.searchsorted(dst, b))
        rows, src_local = np.unique(inp["src"][e0:e1], return_inverse=True)
        chunks.append(((wl.irreps_in1, wl.irreps_in2, wl.irreps_out), inp["x"][rows], inp["sh"][e0:e1],
                       inp["w"][e0:e1], src_local.astype(np.int64), dst[e0:e1], int(a), int(b), layout))
    return chunks


def oracle_by_config(workloads):
    """The oracle as it stands on the other configurations (float64 NumPy):
    one core (median of three runs for the batch and the molecules, one run
    for the 2k-node graph, a bounded sample of the 50k-atom contraction), and
    the same work split over the host cores (at most 16 processes of one
    thread each, by destination range or atom range; worker start-up not
    timed).  Context only: the oracle is the correctness reference."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import symcon as osym, tp as otp
    workers = max(1, min(16, os.cpu_count() or 1))
    ex = cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))
    res = {"host_cpu": _cpu_model(), "host_nproc": os.cpu_count()}
    try:
        list(ex.map(_oracle_warm, range(workers), timeout=120))
        for n in (1, 2, 3):
            wl = workloads.WORKLOADS[n]
            o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
            inp = workloads.tp_inputs(wl, o.weight_fan_in())
            lay = wl.layouts[0]
            E = inp["sh"].shape[0]
            runs = 3 if n in (1, 2) else 1
            times = []
            with threadpool_limits(1):
                for _ in range(runs):
                    t0 = time.perf_counter()
                    o.conv(inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], layout=lay)
                    times.append(time.perf_counter() - t0)
            dt = sorted(times)[len(times) // 2]
            rec = {"workload": wl.name, "edges": E,
                   "one_core": {"s": dt, "value": E / dt, "unit": "edges/s", "cores": 1,
                                "sample": f"whole workload, {'median of 3 runs' if runs == 3 else 'one run'}"}}
            if inp["src"] is not None:
                chunks = _tp_dst_chunks(wl, inp, lay, workers)
                t0 = time.perf_counter()
                list(ex.map(_oracle_chunk, chunks, timeout=300))
                wall = time.perf_counter() - t0
                rec["all_cores"] = {"s": wall, "value": E / wall, "unit": "edges/s", "cores": workers,
                                    "sample": f"whole workload split by destination range over {workers} processes"}
            res[wl.name] = rec
            note(f"oracle timed on {wl.name}")
        s5 = workloads.WORKLOADS[5]
        so = osym.SymmetricContraction(s5.irreps_in, s5.irreps_out)
        per_worker, one = 500, 1000
        si = workloads.symcon_inputs(s5, so.weight_fan_in(), n_atoms=max(one, workers * per_worker))
        with threadpool_limits(1):
            t0 = time.perf_counter()
            so.eval(si["x"][:one], si["species"][:one], si["w"], layout="ir_mul")
            dt = time.perf_counter() - t0
        rec = {"workload": s5.name,
               "one_core": {"s": dt, "value": one / dt, "unit": "atoms/s", "cores": 1,
                            "sample": f"first {one} of the {s5.n_atoms} atoms, ir_mul"}}
        list(ex.map(_symcon_prepare, [(s5.irreps_in, s5.irreps_out)] * workers, timeout=300))
        chunks = [((s5.irreps_in, s5.irreps_out), si["x"][k * per_worker:(k + 1) * per_worker],
                   si["species"][k * per_worker:(k + 1) * per_worker], si["w"], "ir_mul") for k in range(workers)]
        t0 = time.perf_counter()
        list(ex.map(_symcon_chunk, chunks, timeout=300))
        wall = time.perf_counter() - t0
        rec["all_cores"] = {"s": wall, "value": workers * per_worker / wall, "unit": "atoms/s", "cores": workers,
                            "sample": f"first {workers * per_worker} atoms, {per_worker} per process"}
        res[s5.name] = rec
    except Exception as err:   # a worker that cannot start must not cost the bench line
        ex.shutdown(wait=False, cancel_futures=True)
        res["error"] = f"{type(err).__name__}: {err}"
        return res
    ex.shutdown()
    return res


def backward(torch, sp, workloads, hs, x, sh, w, src, dst, N, E, args):
    """Vector-Jacobian product on the same graph, both kernels per call, for
    each handle of ``hs`` (one per layout).  The roofline counts the
    operands and gradients once each (x, g and dx per node; w, sh, dw, dsh
    and the three index arrays per edge).  The per-edge source messages that
    the first kernel writes and the second reads back are this design's own
    workspace round trip, not algorithmic bytes: they are reported beside
    the roofline as overhead, with the counter traffic over the operands."""
    g = torch.from_numpy(workloads.output_gradient(N, hs[0].dim_out, "f32", seed=74)).to(x.device)
    perm = torch.argsort(src, stable=True).to(src.dtype)
    gx, gsh, gw = torch.empty_like(x), torch.empty_like(sh), torch.empty_like(w)
    ws = torch.empty(sp.tp_conv_bwd_workspace(hs[0], E), dtype=torch.uint8, device=x.device)
    res = {}
    for h in hs:
        fb = lambda: sp.tp_conv_bwd(h, x, sh, w, g, src, dst, perm, n_nodes=N, workspace=ws,
                                    grad_x=gx, grad_sh=gsh, grad_w=gw)
        wall, per = time_launches(torch, fb, args.steps, args.warmup)
        kms = sum(per) / len(per)
        operands = (2 * E * h.weight_numel * 4 + 2 * E * h.dim_in2 * 4 + 3 * E * 4 +
                    2 * N * h.dim_in1 * 4 + N * h.dim_out * 4)
        messages = 2 * E * h.dim_in1 * 4
        gbps = operands / (kms * 1e-3) / 1e9
        traffic = stored_traffic(h.layout, "bwd")
        res[h.layout] = {
            "edges_per_s": E / (wall / args.steps), "ms_per_call": kms,
            "hbm": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": gbps / HBM_PEAK_GBPS, "algorithmic_bytes": operands, "traffic": traffic,
                    "traffic_over_algorithmic": None if traffic is None else traffic / operands},
            "design_overhead": {"what": "per-edge source messages written by the edge kernel and read back by "
                                        "the source kernel (workspace round trip, not counted above)",
                                "bytes": messages,
                                "GBps_with_overhead": (operands + messages) / (kms * 1e-3) / 1e9},
            "kernels": ["tp_bwd_edge_kernel", "tp_bwd_src_kernel"]}
        note(f"backward {h.layout} timed")
    del g, perm, gx, gsh, gw, ws
    return res


def linear_layers(torch, sp, workloads, dev, args):
    """The equivariant linear layers on the matrix cores: the layer after
    the 600k-edge convolution (shared weights; forward and backward) and
    the species-indexed layer on 50k atoms (10 sorted classes).  flops =
    2 * sum over weight segments of mul_in * mul_out * (2l + 1) per sample
    (the dense products; the backward does twice that)."""
    import numpy as np

    from oracle import irreps as oir   # sizes only: block multiplicities and l
    res = {}
    for num in (6, 7):
        wl = workloads.WORKLOADS[num]
        h = sp.linear_create(wl.irreps_in, wl.irreps_out, layout=wl.layouts[0])
        inp = workloads.linear_inputs(wl, h.weight_numel)
        x, w = (torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev) for k in ("x", "w"))
        cls = None if inp["classes"] is None else torch.from_numpy(inp["classes"]).to(dev)
        out = torch.empty((wl.n, h.dim_out), dtype=torch.float32, device=dev)
        f = lambda: sp.linear_fwd(h, x, w, classes=cls, out=out)
        wall, per = time_launches(torch, f, args.steps, args.warmup)
        kms = sum(per) / len(per)
        blocks_in, blocks_out = oir.parse(wl.irreps_in), oir.parse(wl.irreps_out)
        macs = sum(mi * mo * (2 * li + 1) for mi, li, pi in blocks_in for mo, lo, po in blocks_out
                   if (li, pi) == (lo, po))
        flops = 2.0 * macs * wl.n
        nbytes = (h.dim_in + h.dim_out) * wl.n * 4 + w.numel() * 4 + (0 if cls is None else wl.n * 4)
        tf = flops / (kms * 1e-3) / 1e12
        r = {"workload": wl.name, "layout": wl.layouts[0], "samples": wl.n, "ms_per_call": kms,
             "samples_per_s": wl.n / (wall / args.steps),
             "roofline": {"bound": "mfma", "achieved": tf, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": tf / FP32_MFMA_PEAK_TFLOPS, "algorithmic_flops": flops},
             "hbm": {"achieved": nbytes / (kms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "algorithmic_bytes": nbytes}}
        # backward: dx and dW (one weight row per class with classes)
        nc = 0 if cls is None else w.shape[0]
        g = torch.from_numpy(workloads.output_gradient(wl.n, h.dim_out, "f32", seed=66)).to(dev)
        ws = torch.empty(max(1, sp.linear_bwd_workspace(h, wl.n, nc)), dtype=torch.uint8, device=dev)
        fb = lambda: sp.linear_bwd(h, x, w, g, classes=cls, num_classes=nc or None, workspace=ws)
        wallb, perb = time_launches(torch, fb, args.steps, args.warmup)
        kb = sum(perb) / len(perb)
        tfb = 2 * flops / (kb * 1e-3) / 1e12
        r["backward"] = {"ms_per_call": kb, "roofline": {"bound": "mfma", "achieved": tfb,
                                                        "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                                        "frac": tfb / FP32_MFMA_PEAK_TFLOPS}}
        del g, ws
        r["library_gemm_reference"] = library_gemm_reference(torch, dev, args, wl, blocks_in, blocks_out, flops)
        res[wl.name] = r
        del x, w, out, cls
    return res


def library_gemm_reference(torch, dev, args, wl, blocks_in, blocks_out, flops):
    """What the vendor BLAS (torch.mm on ROCm: hipBLASLt / rocBLAS, float32,
    no reduced-precision modes) reaches on the same dense products: one
    [n (2l+1), K] x [K, mul_out] GEMM per output block, K = the input
    channels of its type, with one shared weight matrix.  A measuring stick
    for the hand-written kernels on these tall, short-K shapes, never part
    of the layer's path (and for the species-indexed layer a lower bound of
    its work: it ignores the per-class weights)."""
    torch.backends.cuda.matmul.allow_tf32 = False
    mats = []
    for mo, lo, po in blocks_out:
        k = sum(mi for mi, li, pi in blocks_in if (li, pi) == (lo, po))
        if k == 0:
            continue
        m = wl.n * (2 * lo + 1)
        mats.append((torch.randn(m, k, device=dev), torch.randn(k, mo, device=dev), torch.empty(m, mo, device=dev)))
    f = lambda: [torch.mm(a, b, out=c) for a, b, c in mats]
    wall, per = time_launches(torch, f, args.steps, args.warmup)
    ms = sum(per) / len(per)
    tf = flops / (ms * 1e-3) / 1e12
    del mats
    return {"ms_per_call": ms, "shapes": "one GEMM per output block, shared weights",
            "roofline": {"bound": "mfma", "achieved": tf, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / FP32_MFMA_PEAK_TFLOPS}}


def fc_product(torch, sp, workloads, dev, args):
    """The fully connected (uvw) product on the matrix cores, 100k samples
    of 32x0e+32x1o x 32x0e+32x1o -> 32x0e+32x1o, both layouts.  Algorithmic
    flops: the dense contraction over (u, v) of each path, 2 * d_o * mul1 *
    mul2 * mul3 per sample (the couplings that build its operand are not
    counted); the backward's three products (dx1, dx2, dW) count
    2 * (d1 + d2 + d_o) * mul1 * mul2 * mul3."""
    import numpy as np

    from oracle import fctp as ofc   # sizes only: the path list
    wl = workloads.WORKLOADS[8]
    f = ofc.FullyConnectedTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    fwd_macs = bwd_macs = 0
    for i, j, o, _ in f.paths:
        (m1, l1, _), (m2, l2, _), (m3, l3, _) = f.in1[i], f.in2[j], f.out[o]
        fwd_macs += (2 * l3 + 1) * m1 * m2 * m3
        bwd_macs += (2 * l1 + 1 + 2 * l2 + 1 + 2 * l3 + 1) * m1 * m2 * m3
    res = {}
    for lay in wl.layouts:
        h = sp.fctp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=lay, dtype=wl.dtype)
        inp = workloads.fc_inputs(wl, h.weight_numel)
        x1, x2, w = (torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev) for k in ("x1", "x2", "w"))
        g = torch.from_numpy(workloads.output_gradient(wl.n, h.dim_out, wl.dtype, seed=2008)).to(dev)
        out = torch.empty((wl.n, h.dim_out), dtype=torch.float32, device=dev)
        wall, per = time_launches(torch, lambda: sp.fctp_fwd(h, x1, x2, w, out=out), args.steps, args.warmup)
        kms = sum(per) / len(per)
        flops = 2.0 * fwd_macs * wl.n
        tf = flops / (kms * 1e-3) / 1e12
        ws = torch.empty(max(1, sp.fctp_bwd_workspace(h, wl.n)), dtype=torch.uint8, device=dev)
        wallb, perb = time_launches(torch, lambda: sp.fctp_bwd(h, x1, x2, w, g, workspace=ws), args.steps,
                                    args.warmup)
        kb = sum(perb) / len(perb)
        tfb = 2.0 * bwd_macs * wl.n / (kb * 1e-3) / 1e12
        res[lay] = {"workload": wl.name, "samples": wl.n, "ms_per_call": kms, "samples_per_s": wl.n / (wall / args.steps),
                    "kernel": "fctp_kernel",
                    "roofline": {"bound": "mfma", "achieved": tf, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": tf / FP32_MFMA_PEAK_TFLOPS, "algorithmic_flops": flops},
                    "backward": {"ms_per_call": kb, "kernels": ["fctp_kernel (dx1)", "fctp_kernel (dx2)",
                                                                "fctp_dw_kernel", "fctp_dw_fold_kernel"],
                                 "roofline": {"bound": "mfma", "achieved": tfb, "peak": FP32_MFMA_PEAK_TFLOPS,
                                              "unit": "TFLOP/s", "frac": tfb / FP32_MFMA_PEAK_TFLOPS,
                                              "algorithmic_flops": 2.0 * bwd_macs * wl.n}}}
        del x1, x2, w, g, out, ws
    return res


def fc_conv(torch, sp, workloads, dev, args):
    """The fully connected product as a convolution with one weight row per
    edge on the 20k-node / 600k-edge graph (16x0e+16x1o features, l <= 2
    harmonics), both layouts.  Algorithmic bytes: every operand read or
    written once: per edge the weight row, the harmonics and the two
    indices; per node the x row and the output row."""
    import numpy as np

    from oracle import fctp as ofc   # sizes only
    wl = workloads.WORKLOADS[9]
    f = ofc.FullyConnectedTP(wl.irreps_in1, wl.irreps_sh, wl.irreps_out)
    inp = workloads.fcconv_inputs(wl, f.weight_numel)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, sh, w, src, dst = (to(inp[k]) for k in ("x", "sh", "w", "src", "dst"))
    N, E = inp["n_nodes"], inp["dst"].shape[0]
    del inp
    nbytes = E * (f.weight_numel + f.dim_in2) * 4 + 2 * E * 4 + N * (f.dim_in1 + f.dim_out) * 4
    res = {"workload": wl.name, "nodes": N, "edges": E, "algorithmic_bytes": nbytes}
    for lay in wl.layouts:
        h = sp.fctp_create(wl.irreps_in1, wl.irreps_sh, wl.irreps_out, layout=lay, dtype=wl.dtype)
        out = torch.empty((N, h.dim_out), dtype=torch.float32, device=dev)
        wall, per = time_launches(torch, lambda: sp.fctp_conv_fwd(h, x, sh, w, src, dst, N, out=out), args.steps,
                                  args.warmup)
        kms = sum(per) / len(per)
        gbps = nbytes / (kms * 1e-3) / 1e9
        res[lay] = {"ms_per_call": kms, "edges_per_s": E / (wall / args.steps), "kernel": "fcconv_kernel",
                    "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                 "frac": gbps / HBM_PEAK_GBPS}}
        # backward: per edge the weight row read and its gradient written, the
        # harmonics and their gradient and three indices; per node the
        # output-gradient row; per source x and dx (the source message written
        # and read back is reported apart, as the design's overhead)
        g = torch.from_numpy(workloads.output_gradient(N, h.dim_out, wl.dtype, seed=2009)).to(dev)
        perm = torch.argsort(src, stable=True).to(src.dtype)
        ws = torch.empty(max(1, sp.fctp_conv_bwd_workspace(h, E)), dtype=torch.uint8, device=dev)
        wallb, perb = time_launches(torch, lambda: sp.fctp_conv_bwd(h, x, sh, w, g, src, dst, perm, N, workspace=ws),
                                    args.steps, args.warmup)
        kb = sum(perb) / len(perb)
        bbytes = (E * (2 * f.weight_numel + 2 * f.dim_in2) * 4 + 3 * E * 4 +
                  N * f.dim_out * 4 + 2 * N * f.dim_in1 * 4)
        msg = 2 * E * f.dim_in1 * 4
        res[lay]["backward"] = {"ms_per_call": kb, "kernels": ["fcconv_bwd_edge_kernel", "fcconv_bwd_src_kernel"],
                                "roofline": {"bound": "hbm", "achieved": bbytes / (kb * 1e-3) / 1e9,
                                             "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                             "frac": bbytes / (kb * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                             "algorithmic_bytes": bbytes},
                                "design_overhead": {"what": "per-edge source messages (workspace round trip, "
                                                            "not counted above)", "bytes": msg,
                                                    "GBps_with_overhead": (bbytes + msg) / (kb * 1e-3) / 1e9}}
        del out, g, perm, ws
    del x, sh, w, src, dst
    return res


def fc_per_sample(torch, sp, workloads, dev, args):
    """The fully connected product with one weight row per sample (20k
    samples of 16x0e+16x1o x 8x0e+8x1o -> 16x0e+16x1o, 8,192 weights per
    sample), both layouts.  Algorithmic bytes: every operand read or written
    once; per sample forward the weight row, x1, x2 and the output row;
    backward the weight row, x1, x2 and the output gradient read, the
    weight-gradient row and both input gradients written."""
    import numpy as np

    from oracle import fctp as ofc   # sizes only
    wl = workloads.WORKLOADS[10]
    f = ofc.FullyConnectedTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.fc_inputs(wl, f.weight_numel)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x1, x2, w = (to(inp[k]) for k in ("x1", "x2", "w"))
    del inp
    g = to(workloads.output_gradient(wl.n, f.dim_out, wl.dtype, seed=2010))
    n = wl.n
    fbytes = n * (f.weight_numel + f.dim_in1 + f.dim_in2 + f.dim_out) * 4
    bbytes = n * (2 * f.weight_numel + 2 * f.dim_in1 + 2 * f.dim_in2 + f.dim_out) * 4
    res = {"workload": wl.name, "samples": n, "weights_per_sample": f.weight_numel,
           "algorithmic_bytes": {"forward": fbytes, "backward": bbytes}}
    out = torch.empty((n, f.dim_out), dtype=torch.float32, device=dev)
    g1, g2, gw = torch.empty_like(x1), torch.empty_like(x2), torch.empty_like(w)
    for lay in wl.layouts:
        h = sp.fctp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=lay, dtype=wl.dtype)
        st = sp._stream_ptr(x1.device)
        fwd = lambda: sp._check(sp.lib.fctp_fwd_per_sample(h._h, sp._ptr(x1), sp._ptr(x2), sp._ptr(w), n,
                                                           sp._ptr(out), st))
        wall, per = time_launches(torch, fwd, args.steps, args.warmup)
        kms = sum(per) / len(per)
        bwd = lambda: sp._check(sp.lib.fctp_bwd_per_sample(h._h, sp._ptr(x1), sp._ptr(x2), sp._ptr(w), sp._ptr(g),
                                                           n, sp._ptr(g1), sp._ptr(g2), sp._ptr(gw), st))
        wallb, perb = time_launches(torch, bwd, args.steps, args.warmup)
        kb = sum(perb) / len(perb)
        fg, bg = fbytes / (kms * 1e-3) / 1e9, bbytes / (kb * 1e-3) / 1e9
        res[lay] = {"ms_per_call": kms, "samples_per_s": n / (wall / args.steps), "kernel": "fctp_ps_fwd_kernel",
                    "roofline": {"bound": "hbm", "achieved": fg, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                 "frac": fg / HBM_PEAK_GBPS},
                    "backward": {"ms_per_call": kb, "kernel": "fctp_ps_bwd_kernel",
                                 "roofline": {"bound": "hbm", "achieved": bg, "peak": HBM_PEAK_GBPS,
                                              "unit": "GB/s", "frac": bg / HBM_PEAK_GBPS}}}
    del x1, x2, w, g, out, g1, g2, gw
    return res


def eager_per_path(torch, h, wl, t, N, E, dev):
    """Context for the fusion: the same convolution as plain PyTorch-ROCm
    operations, one gather, contraction and index_add_ per path (the
    launch-per-path form the fused kernel replaces), on the same GPU and
    inputs; ir_mul blocks, coefficients read from the descriptor."""
    import numpy as np

    from oracle import irreps as oir   # sizes only: block offsets

    def offsets(irreps):
        o, r = 0, []
        for mul, l, _ in oir.parse(irreps):
            r.append(o)
            o += mul * (2 * l + 1)
        return r
    assert h.layout == "ir_mul"
    off1, off2 = offsets(wl.irreps_in1), offsets(wl.irreps_in2)
    paths = []
    for p in range(h.num_paths):
        i = h.path_info(p)
        d1, d2, d3 = 2 * i["l1"] + 1, 2 * i["l2"] + 1, 2 * i["lo"] + 1
        C = torch.from_numpy(h.path_cg(p).astype(np.float32)).to(dev)
        paths.append((off1[i["in1_block"]], off2[i["in2_block"]], i["out_offset"], i["weight_offset"],
                      i["mul"], d1, d2, d3, C))
    x, sh, w, src, dst = t["x"], t["sh"], t["w"], t["src"].long(), t["dst"].long()
    out = torch.zeros((N, h.dim_out), dtype=x.dtype, device=dev)

    def run():
        out.zero_()
        for o1, o2, oo, wo, mul, d1, d2, d3, C in paths:
            xb = x[:, o1:o1 + d1 * mul].index_select(0, src).view(E, d1, mul)
            m = torch.einsum("abk,eau,eb->eku", C, xb, sh[:, o2:o2 + d2]) * w[:, wo:wo + mul].view(E, 1, mul)
            out[:, oo:oo + d3 * mul].index_add_(0, dst, m.reshape(E, d3 * mul))
    run()
    torch.cuda.synchronize()
    diff = float((out - t["out"]).abs().max()) / max(float(t["out"].abs().max()), 1e-30)
    steps = 20
    wall, per = time_launches(torch, run, steps, 3)
    return {"what": "one gather, contraction and index_add_ per path in PyTorch (fp32), same inputs",
            "paths": len(paths), "us_per_call": wall * 1e6 / steps,
            "max_rel_diff_to_fused": diff}


def other_workloads(torch, sp, workloads, dev, args):
    """The smaller workloads: microseconds per call (eager, and replayed from
    a HIP graph for the launch-bound molecular batch) and edges/s; the
    medium graph is timed cold by rotating four input sets (4 x 187 MB >
    the 256 MB Infinity Cache)."""
    import numpy as np
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = {}
    for n in (1, 2, 3):
        wl = workloads.WORKLOADS[n]
        h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=wl.layouts[0], dtype=wl.dtype)
        fan = workloads.fan_in_from_irreps_out(h.irreps_out)
        sets = []
        for r in range(4 if n == 3 else 1):
            inp = workloads.tp_inputs(wl, fan, seed=1000 + n + 100 * r)
            t = dict(x=to(inp["x"]), sh=to(inp["sh"]), w=to(inp["w"]),
                     src=to(inp["src"]) if inp["src"] is not None else None,
                     dst=to(inp["dst"]) if inp["dst"] is not None else None)
            t["out"] = torch.empty((inp["n_nodes"], h.dim_out), dtype=t["x"].dtype, device=dev)
            sets.append(t)
        N, E = inp["n_nodes"], inp["sh"].shape[0]
        k = [0]

        def fwd():
            t = sets[k[0] % len(sets)]
            k[0] += 1
            sp.tp_conv_fwd(h, t["x"], t["sh"], t["w"], t["src"], t["dst"], n_nodes=N, out=t["out"])
        steps = max(args.steps, args.small_steps)
        wall, per = time_launches(torch, fwd, steps, args.warmup)
        rec = {"workload": wl.name, "layout": wl.layouts[0], "dtype": wl.dtype, "nodes": N, "edges": E,
               "kernel": h.kernel_name, "us_per_call": wall * 1e6 / steps,
               "kernel_us_mean": 1e3 * sum(per) / len(per), "kernel_us_median": 1e3 * per[len(per) // 2],
               "edges_per_s": E * steps / wall}
        if n == 3:
            b = E * (h.weight_numel + h.dim_in2 + 2) * 4 + N * (h.dim_in1 + h.dim_out) * 4
            rec["cold_input_sets"] = len(sets)
            rec["hbm_GBps_algorithmic"] = b / (sum(per) / len(per) * 1e-3) / 1e9
            if not args.no_eager:
                rec["eager_per_path"] = eager_per_path(torch, h, wl, sets[0], N, E, dev)
        if n in (2, 3):
            # row pointers built once per graph (timed apart) replace the
            # per-destination range search of every call
            t = sets[0]
            rp = sp.tp_rowptr_build(t["dst"], N)
            _, per_b = time_launches(torch, lambda: sp.tp_rowptr_build(t["dst"], N, out=rp), steps, args.warmup)
            fr = lambda: sp.tp_conv_fwd_rowptr(h, t["x"], t["sh"], t["w"], t["src"], rp, out=t["out"])
            wall_r, per_r = time_launches(torch, fr, steps, args.warmup)
            rec["rowptr"] = {"build_kernel_us_mean": 1e3 * sum(per_b) / len(per_b),
                             "kernel_us_mean": 1e3 * sum(per_r) / len(per_r),
                             "kernel_us_median": 1e3 * per_r[len(per_r) // 2],
                             "us_per_call": wall_r * 1e6 / steps, "edges_per_s": E * steps / wall_r,
                             "what": "tp_conv_fwd_rowptr with row pointers built once (input set 0, warm)"}
            # backward on the same graph: with the in-kernel searches, and
            # with destination and source row pointers built once
            g = torch.from_numpy(workloads.output_gradient(N, h.dim_out, wl.dtype, seed=74)).to(dev, t["x"].dtype)
            perm = torch.argsort(t["src"], stable=True).to(t["src"].dtype)
            gx, gsh, gw = torch.empty_like(t["x"]), torch.empty_like(t["sh"]), torch.empty_like(t["w"])
            ws = torch.empty(sp.tp_conv_bwd_workspace(h, E), dtype=torch.uint8, device=dev)
            srp = sp.tp_src_rowptr_build(t["src"], perm, t["x"].shape[0])
            kw = dict(workspace=ws, grad_x=gx, grad_sh=gsh, grad_w=gw)
            fb = lambda: sp.tp_conv_bwd(h, t["x"], t["sh"], t["w"], g, t["src"], t["dst"], perm, n_nodes=N, **kw)
            fbr = lambda: sp.tp_conv_bwd_rowptr(h, t["x"], t["sh"], t["w"], g, t["src"], t["dst"], perm, rp, srp, **kw)
            _, per_sb = time_launches(torch, lambda: sp.tp_src_rowptr_build(t["src"], perm, t["x"].shape[0], out=srp),
                                      steps, args.warmup)
            _, per_bw = time_launches(torch, fb, steps, args.warmup)
            _, per_bwr = time_launches(torch, fbr, steps, args.warmup)
            rec["backward"] = {"us_per_call_events": 1e3 * sum(per_bw) / len(per_bw),
                               "us_per_call_events_median": 1e3 * per_bw[len(per_bw) // 2],
                               "rowptr_us_per_call_events": 1e3 * sum(per_bwr) / len(per_bwr),
                               "rowptr_us_per_call_events_median": 1e3 * per_bwr[len(per_bwr) // 2],
                               "src_rowptr_build_us": 1e3 * sum(per_sb) / len(per_sb),
                               "what": "tp_conv_bwd (all launches of one call, HIP events), and "
                                       "tp_conv_bwd_rowptr with both row pointers built once"}
            del g, perm, gx, gsh, gw, ws, srp
        if n == 2:
            # HIP graph replay of 20 calls (the path has no memset or host work)
            t = sets[0]
            ref = t["out"].clone()
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                fwd()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for _ in range(20):
                    sp.tp_conv_fwd(h, t["x"], t["sh"], t["w"], t["src"], t["dst"], n_nodes=N, out=t["out"])
            ok = True
            for _ in range(3):
                t["out"].zero_()
                g.replay()
                torch.cuda.synchronize()
                ok = ok and bool(torch.equal(t["out"], ref))
            reps = 20
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            rec["graph_us_per_call"] = (time.perf_counter() - t0) * 1e6 / (reps * 20)
            rec["graph_replays_match_eager"] = ok
        out[wl.name] = rec
        del sets
    return out


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
