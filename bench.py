"""Throughput of the GIFT encode + decode-reduce unit on one MI355X.

Unit of work (one "step"): gift_encode of one replica's 1536 x 6144 fp32
gradient (rank-32 input-side whitening, E4M3, per-tensor scale) and
gift_decode_reduce of R = 8 replica payloads into one fp32 gradient, on one
stream.  The other 7 payloads are encoded during setup.  Statistics
(T = 16384 bf16 tokens) and the rank-32 refresh run in setup and are timed
separately, as is the encode alone, without and with error feedback
(stage_rooflines).

Timed region: W untimed warmup steps, then K steps bracketed by
torch.cuda.synchronize(); the input buffers rotate over 4 independent sets
(W, 8 payloads, output: 604 MB in all, more than twice the 256 MB Infinity
Cache) so each step reads inputs that are not cache-resident.  The kernel
durations behind `roofline` come from K encode calls and then K
decode-reduce calls back to back over the same buffer sets, each batch
between one pair of HIP events (event pairs around single calls would
lengthen them, and they stay out of the pass `value` is measured on).

Prints one JSON line (the metric, roofline of the dominant kernel, the oracle
timed on the host cores as a baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2500.0
FP64_PEAK_TFS = 78.6
FP32_PEAK_TFS = 157.3
# The refresh's six A X products: the last one of the subspace iteration and
# the Rayleigh-Ritz product on the fp64 matrix cores, the other four on the
# fp32 ones.  Its peak is the rate at which the six would run, each at its
# own unit's peak.
REFRESH_PEAK_TFS = 6.0 / (2.0 / FP64_PEAK_TFS + 4.0 / FP32_PEAK_TFS)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--scaling", default="tensor", choices=["tensor", "block"])
    p.add_argument("--sets", type=int, default=4)
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    p.add_argument("--layers", type=int, default=24,
                   help="selective: decoder layers of the 600M-class model (24: the stated shapes, 906M "
                        "parameters; 16: 604M, the stated total)")
    p.add_argument("--config", default="unit",
                   choices=["unit", "selective", "stress", "slab", "ablation", "fidelity"],
                   help="unit: the headline encode + decode unit (default); selective: the whole "
                        "600M-class gradient buffer (168 tensors, 13 rank-32); stress: one step of "
                        "the 4096 x 16384 stress layer (statistics, refresh, encode, decode R = 16); "
                        "slab: one GPU's share of the row-slab exchange at R = 8 (the kernels between "
                        "the collectives, which are not run); ablation: the 1536 x 6144 layer with every "
                        "transform (two-sided K-FAC, input-side Cholesky, rank-32, diagonal, Euclidean): "
                        "statistics, refresh, encode + decode-reduce times and fidelity; fidelity: the decoded "
                        "mean of every configuration against the fp32 mean gradient")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only (the multi-GPU reduce-scatter / all-gather exchange is not "
              "implemented); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import fac_whitening_amd as fw
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config == "selective":
        return bench_selective(args, torch, fw, synth, dev)
    if args.config == "stress":
        return bench_stress(args, torch, fw, synth, dev)
    if args.config == "slab":
        return bench_slab(args, torch, fw, synth, dev)
    if args.config == "ablation":
        return bench_ablation(args, torch, fw, synth, dev)
    if args.config == "fidelity":
        return bench_fidelity(args, torch, fw, synth, dev)
    m, d, T, R, k = 1536, 6144, 16384, 8, 32
    scaling = fw.SCALINGS[args.scaling]
    nb = fw.nblocks(m, d, scaling)

    # ---- setup: synthetic layer (Llama-600M fc2 shape), statistics, refresh
    t0 = time.time()
    case = synth.make_layer(4, device=dev, R=R)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    L = fw.Layer(m, d, "lowrank", rank=k, oversample=16, power_iters=4, ema_decay=0.0, device=dev)
    L.accumulate_stats(case.a_steps[0], fw.SIDE_A, commit=True)
    L.refresh(case.omega)
    torch.cuda.synchronize()
    assert L.flags() == 0, "non-finite factor"

    # ---- the statistics and refresh steps, timed warm (outside the unit)
    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    scratch = fw.Layer(16, d, "diag", device=dev)    # its window absorbs the repeated batches
    t_stats_ms = timed(lambda: scratch.accumulate_stats(case.a_steps[0], fw.SIDE_A))
    del scratch
    t_refresh_ms = timed(lambda: L.refresh(case.omega))
    assert L.flags() == 0, "non-finite factor"
    stats_flop = float(T) * d * (d + 1)                     # the symmetric triangle
    refresh_flop = 12.0 * d * d * min(k + 16, d)            # six A X products of width l = 48
    refresh_bytes = 6.0 * d * d * 4                          # A read by each product
    stage_rooflines = {
        "stats": {"ms": round(t_stats_ms, 4), "bound": "mfma", "achieved": round(stats_flop / t_stats_ms / 1e9, 1),
                  "peak": BF16_PEAK_TFS, "unit": "TFLOP/s",
                  "frac": round(stats_flop / t_stats_ms / 1e9 / BF16_PEAK_TFS, 4),
                  "work": "A += a^T a, 16384 bf16 tokens x 6144 (triangle flops)"},
        "refresh": {"ms": round(t_refresh_ms, 4), "bound": "mfma",
                    "achieved": round(refresh_flop / t_refresh_ms / 1e9, 2), "peak": round(REFRESH_PEAK_TFS, 1),
                    "unit": "TFLOP/s", "frac": round(refresh_flop / t_refresh_ms / 1e9 / REFRESH_PEAK_TFS, 4),
                    "peak_note": "2 products at the fp64 matrix peak, 4 at the fp32 matrix peak",
                    "hbm_frac": round(refresh_bytes / (t_refresh_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "work": "rank-32 subspace iteration (q = 4, l = 48) on the 6144 x 6144 A"},
    }

    # ---- payloads: replica 0 is encoded inside each step; 1..R-1 in setup
    sets = []
    pay_codes = torch.empty(R, m, d, dtype=torch.uint8, device=dev)
    pay_scales = torch.empty(R, nb, dtype=torch.float32, device=dev)
    for r in range(1, R):
        L.encode(case.W[r], fw.E4M3, scaling, codes=pay_codes[r], scales=pay_scales[r])
    for s in range(args.sets):
        W = case.W[0].clone()
        codes = pay_codes.clone()
        scales = pay_scales.clone()
        out = torch.empty(m, d, dtype=torch.float32, device=dev)
        sets.append((W, codes, scales, out))
    # a plain copy of known size (268 MB read + 268 MB written): the
    # reference dispatch for scaling the HBM byte counters of a profiler pass
    calib_src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.neg(calib_src, out=calib_dst)
    del calib_src, calib_dst
    torch.cuda.synchronize()

    def step(i):
        W, codes, scales, out = sets[i % len(sets)]
        L.encode(W, fw.E4M3, scaling, codes=codes[0], scales=scales[0])
        L.decode_reduce(codes, scales, fw.E4M3, scaling, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: K steps back to back, with events only at the 5 batch
    # boundaries (median, p10, p90); `value` comes from it.
    nbat = min(5, args.steps)
    bounds = [args.steps * j // nbat for j in range(nbat + 1)]
    bat_ev = {b: torch.cuda.Event(enable_timing=True) for b in bounds}
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    bat_ev[0].record()
    for i in range(args.steps):
        step(i)
        if i + 1 in bat_ev:
            bat_ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = bat_ev[0].elapsed_time(bat_ev[args.steps])
    bat_ms = [bat_ev[bounds[j]].elapsed_time(bat_ev[bounds[j + 1]]) / (bounds[j + 1] - bounds[j])
              for j in range(nbat)]
    ms_per_step = total_ms / args.steps
    # Kernel durations: K encode calls back to back, then K decode-reduce
    # calls back to back, over the same rotating buffer sets, each batch
    # bracketed by one pair of HIP events on the stream the kernels run on
    # (torch's current stream): the average launch-to-launch duration of
    # each kernel, without the few microseconds an event pair adds to a call.
    def batch_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def enc_only(i):
        W, codes, scales, _ = sets[i % len(sets)]
        L.encode(W, fw.E4M3, scaling, codes=codes[0], scales=scales[0])

    def dec_only(i):
        _, codes, scales, out = sets[i % len(sets)]
        L.decode_reduce(codes, scales, fw.E4M3, scaling, out=out)

    t_enc = batch_ms(enc_only)
    t_dec = batch_ms(dec_only)
    grad_bytes = 4.0 * m * d
    value = grad_bytes / (ms_per_step * 1e-3) / 1e9         # GB/s of fp32 gradient

    # algorithmic bytes per unit: encode reads W and U, writes codes + scales;
    # decode reads R payloads and U, writes the fp32 gradient
    u_bytes = d * k * 4 + 68 * 4
    enc_bytes = 4.0 * m * d + u_bytes + m * d + 4 * nb
    dec_bytes = R * (m * d + 4 * nb) + u_bytes + 4.0 * m * d
    dominant = "decode"
    dom_bytes = dec_bytes
    dom_ms = t_dec
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    kernel = f"k_rank_{dominant}<0, {R}, 0>"   # FP8 format, replica count, per-tensor scale
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(kernel, args.scaling),
                "kernel": kernel,
                "unit_frac": round((enc_bytes + dec_bytes) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "decode_ms": round(t_dec, 5), "encode_ms": round(t_enc, 5),
                "durations": "K calls of each kernel back to back over the rotating sets, one event pair per batch",
                "alg_bytes_encode": int(enc_bytes), "alg_bytes_decode": int(dec_bytes)}

    # ---- beside the headline: batch spread, the unit with one buffer set
    # (warm), the per-128x128-block unit, a plain streaming copy (the
    # achievable HBM ceiling on this machine) and the fp32-equivalent flops
    def unit_on(sc, c, s_, W, out):
        L.encode(W, fw.E4M3, sc, codes=c[0], scales=s_[0])
        L.decode_reduce(c, s_, fw.E4M3, sc, out=out)

    W0, c0, s0, o0 = sets[0]
    t_warm = _event_ms(torch, lambda: unit_on(scaling, c0, s0, W0, o0), args.steps)
    other = fw.SCALE_BLOCK128 if scaling == fw.SCALE_TENSOR else fw.SCALE_TENSOR
    nb_o = fw.nblocks(m, d, other)
    bsets = []
    for j in range(len(sets)):
        c = torch.empty(R, m, d, dtype=torch.uint8, device=dev)
        s_ = torch.empty(R, nb_o, dtype=torch.float32, device=dev)
        if j == 0:
            for r in range(1, R):
                L.encode(case.W[r], fw.E4M3, other, codes=c[r], scales=s_[r])
        else:
            c.copy_(bsets[0][0])
            s_.copy_(bsets[0][1])
        bsets.append((c, s_))
    bturn = [0]

    def unit_other():
        j = bturn[0] % len(sets)
        bturn[0] += 1
        unit_on(other, bsets[j][0], bsets[j][1], sets[j][0], sets[j][3])

    t_other = _event_ms(torch, unit_other, args.steps)
    del bsets

    # the same unit with the FP4 payload (E2M1 codes, an E4M3 scale per 16
    # elements of a row, one fp32 tensor scale), over its own rotating sets
    c4s, b4s, t4s = (torch.empty(R, m, d // 2, dtype=torch.uint8, device=dev),
                     torch.empty(R, m, d // 16, dtype=torch.uint8, device=dev),
                     torch.empty(R, dtype=torch.float32, device=dev))
    for r in range(1, R):
        L.encode_fp4(case.W[r], codes=c4s[r], bscales=b4s[r], tscale=t4s[r:r + 1])
    fsets = [(c4s.clone(), b4s.clone(), t4s.clone()) for _ in sets]
    del c4s, b4s, t4s
    fturn = [0]

    def fp4_part(i, e, dcd):
        W, _, _, out = sets[i % len(sets)]
        c4, b4, t4 = fsets[i % len(sets)]
        if e:
            L.encode_fp4(W, codes=c4[0], bscales=b4[0], tscale=t4[0:1])
        if dcd:
            L.decode_reduce_fp4(c4, b4, t4, out=out)

    def fp4_unit():
        fp4_part(fturn[0], True, True)
        fturn[0] += 1

    t_fp4 = _event_ms(torch, fp4_unit, args.steps)
    t_fp4_enc = batch_ms(lambda i: fp4_part(i, True, False))
    t_fp4_dec = batch_ms(lambda i: fp4_part(i, False, True))
    torch.cuda.synchronize()
    assert L.flags() == 0
    del fsets
    pay4 = m * d // 2 + m * d // 16 + 4
    enc4_bytes = 4.0 * m * d + u_bytes + pay4
    dec4_bytes = R * pay4 + u_bytes + 4.0 * m * d
    csrc = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    t_copy = _event_ms(torch, lambda: torch.neg(csrc, out=cdst), 10)
    del csrc, cdst
    copy_gbs = 2.0 * 4 * (64 << 20) / (t_copy * 1e-3) / 1e9
    unit_detail = {
        "batches_ms_per_step": {"median": round(float(np.median(bat_ms)), 5),
                                "p10": round(float(np.percentile(bat_ms, 10)), 5),
                                "p90": round(float(np.percentile(bat_ms, 90)), 5), "batches": nbat},
        "warm_one_set": {"ms_per_step": round(t_warm, 5),
                         "GB_s_of_grad": round(grad_bytes / (t_warm * 1e-3) / 1e9, 1)},
        ("block128" if other == fw.SCALE_BLOCK128 else "tensor"): {
            "ms_per_step": round(t_other, 5), "GB_s_of_grad": round(grad_bytes / (t_other * 1e-3) / 1e9, 1),
            "cache": f"cold ({args.sets} rotating buffer sets)"},
        "fp4": {"ms_per_step": round(t_fp4, 5), "GB_s_of_grad": round(grad_bytes / (t_fp4 * 1e-3) / 1e9, 1),
                "unit_frac": round((enc4_bytes + dec4_bytes) / (t_fp4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "encode_ms": round(t_fp4_enc, 5), "decode_ms": round(t_fp4_dec, 5),
                "decode_frac": round(dec4_bytes / (t_fp4_dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "alg_bytes_encode": int(enc4_bytes), "alg_bytes_decode": int(dec4_bytes),
                "work": "E2M1 codes with E4M3 scales per 16 elements of a row; encode of replica 0, "
                        "decode-reduce of the 8 payloads", "cache": f"cold ({args.sets} rotating buffer sets)"},
        "copy_ceiling": {"kernel": "torch.neg, 64 Mi fp32 (256 MiB read + 256 MiB written)",
                         "GB_s": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
                         "unit_frac_of_copy": round((enc_bytes + dec_bytes) / (ms_per_step * 1e-3) / 1e9 / copy_gbs,
                                                    4)},
        "fp32_equivalent": {"flop_per_elem": 256, "TFLOP_s": round(256.0 * m * d / (ms_per_step * 1e-3) / 1e12, 2),
                            "frac_of_fp32_peak": round(256.0 * m * d / (ms_per_step * 1e-3) / 1e12 / FP32_PEAK_TFS,
                                                       4)},
    }

    # the encode alone, without and with error feedback (Algorithm 1: the
    # residual is read and rewritten beside the codes), outside the unit
    resids = [torch.zeros(m, d, dtype=torch.float32, device=dev) for _ in sets]
    turn = [0]

    def enc(ef):
        j = turn[0] % len(sets)
        turn[0] += 1
        W, codes, scales, _ = sets[j]
        L.encode(W, fw.E4M3, scaling, codes=codes[0], scales=scales[0], resid=resids[j] if ef else None)

    for name, ef in (("encode", False), ("encode_ef", True)):
        t = _event_ms(torch, lambda: enc(ef), 40)
        b = enc_bytes + (8.0 * m * d if ef else 0.0)
        stage_rooflines[name] = {
            "ms": round(t, 5), "bound": "hbm", "achieved": round(b / (t * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": int(b),
            "work": "rank-32 whitening, amax, E4M3 codes of one replica"
                    + (" + fp32 residual read and rewritten" if ef else "")}
    torch.cuda.synchronize()
    assert L.flags() == 0

    # fidelity of the headline layer's decoded mean against the fp32 mean of
    # the 8 replicas: GIFT rank-32 (local scales) and the Euclidean baseline
    # (shared amax), per tensor and per 128 x 128 block
    LE = fw.Layer(m, d, "euclid", device=dev)
    fid = fidelity_rows(torch, fw, case.W, L.buffers()["A"], {"gift_rank32": L, "euclid": LE})
    del LE
    result = {
        "metric": "GIFT encode+decode GB/s of fp32 grad (1536\u00d76144, r=32); % of HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded Llama-600M fc2 layer: a ~ N(0, Q diag(i^-1.5) Q^T) bf16, W = delta^T a / T)",
        "config": {"workload": "fc2 1536x6144 fp32 gradient, rank-32 lowrank whitening, E4M3 "
                               f"{args.scaling} scale, R=8 replicas", "d_out": m, "d_in": d, "rank": k,
                   "replicas": R, "tokens": T, "format": "e4m3", "scaling": args.scaling,
                   "cache": f"cold ({args.sets} rotating buffer sets)"},
        "roofline": roofline,
        "stage_rooflines": stage_rooflines,
        "unit_detail": unit_detail,
        "fidelity": fid,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(case, L.buffers()["A"], R, m, d, args.scaling)
    print(json.dumps(result), flush=True)


def _event_ms(torch, fn, reps):
    """Mean event-timed milliseconds of fn() over reps calls (one untimed call first)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_selective(args, torch, fw, synth, dev):
    """Whole-buffer encode + decode-reduce of the 600M-class deployment (the
    figures below are for the default 24 layers; --layers 16 gives the
    604M-parameter buffer): 168 weight gradients (906M fp32 values, 3.62 GB), the fc2 gradients of 13
    layers rank-32 whitened, the other 155 Euclidean; E4M3 per tensor,
    R = 8 (replicas 1..7 encoded in setup).  One step = worker 0's share:
    the 155 Euclidean tensors as one flat bucket (local amax and quantise
    with the shared amax of the 8 replicas, then the decode-reduce: three
    launches) and, for each rank-32 layer, its encode and decode-reduce (one
    launch each).  The Euclidean tensors are also timed with one launch per
    tensor and per phase (the same buffers), and with 512-element block
    scales (the per-block Euclidean baseline).  The rank-32 layers'
    statistics (T = 8192 bf16 tokens) and refresh run in setup.  Gradients:
    the direct Gaussian draw (synth.direct_gradient)."""
    R, Ttok = 8, 8192
    f, s = fw.E4M3, fw.SCALE_TENSOR
    t0 = time.time()
    state_gift = 0
    gift_items, eu = [], []
    shared_work = None   # one workspace for every rank-32 layer (their windows commit in one call each)
    for k, (l, name, mo, di, alpha, gift) in enumerate(synth.selective_tensors(args.layers)):
        seed = lambda r, l=l, name=name: synth.seed_for(3, synth.ROLE_A, l * 8 + list(synth.SELECTIVE_SHAPES).index(name),
                                                        r)
        if not gift:
            eu.append((mo, di, alpha, seed))
            continue
        L = fw.Layer(mo, di, "lowrank", device=dev, transient_stats=True, workspace=shared_work)
        shared_work = L.work
        a = synth.gaussian_rows(Ttok, di, alpha, None, synth.seed_for(3, synth.ROLE_A, l, 0, 1), dev, torch.bfloat16)
        L.accumulate_stats(a, fw.SIDE_A, commit=True)
        del a
        L.refresh(synth.omega(di, 48, synth.seed_for(3, synth.ROLE_OMEGA, l), dev))
        state_gift += L.state.numel()
        codes = torch.empty(R, mo, di, dtype=torch.uint8, device=dev)
        scales = torch.empty(R, 1, dtype=torch.float32, device=dev)
        for r in range(1, R):
            Wr = synth.direct_gradient(mo, di, alpha, Ttok, seed(r), dev)
            L.encode(Wr, f, s, codes=codes[r], scales=scales[r])
            del Wr
        W0 = synth.direct_gradient(mo, di, alpha, Ttok, seed(0), dev)
        gift_items.append((L, W0, codes, scales, torch.empty(mo, di, dtype=torch.float32, device=dev)))
    # the Euclidean tensors: one flat bucket per replica
    sizes = [mo * di for (mo, di, _, _) in eu]
    B = fw.Bucket(sizes, fw.SCALE_TENSOR, device=dev)
    B512 = fw.Bucket(sizes, fw.SCALE_BLOCK512, device=dev)
    n_eu = B.numel
    stride = -(-n_eu // 16) * 16
    codes_eu = torch.empty(R, stride, dtype=torch.uint8, device=dev)[:, :n_eu]
    codes_512 = torch.empty(R, stride, dtype=torch.uint8, device=dev)[:, :n_eu]
    scales_eu = torch.empty(R, B.nscales, dtype=torch.float32, device=dev)
    scales_512 = torch.empty(R, B512.nscales, dtype=torch.float32, device=dev)

    def replica(r):
        g = torch.empty(n_eu, dtype=torch.float32, device=dev)
        off = 0
        for (mo, di, alpha, seed) in eu:
            g[off:off + mo * di] = synth.direct_gradient(mo, di, alpha, Ttok, seed(r), dev).reshape(-1)
            off += mo * di
        return g
    # AllReduceMax of the local amaxes over the replicas, then replicas 1..7
    amax, amax512 = None, None
    for r in range(R):
        g = replica(r)
        a, a5 = B.amax(g), B512.amax(g)
        amax = a if amax is None else torch.maximum(amax, a)
        amax512 = a5 if amax512 is None else torch.maximum(amax512, a5)
        del g
    for r in range(1, R):
        g = replica(r)
        B.encode(g, f, amax_in=amax, codes=codes_eu[r], scales=scales_eu[r])
        B512.encode(g, f, amax_in=amax512, codes=codes_512[r], scales=scales_512[r])
        del g
    g0 = replica(0)
    am0 = torch.empty(B.nscales, dtype=torch.float32, device=dev)
    am0_512 = torch.empty(B512.nscales, dtype=torch.float32, device=dev)
    out_eu = torch.empty(n_eu, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    assert all(L.flags() == 0 for L, *_ in gift_items) and B.flags() == 0
    print(f"[bench selective] {len(eu)} Euclidean + {len(gift_items)} rank-32 tensors ready in "
          f"{time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def gift_layers():
        for L, W0, codes, scales, out in gift_items:
            L.encode(W0, f, s, codes=codes[0], scales=scales[0])
            L.decode_reduce(codes, scales, f, s, out=out)

    # the same rank-32 layers as one group: one launch encodes all of them,
    # one launch decode-reduces them
    group = fw.Group([dict(layer=L, W=W0, codes=codes[0], scales=scales[0], rcodes=codes, rscales=scales, out=out)
                      for L, W0, codes, scales, out in gift_items], R, f, s, device=dev)

    def gift_group():
        group.encode()
        group.decode_reduce()

    def euclid_bucket():
        B.encode(g0, f, amax_in=amax, amax_out=am0, codes=codes_eu[0], scales=scales_eu[0])
        B.decode_reduce(codes_eu, scales_eu, f, out=out_eu)

    def euclid_bucket_512():
        B512.encode(g0, f, amax_in=amax512, amax_out=am0_512, codes=codes_512[0], scales=scales_512[0])
        B512.decode_reduce(codes_512, scales_512, f, out=out_eu)

    # the same Euclidean work with one launch per tensor and per phase
    views, off = [], 0
    for k, (mo, di, _, _) in enumerate(eu):
        L = fw.Layer(mo, di, "euclid", device=dev)
        views.append((L, g0[off:off + mo * di].view(mo, di),
                      codes_eu[:, off:off + mo * di].unflatten(1, (mo, di)), scales_eu[:, k:k + 1],
                      amax[k:k + 1], am0[k:k + 1], out_eu[off:off + mo * di].view(mo, di)))
        off += mo * di

    def euclid_per_tensor():
        for L, W, c, sc, a_in, a_out, o in views:
            L.encode(W, f, s, amax_in=a_in, amax_out=a_out, codes=c[0], scales=sc[0])
            L.decode_reduce(c, sc, f, s, out=o)

    # (the grouped launch measured slower than one launch per layer and
    # phase: the step keeps the per-layer launches; both are reported)
    def step():
        euclid_bucket()
        gift_layers()

    steps = max(1, min(args.steps, 20))
    ms = _event_ms(torch, step, steps)
    ms_gift = _event_ms(torch, gift_layers, steps)
    ms_group = _event_ms(torch, gift_group, steps)
    ms_bucket = _event_ms(torch, euclid_bucket, steps)
    ms_per_tensor = _event_ms(torch, euclid_per_tensor, steps)
    ms_512 = _event_ms(torch, euclid_bucket_512, steps)
    torch.cuda.synchronize()
    assert all(L.flags() == 0 for L, *_ in gift_items) and B.flags() == 0 and B512.flags() == 0
    n_gift = sum(W0.numel() for _, W0, *_ in gift_items)
    n = n_eu + n_gift
    # algorithmic bytes: encode reads 4 B and writes 1 B per element, decode
    # reads R payloads and writes 4 B (scales and U_k included)
    alg_eu = (4.0 + 1 + 4) * n_eu + R * n_eu + 4 * (R + 1) * B.nscales
    alg_512 = (4.0 + 1 + 4) * n_eu + R * n_eu + 4 * (R + 1) * B512.nscales
    alg_gift = sum((4.0 + 1 + 4) * W0.numel() + R * W0.numel() + 4 * (R + 1) + 2 * W0.shape[1] * 32 * 4
                   for _, W0, *_ in gift_items)
    alg = alg_eu + alg_gift
    grad_bytes = 4.0 * n

    def stage(t, b, work):
        return {"ms": round(t, 4), "bound": "hbm", "achieved": round(b / (t * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": int(b),
                "work": work}
    result = {
        "metric": "whole-buffer encode+decode GB/s of fp32 grad (600M-class selective deployment)",
        "value": round(grad_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "f32",
        "data": "synthetic (direct Gaussian gradients, bf16 power-law activations for the rank-32 layers)",
        "config": {"workload": f"600M-class selective: {args.layers} layers x {{q,k,v,o 1536x1536, fc1/fc3 "
                               f"6144x1536, fc2 1536x6144}}; fc2 of {len(gift_items)} layers rank-32, the rest "
                               "Euclidean; E4M3 per tensor; R=8", "layers": args.layers, "tensors": len(eu) + len(gift_items),
                   "rank32_tensors": len(gift_items),
                   "params": n},
        "roofline": {"bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "alg_bytes": int(alg)},
        "stages": {
            "euclid_bucket": stage(ms_bucket, alg_eu, f"{len(eu)} Euclidean tensors, one bucket: 3 launches"),
            "euclid_per_tensor": stage(ms_per_tensor, alg_eu, "the same with one launch per tensor and phase"),
            "euclid_bucket_block512": stage(ms_512, alg_512, "per-block Euclidean baseline, 512-element blocks"),
            "rank32_group": stage(ms_group, alg_gift, f"{len(gift_items)} rank-32 fc2 layers as one group: one "
                                  "launch for the encodes, one for the decode-reduces"),
            "rank32_per_layer": stage(ms_gift, alg_gift, f"the same layers, fused encode + decode one layer "
                                      "at a time (2 launches per layer)"),
        },
        "memory": memory_report(gift_items, grad_bytes, state_gift, shared_work.numel()),
    }
    print(json.dumps(result), flush=True)


def memory_report(gift_items, grad_bytes, state_gift, work_bytes):
    """Memory of the geometry-aware layers beside the gradient buffer: as the
    pages count it ("GIFT 阅读笔记", 实验结果 / 内存开销: the rank-32 factor and
    the error-feedback buffer of the selected layers), and this library's
    whole layer state (the committed d x d statistics the subspace iteration
    reads, the packed factor, the exchange words; the layers keep no window
    sum: each window is accumulated in the one workspace they share)."""
    factor = sum(W0.shape[1] * 32 * 4 + 68 * 4 for _, W0, *_ in gift_items)   # U_k and the coefficients
    ef = sum(4 * W0.numel() for _, W0, *_ in gift_items)                      # fp32 residual per layer
    return {"grad_bytes": int(grad_bytes),
            "pages_terms": {"factor_bytes": int(factor), "error_feedback_bytes": int(ef),
                            "over_grad": round((factor + ef) / grad_bytes, 4)},
            "library_state_bytes": int(state_gift), "library_state_over_grad": round(state_gift / grad_bytes, 4),
            "shared_workspace_bytes": int(work_bytes)}


def bench_stress(args, torch, fw, synth, dev):
    """One step of the stress layer (W 4096 x 16384, heavy-tailed): statistics
    of T = 8192 bf16 tokens and commit, rank-32 refresh (every step), encode
    of replica 0 and decode-reduce of R = 16 payloads, E5M2 per 128 x 128
    block (replicas 1..15 encoded in setup).  Each stage event-timed; the
    encode + decode also with the FP4 payload (E2M1 with 16-element E4M3
    block scales) as a stage of its own."""
    m, d, Ttok, R = 4096, 16384, 8192, 16
    f, s = fw.E5M2, fw.SCALE_BLOCK128
    nb = fw.nblocks(m, d, s)
    a = synth.stress_activations(Ttok, d, 0, dev)
    om = synth.omega(d, 48, synth.seed_for(5, synth.ROLE_OMEGA), dev)
    L = fw.Layer(m, d, "lowrank", device=dev)
    L.accumulate_stats(a, fw.SIDE_A, commit=True)
    L.refresh(om)
    codes = torch.empty(R, m, d, dtype=torch.uint8, device=dev)
    scales = torch.empty(R, nb, dtype=torch.float32, device=dev)
    for r in range(1, R):
        Wr = synth.stress_gradient(m, d, 0, r, dev)
        L.encode(Wr, f, s, codes=codes[r], scales=scales[r])
        del Wr
    W0 = synth.stress_gradient(m, d, 0, 0, dev)
    out = torch.empty(m, d, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    assert L.flags() == 0
    reps = 5
    t_stats = _event_ms(torch, lambda: L.accumulate_stats(a, fw.SIDE_A, commit=True), reps)
    t_refresh = _event_ms(torch, lambda: L.refresh(om), reps)

    def unit():
        L.encode(W0, f, s, codes=codes[0], scales=scales[0])
        L.decode_reduce(codes, scales, f, s, out=out)
    t_unit = _event_ms(torch, unit, reps)
    assert L.flags() == 0
    n = m * d
    alg = (4.0 + 1) * n + R * n + 4.0 * n + 4 * nb * (R + 1) + d * 32 * 4 * 2
    # the FP4 payload (E2M1, 16-element row blocks with E4M3 scales): the
    # same unit with R = 16 FP4 payloads
    del codes
    c4 = torch.empty(R, m, d // 2, dtype=torch.uint8, device=dev)
    b4 = torch.empty(R, m, d // 16, dtype=torch.uint8, device=dev)
    t4 = torch.empty(R, dtype=torch.float32, device=dev)
    for r in range(1, R):
        Wr = synth.stress_gradient(m, d, 0, r, dev)
        L.encode_fp4(Wr, codes=c4[r], bscales=b4[r], tscale=t4[r:r + 1])
        del Wr

    def unit_fp4():
        L.encode_fp4(W0, codes=c4[0], bscales=b4[0], tscale=t4[0:1])
        L.decode_reduce_fp4(c4, b4, t4, out=out)
    t_fp4 = _event_ms(torch, unit_fp4, reps)
    assert L.flags() == 0
    pay4 = n / 2 + n / 16
    alg4 = 4.0 * n + pay4 + R * pay4 + 4.0 * n + 4 * (R + 1) + d * 32 * 4 * 2
    stats_flop = float(Ttok) * d * (d + 1)
    refresh_flop = 12.0 * d * d * 48
    result = {
        "metric": "stress layer step: encode+decode GB/s of fp32 grad (4096x16384, R=16, E5M2 per block)",
        "value": round(4.0 * n / (t_unit * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": reps,
        "ms_per_step": round(t_stats + t_refresh + t_unit, 4), "higher_is_better": True, "dtype": "f32",
        "data": "synthetic (Student-t(3) x i^-1.5 column scales, 0.1% outlier columns x100)",
        "config": {"workload": "stress 4096x16384, rank-32 refreshed every step (q=4, p=16), E5M2 per "
                               "128x128 block, R=16", "tokens": Ttok},
        "stages_ms": {"stats_commit": round(t_stats, 4), "refresh": round(t_refresh, 4),
                      "encode_decode": round(t_unit, 4), "encode_decode_fp4": round(t_fp4, 4)},
        "roofline": {"bound": "hbm", "achieved": round(alg / (t_unit * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(alg / (t_unit * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "alg_bytes": int(alg)},
        "stage_rooflines": {
            "stats": {"achieved": round(stats_flop / t_stats / 1e9, 1), "peak": BF16_PEAK_TFS, "unit": "TFLOP/s",
                      "frac": round(stats_flop / t_stats / 1e9 / BF16_PEAK_TFS, 4)},
            "refresh": {"achieved": round(refresh_flop / t_refresh / 1e9, 2), "peak": round(REFRESH_PEAK_TFS, 1),
                        "unit": "TFLOP/s", "frac": round(refresh_flop / t_refresh / 1e9 / REFRESH_PEAK_TFS, 4)},
            "encode_decode_fp4": {"achieved": round(alg4 / (t_fp4 * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(alg4 / (t_fp4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "alg_bytes": int(alg4),
                                  "work": "encode of replica 0 and decode-reduce of 16 FP4 payloads"}},
    }
    print(json.dumps(result), flush=True)


def bench_slab(args, torch, fw, synth, dev):
    """One GPU's share of the row-slab exchange for the 1536 x 6144 rank-32
    layer at R = 8 GPUs (the multi-GPU design: every GPU encodes its whole
    gradient in whitened coordinates; an all-to-all gives GPU g the 192-row
    slab g of all 8 payloads; it dequantises and sums them and requantises
    the mean in whitened coordinates with one scale shared by all slabs (an
    AllReduceMax of the slab amax); an all-gather brings every GPU all 8
    requantised slabs, one tensor with one scale; each unwhitens it, R = 1).
    Timed: GPU 0's kernels before, between and after the collectives (the
    encode of its gradient, slab dequant-sum, slab amax, requantise,
    unwhitening of the gathered tensor, one launch each); the collectives
    are not run (one GPU): the shared amax and the other slabs come from
    setup."""
    m, d, T, R, k = 1536, 6144, 16384, 8, 32
    rows = m // R
    case = synth.make_layer(4, device=dev, R=R)
    L = fw.Layer(m, d, "lowrank", rank=k, oversample=16, power_iters=4, ema_decay=0.0, device=dev)
    L.accumulate_stats(case.a_steps[0], fw.SIDE_A, commit=True)
    L.refresh(case.omega)
    codes = torch.empty(R, m, d, dtype=torch.uint8, device=dev)
    scales = torch.empty(R, 1, dtype=torch.float32, device=dev)
    for r in range(R):
        L.encode(case.W[r], fw.E4M3, fw.SCALE_TENSOR, codes=codes[r], scales=scales[r])
    Le = fw.Layer(rows, d, "euclid", device=dev)          # slab reduce, amax and requantise
    mean = torch.empty(rows, d, dtype=torch.float32, device=dev)
    gathered = torch.empty(1, m, d, dtype=torch.uint8, device=dev)   # the all-gather's result
    gscale = torch.empty(1, 1, dtype=torch.float32, device=dev)
    am_local = torch.empty(1, dtype=torch.float32, device=dev)
    out = torch.empty(m, d, dtype=torch.float32, device=dev)
    # setup: every slab's mean and amax (the AllReduceMax's inputs), then the
    # other GPUs' requantised slabs with the shared scale
    ams = []
    for g in range(R):
        Le.decode_reduce(codes[:, g * rows:(g + 1) * rows, :], scales, fw.E4M3, fw.SCALE_TENSOR, out=mean)
        a = torch.empty(1, dtype=torch.float32, device=dev)
        Le.encode(mean, fw.E4M3, fw.SCALE_TENSOR, amax_out=a, want_codes=False)
        ams.append(a)
    shared = torch.stack(ams).max(dim=0).values
    for g in range(1, R):
        Le.decode_reduce(codes[:, g * rows:(g + 1) * rows, :], scales, fw.E4M3, fw.SCALE_TENSOR, out=mean)
        Le.encode(mean, fw.E4M3, fw.SCALE_TENSOR, amax_in=shared, codes=gathered[0, g * rows:(g + 1) * rows],
                  scales=gscale[0])
    slab0 = codes[:, :rows, :]

    def encode_own():   # this GPU's whole gradient, before the all-to-all
        L.encode(case.W[0], fw.E4M3, fw.SCALE_TENSOR, codes=codes[0], scales=scales[0])

    def reduce():
        Le.decode_reduce(slab0, scales, fw.E4M3, fw.SCALE_TENSOR, out=mean)

    def requant():
        Le.encode(mean, fw.E4M3, fw.SCALE_TENSOR, amax_out=am_local, want_codes=False)   # into the AllReduceMax
        Le.encode(mean, fw.E4M3, fw.SCALE_TENSOR, amax_in=shared, codes=gathered[0, :rows], scales=gscale[0])

    def unwhiten():
        L.decode_reduce(gathered, gscale, fw.E4M3, fw.SCALE_TENSOR, out=out)

    def step():
        encode_own()
        reduce()
        requant()
        unwhiten()

    steps = max(1, args.steps)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    ms = _event_ms(torch, step, steps)
    t_encode = _event_ms(torch, encode_own, steps)
    t_reduce = _event_ms(torch, reduce, steps)
    t_requant = _event_ms(torch, requant, steps)
    t_unwhiten = _event_ms(torch, unwhiten, steps)
    torch.cuda.synchronize()
    assert L.flags() == 0 and Le.flags() == 0
    n_slab, n = rows * d, m * d
    alg = ((4.0 * n + n + d * 32 * 4) + (R * n_slab + 4.0 * n_slab) + (4.0 * n_slab) + (4.0 * n_slab + n_slab)
           + (n + 4.0 * n + d * 32 * 4))
    ingress = 2 * (R - 1) * n_slab            # FP8 bytes in per GPU: all-to-all + all-gather
    result = {
        "metric": "row-slab exchange, one GPU's kernels: GB/s of the fp32 gradient (1536x6144, r=32, R=8)",
        "value": round(4.0 * n / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (the unit's layer and payloads), warm",
        "config": {"workload": f"GPU 0 of {R}: slab of {rows} rows x {d}, E4M3, one requantisation scale "
                               "shared by the slabs", "rows_per_gpu": rows, "replicas": R},
        "stages_ms": {"encode_own": round(t_encode, 5), "slab_dequant_sum": round(t_reduce, 5), "slab_amax_and_requantise": round(t_requant, 5),
                      "unwhiten_gathered": round(t_unwhiten, 5)},
        "roofline": {"bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes": int(alg)},
        "exchange": {"fp8_ingress_bytes_per_gpu": int(ingress),
                     "fp32_ring_allreduce_ingress_bytes_per_gpu": int(2 * (R - 1) * 4 * n_slab),
                     "note": "not run: one GPU"},
    }
    print(json.dumps(result), flush=True)



# ---------------------------------------------------------------------------
# Fidelity of the decoded mean ("GIFT 阅读笔记", §简化一 Eq. (15): RelL2, Cos,
# MaxErr, MSE against the uncompressed mean; the A-metric error of
# §核心想法 Eq. (6) with G = I: sqrt(tr(E A E^T) / tr(W A W^T)), A the
# undamped input statistics).  Measurement code, in float64 on the device.
# ---------------------------------------------------------------------------

def fidelity(torch, W_hat, W_ref, A=None):
    Wh, g = W_hat.double(), W_ref.double()
    e = Wh - g
    out = {"RelL2": (e.norm() / g.norm()).item(),
           "Cos": ((Wh * g).sum() / (Wh.norm() * g.norm())).item(),
           "MaxErr": e.abs().max().item(), "MSE": (e * e).mean().item()}
    if A is not None:
        Ad = A.double()
        out["ARel"] = float(((e @ Ad) * e).sum().item() / ((g @ Ad) * g).sum().item()) ** 0.5
    return {k: float(f"{v:.5g}") for k, v in out.items()}


def decoded_mean(torch, fw, L, Ws, fmt, scaling, shared_amax=False):
    """Encode every replica with layer L and decode-reduce them.  With
    shared_amax the replicas quantise with the max of their local amaxes (the
    AllReduceMax of the Euclidean branch of Algorithm 1), else each with its
    own (the geometry branch's local scale)."""
    m, d = Ws[0].shape
    nb = fw.nblocks(m, d, scaling)
    amax_in = None
    if shared_amax:
        am = torch.empty(len(Ws), nb, dtype=torch.float32, device=Ws[0].device)
        for r, W in enumerate(Ws):
            L.encode(W, fmt, scaling, amax_out=am[r], want_codes=False)
        amax_in = am.max(0).values.contiguous()
    codes = torch.empty(len(Ws), m, d, dtype=torch.uint8, device=Ws[0].device)
    scales = torch.empty(len(Ws), nb, dtype=torch.float32, device=Ws[0].device)
    for r, W in enumerate(Ws):
        L.encode(W, fmt, scaling, amax_in=amax_in, codes=codes[r], scales=scales[r])
    out = L.decode_reduce(codes, scales, fmt, scaling)
    del codes
    return out


def variant_layer(torch, fw, kind, m, d, a, dl, omega, ema=0.0, a_steps=None):
    L = fw.Layer(m, d, kind, rank=32, oversample=16, power_iters=4, ema_decay=ema, device=a.device)
    if kind != "euclid":
        for x in (a_steps or [a]):
            L.accumulate_stats(x, fw.SIDE_A, commit=True)
    if kind == "twosided":
        L.accumulate_stats(dl, fw.SIDE_G, commit=True)
    L.refresh(omega)
    return L


def fidelity_rows(torch, fw, Ws, A, layers, fmts=("e4m3",), scalings=("tensor", "block")):
    """{variant: {format/scaling: metrics}} for the given layers (kind -> L)."""
    Wbar = torch.stack([w.double() for w in Ws]).mean(0)
    rows = {}
    for kind, L in layers.items():
        rows[kind] = {}
        for fm in fmts:
            for sc in scalings:
                out = decoded_mean(torch, fw, L, Ws, fw.FORMATS[fm], fw.SCALINGS[sc], shared_amax=kind == "euclid")
                rows[kind][f"{fm}/{sc}"] = fidelity(torch, out, Wbar, A)
                del out
    return rows


def bench_ablation(args, torch, fw, synth, dev):
    """The two-sided K-FAC ablation on one 1536 x 6144 fc2 layer: A (6144^2)
    and G (1536^2) from T = 16384 bf16 tokens, E4M3 per 128 x 128 block,
    R = 8, every transform.  Times the statistics, each refresh (blocked fp64
    Cholesky and triangular inverse for the full variants, subspace
    iteration for rank 32), the encode of one replica and the decode-reduce
    of the 8 payloads, and scores each decoded mean against the fp32 mean
    gradient."""
    case = synth.make_layer(4, device=dev)
    m, d = case.cfg["m"], case.cfg["d"]
    a, dl = case.a_steps[0], case.delta_steps[0]
    f, s = fw.E4M3, fw.SCALE_BLOCK128
    nb = fw.nblocks(m, d, s)
    reps = 5
    scratch = fw.Layer(16, d, "diag", device=dev)
    t_stats_a = _event_ms(torch, lambda: scratch.accumulate_stats(a, fw.SIDE_A), reps)
    del scratch
    layers, variants = {}, {}
    for kind in ("twosided", "chol", "lowrank", "diag", "euclid"):
        L = variant_layer(torch, fw, kind, m, d, a, dl, case.omega)
        t_ref = _event_ms(torch, lambda: L.refresh(case.omega), 3) if kind != "euclid" else 0.0
        codes = torch.empty(len(case.W), m, d, dtype=torch.uint8, device=dev)
        scales = torch.empty(len(case.W), nb, dtype=torch.float32, device=dev)
        for r, W in enumerate(case.W):
            L.encode(W, f, s, codes=codes[r], scales=scales[r])
        out = torch.empty(m, d, dtype=torch.float32, device=dev)
        t_enc = _event_ms(torch, lambda: L.encode(case.W[0], f, s, codes=codes[0], scales=scales[0]), reps)
        t_dec = _event_ms(torch, lambda: L.decode_reduce(codes, scales, f, s, out=out), reps)
        torch.cuda.synchronize()
        assert L.flags() == 0, kind
        variants[kind] = {"refresh_ms": round(t_ref, 4), "encode_ms": round(t_enc, 5), "decode_ms": round(t_dec, 5),
                          "route": L.route("encode") if kind in ("lowrank", "euclid") else "multi"}
        layers[kind] = L
        del codes, out
    if "twosided" in layers:
        scratch = fw.Layer(m, 16, "twosided", device=dev)
        variants["twosided"]["stats_G_ms"] = round(
            _event_ms(torch, lambda: scratch.accumulate_stats(dl, fw.SIDE_G), reps), 4)
        del scratch
    A = layers["chol"].buffers()["A"]
    fid = fidelity_rows(torch, fw, case.W, A, layers, scalings=("block", "tensor"))
    for kind in variants:
        variants[kind]["fidelity"] = fid[kind]
    chol_flop = 2.0 * (2.0 * d ** 3 / 3.0)              # factor d^3/3 + triangular inverse d^3/3 multiply-adds
    apply_flop = 2.0 * m * d * d / 2.0                   # W L^-T: a triangular product, m d^2 / 2 multiply-adds
    result = {
        "metric": "two-sided K-FAC ablation, 1536x6144 fc2 layer: per-variant times and fidelity",
        "n_gpus": 1, "dtype": "f32", "data": "synthetic (a ~ N(0, Q_A diag(i^-1.5) Q_A^T), delta ~ "
        "N(0, Q_G diag(j^-1) Q_G^T), bf16, T=16384; W_r = delta_r^T a_r / T)",
        "config": {"workload": "fc2 1536x6144, A 6144^2 and G 1536^2 from 16384 bf16 tokens, E4M3 per 128x128 "
                               "block (fidelity also per tensor), R=8", "replicas": len(case.W)},
        "stats_A_ms": round(t_stats_a, 4),
        "variants": variants,
        "flops": {"cholesky_and_inverse_A": chol_flop, "triangular_apply_each_way": apply_flop},
        "fp64_fraction": {"cholesky_refresh": round(chol_flop / (variants["chol"]["refresh_ms"] * 1e-3) / 1e12
                                                    / FP64_PEAK_TFS, 4),
                          "triangular_apply_encode": round(apply_flop / (variants["chol"]["encode_ms"] * 1e-3) / 1e12
                                                           / FP64_PEAK_TFS, 4)},
        "fidelity_note": "decoded mean of the 8 replicas against their fp32 mean; Euclidean with the shared "
                         "amax (AllReduceMax), the others with local scales; ARel uses the undamped A",
    }
    print(json.dumps(result), flush=True)


def bench_fidelity(args, torch, fw, synth, dev):
    """Fidelity of every configuration's decoded mean against the fp32 mean
    of its replicas (the synthetic analogue of Tables I and II)."""
    res = {}
    t0 = time.time()
    # tiny: 64 x 256, fp32 activations, R = 4; every input-side variant
    c1 = synth.make_layer(1, device=dev)
    lay = {k: variant_layer(torch, fw, k, 64, 256, c1.a_steps[0], c1.delta_steps[0], c1.omega)
           for k in ("euclid", "diag", "lowrank", "chol", "twosided")}
    res["tiny_64x256_r4"] = fidelity_rows(torch, fw, c1.W, lay["chol"].buffers()["A"], lay)
    del lay
    # 300M fc2: 1024 x 4096, 4 EMA steps (beta 0.95), R = 8
    c2 = synth.make_layer(2, device=dev)
    lay = {k: variant_layer(torch, fw, k, 1024, 4096, c2.a_steps[-1], None, c2.omega, ema=0.95, a_steps=c2.a_steps)
           for k in ("euclid", "lowrank")}
    res["fc2_300m_1024x4096_r8"] = fidelity_rows(torch, fw, c2.W, lay["lowrank"].buffers()["A"], lay)
    del lay, c2
    # 600M fc2 (the metric layer and the ablation): every variant
    c4 = synth.make_layer(4, device=dev)
    lay = {k: variant_layer(torch, fw, k, 1536, 6144, c4.a_steps[0], c4.delta_steps[0], c4.omega)
           for k in ("euclid", "diag", "lowrank", "chol", "twosided")}
    res["fc2_600m_1536x6144_r8"] = fidelity_rows(torch, fw, c4.W, lay["chol"].buffers()["A"], lay)
    del lay, c4
    torch.cuda.empty_cache()
    # stress: 4096 x 16384, Student-t gradients with outlier columns, R = 16
    m, d, Ttok = 4096, 16384, 8192
    a = synth.stress_activations(Ttok, d, 0, dev)
    om = synth.omega(d, 48, synth.seed_for(5, synth.ROLE_OMEGA), dev)
    Ws = [synth.stress_gradient(m, d, 0, r, dev) for r in range(16)]
    lay = {k: variant_layer(torch, fw, k, m, d, a, None, om) for k in ("euclid", "lowrank")}
    res["stress_4096x16384_r16"] = fidelity_rows(torch, fw, Ws, lay["lowrank"].buffers()["A"], lay,
                                                 fmts=("e5m2", "e4m3"), scalings=("block",))
    del lay, Ws, a
    result = {"metric": "fidelity of the decoded mean against the fp32 mean gradient, every configuration",
              "n_gpus": 1, "data": "synthetic, seeded", "seconds": round(time.time() - t0, 1),
              "note": "RelL2, Cos, MaxErr, MSE (Eq. (15)) and ARel = sqrt(tr(E A E^T) / tr(W A W^T)) with the "
                      "layer's undamped A; Euclidean quantises with the shared amax (AllReduceMax), the other "
                      "variants with local scales; keys are format/scaling",
              "fidelity": res}
    print(json.dumps(result), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, A_gpu, R, m, d, scaling, budget_s=10.0, max_units=30):
    """The oracle (numpy fp64) on the same unit: encode of one replica +
    decode-reduce of R payloads, with the oracle's own dense T_A (built from
    the GPU's A outside the timed part).  Whole units are repeated until
    about `budget_s` seconds of CPU work have run (at most `max_units`), with
    the BLAS threads numpy has; then one whole unit with one BLAS thread, and
    each stage of the path on its own (statistics on a 2048-token sample
    scaled to the layer's 16384 tokens, refresh, whiten, quantise,
    decode-reduce)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import gift as G
    A = A_gpu.double().cpu().numpy()
    omega = case.omega.cpu().numpy()
    lam = G.damping(A)
    T, Tinv = G.transform_lowrank(G.lowrank_factor(A, omega, 32, 4, lam))
    Ws = [w.cpu().numpy() for w in case.W]
    pre = [G.encode(Ws[r], T, "e4m3", scaling) for r in range(1, R)]

    def unit():
        e0 = G.encode(Ws[0], T, "e4m3", scaling)
        G.decode_reduce([e0["codes"]] + [p["codes"] for p in pre], [e0["scales"]] + [p["scales"] for p in pre],
                        Tinv, "e4m3", scaling)

    units = 0
    t0 = time.perf_counter()
    while True:
        unit()
        units += 1
        t = time.perf_counter() - t0
        if t >= budget_s or units >= max_units:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])

    def once(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    grad_gb = 4.0 * m * d / 1e9
    with threadpool_limits(limits=1):
        t1 = once(unit)
    a = case.a_steps[0]
    T_tok = a.shape[0]
    sample = a[:2048].float().cpu().numpy()
    enc0 = G.encode(Ws[0], T, "e4m3", scaling)
    stages = {
        "stats_ms": once(lambda: G.second_moment(sample)) * 1e3 * (T_tok / sample.shape[0]),
        "refresh_ms": once(lambda: G.lowrank_factor(A, omega, 32, 4, lam)) * 1e3,
        "whiten_ms": once(lambda: G.whiten(Ws[0], T)) * 1e3,
        "quantise_ms": once(lambda: G.quantize(enc0["whitened"], "e4m3", scaling)) * 1e3,
        "decode_reduce_ms": once(lambda: G.decode_reduce([enc0["codes"]] + [p["codes"] for p in pre],
                                                         [enc0["scales"]] + [p["scales"] for p in pre], Tinv,
                                                         "e4m3", scaling)) * 1e3,
    }
    return {"value": round(units * grad_gb / t, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{units} full units (encode 1 replica + decode-reduce 8) at 1536x6144, numpy fp64 "
                      "with dense T_A, BLAS threads as listed",
            "seconds": round(t, 3), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
            "one_thread": {"value": round(grad_gb / t1, 4), "unit": "GB/s", "seconds": round(t1, 3),
                           "sample": "1 full unit, BLAS limited to 1 thread"},
            "stages_ms": {k: round(v, 1) for k, v in stages.items()},
            "stages_note": "one run each with the BLAS threads above; statistics timed on 2048 of the 16384 "
                           "tokens and scaled"}


def kernel_source_sha():
    """Hash of the sources the fused kernels are built from: k_fused.hip,
    fp8_codec.hpp and the FusedArgs declaration of gift_internal.hpp."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fac_whitening_amd", "csrc")
    for f in ("k_fused.hip", "fp8_codec.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(csrc, "gift_internal.hpp")) as fh:
        text = fh.read()
    i = text.index("struct FusedArgs {")
    h.update(text[i:text.index("};", i)].encode())
    return h.hexdigest()


def measured_traffic(kernel, scaling):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE passes, scaled by the copy factor), or None
    when there is none for this scaling or the kernel source has changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "k_rank_traffic_1536x6144_r8.md")
    if not os.path.exists(path):
        return None
    sha = kernel_source_sha()
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-json: "):
                rec = json.loads(line[len("traffic-json: "):])
                if rec.get("kernel") == kernel and rec.get("scaling") == scaling and rec.get("source_sha256") == sha:
                    return rec["bytes_per_launch"]
    return None


if __name__ == "__main__":
    main()
