"""Benchmark: encode + decode of a Qwen3-32B-shaped bf16 KV cache on one MI355X.

One step = skv_encode + skv_decode of the whole cache (64 layers x {K,V} x 8
KV heads x 8192 tokens x 128), inputs resident in HBM.  sigma and p_hat are
calibrated on the GPU first (128 seeded sequences of 512 tokens, not timed).
Prints one JSON line: `value` = raw-KV GB/s of the round trip over the wall
clock of the timed steps; per-direction GB/s and HBM fractions from the median
of HIP events around each ABI call (model build included); bits/scalar; the
roofline of the dominant kernel from its average launch time, taken by the
library's own event pairs on the launch stream during the timed steps; and the
CPU oracle timed on a bounded sample of the same workload.
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "encode & decode GB/s of raw KV (bf16, e4m3), % HBM roofline; bits/scalar"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="qwen3_32b_bf16")
    p.add_argument("--calib-seqs", type=int, default=None, help="calibration sequences (default: the workload's 128)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--traffic-probe", action="store_true",
                   help="for rocprofv3 --pmc: one 1 GiB device copy (the scale reference), then one "
                        "encode + decode, no timing")
    return p.parse_args()


def csrc_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "lossless_kv_cache_scalar_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def counter_record(kernel: str, workload: str):
    """The committed rocprofv3 counter record of a kernel on a workload
    (profiles/traffic_<kernel>_<workload>.json), if it was taken on the
    current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("csrc_hash") != csrc_hash() or rec.get("workload") != workload:
        return None
    return rec


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs (FETCH_SIZE and
    WRITE_SIZE scaled by a copy of known size), or None."""
    rec = counter_record(kernel, workload)
    return None if rec is None else rec.get("bytes_per_launch")


# VALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one pass of a 64-lane
# instruction every 4 cycles (simple 32-bit adds, logic and fp32 fma can issue
# faster, so a kernel made mostly of them can exceed it)
VALU_PEAK_LANE_INSTR_PER_S = 256 * 4 * 16 * 2.4e9


def valu_use(kernel: str, workload: str, n_symbols: int, launch_ms: float):
    """VALU instructions per symbol from the committed SQ_INSTS_VALU counter run,
    and the lane-instruction rate they imply at the measured launch time."""
    rec = counter_record(kernel, workload)
    if rec is None or not rec.get("valu_instr_per_symbol"):
        return None
    per = float(rec["valu_instr_per_symbol"])
    rate = per * n_symbols / (launch_ms * 1e-3)
    return {"instr_per_symbol": per, "achieved": round(rate / 1e12, 3), "peak": round(VALU_PEAK_LANE_INSTR_PER_S / 1e12, 3),
            "unit": "T lane-instr/s", "frac": round(rate / VALU_PEAK_LANE_INSTR_PER_S, 4),
            "source": "SQ_INSTS_VALU x 64 / symbols, counter run on the same kernel sources"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: chunks code independently, and it measures one GPU's share "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lossless_kv_cache_scalar_amd import build as B
    from lossless_kv_cache_scalar_amd import skv, synth

    if not B.is_built():
        B.build()
    skv.load()
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    nseq = w.calib_seqs if args.calib_seqs is None else args.calib_seqs

    # ---- inputs in HBM (not timed)
    t0 = time.time()
    x, mu = synth.generate(w, device=dev)
    csh = skv.shape(w.layers, w.kv_heads, w.calib_tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode)
    state = torch.empty(skv.calib_state_size(csh), dtype=torch.uint8, device=dev)
    sigma = torch.empty(skv.sigma_floats(csh), dtype=torch.float32, device=dev)
    hist = torch.empty(65536 if w.sym_fmt == 0 else 256, dtype=torch.int64, device=dev)
    assert skv.calib_reset(state, csh) == skv.OK
    for j in range(nseq):
        cx, cm = synth.calibration_set(w, j, device=dev)
        assert skv.calib_accumulate(state, csh, cx, cm) == skv.OK
        del cx, cm
    assert skv.calib_finalize(state, csh, sigma, hist) == skv.OK
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s: {w.name}, {w.n_scalars} scalars, {nseq} calibration sequences",
          file=sys.stderr, flush=True)

    sh = skv.shape(w.layers, w.kv_heads, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode, w.phat_mode)
    buf = skv.Buffers(sh, device=dev)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    if args.traffic_probe:
        # a plain elementwise copy of exactly 1 GiB (read 1 GiB, write 1 GiB): its
        # FETCH_SIZE / WRITE_SIZE readings give the counters' scale; then one
        # encode and one decode of the workload
        src = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        buf.encode(x, mu, sigma, hist, stream)
        buf.decode(mu, sigma, hist, out, stream=stream)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": w.name, "copy_bytes": 1 << 30, "stream_bytes": buf.stream_bytes(),
                          "n_scalars": w.n_scalars, "n_chunks": buf.n_chunks, "sym_bytes": w.sym_bytes,
                          "mu_bytes": w.mu_bytes, "exact": bool(torch.equal(out, x)),
                          "csrc_hash": csrc_hash()}), flush=True)
        return

    # encode and decode report into separate status words, so both are known
    # after the timed steps without a synchronisation between the two calls
    dstatus = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        buf.encode(x, mu, sigma, hist, stream)
        if ev is not None:
            ev[1].record(stream)
        buf.decode(mu, sigma, hist, out, stream=stream, status=dstatus)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    copy_gbps = measured_copy_peak(torch, dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    # per-kernel HIP events, recorded by the library on the launch stream
    skv.timing_start(8 * args.steps + 8)
    torch.cuda.synchronize()
    tstart = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - tstart
    recs = skv.timing_stop(8 * args.steps + 8)
    kern_ms = {}
    for name, ms in recs:
        kern_ms.setdefault(name, []).append(ms)
    kern_avg = {k: float(np.mean(v)) for k, v in kern_ms.items()}
    enc_ms = float(np.median([e[0].elapsed_time(e[1]) for e in events]))
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in events]))
    ms_per_step = wall * 1000.0 / args.steps

    enc_status = int(buf.status.item())
    dec_status = int(dstatus.item())
    status = enc_status if enc_status != skv.OK else dec_status
    exact = bool(torch.equal(out, x))
    nbytes = buf.stream_bytes()
    n = w.n_scalars
    raw = n * w.sym_bytes
    bits_per_scalar = 8.0 * (nbytes + 8 * (buf.n_chunks + 1)) / n
    # algorithmic bytes of one direction: x and mu one way, the stream (with its
    # offsets) the other
    moved = n * (w.sym_bytes + w.mu_bytes) + nbytes + 8 * (buf.n_chunks + 1)
    enc_gbps = raw / enc_ms / 1e6
    dec_gbps = raw / dec_ms / 1e6
    enc_hbm = moved / enc_ms / 1e6
    dec_hbm = moved / dec_ms / 1e6
    kern = "k_decode" if kern_avg["k_decode"] >= kern_avg["k_encode"] else "k_encode"
    kms = kern_avg[kern]
    traffic = measured_traffic(kern, w.name)
    hbm_gbps = moved / kms / 1e6
    hbm = {"achieved": round(hbm_gbps, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(hbm_gbps / HBM_PEAK_GBPS, 5), "traffic": traffic, "bytes_per_launch": moved,
           "bytes_per_scalar": round(moved / n, 5), "measured_copy_peak": round(copy_gbps, 1),
           "frac_of_measured_copy_peak": round(hbm_gbps / copy_gbps, 5)}
    valu = valu_use(kern, w.name, n, kms)
    if valu is not None and valu["frac"] > hbm["frac"]:
        # the counters say the kernel is limited by VALU issue: that is its roofline
        roofline = {"kernel": kern, "bound": "alu", "achieved": valu["achieved"], "peak": valu["peak"],
                    "unit": valu["unit"], "frac": valu["frac"], "traffic": traffic, "launch_ms": round(kms, 4),
                    "work": f"{valu['instr_per_symbol']} VALU instructions per symbol (SQ_INSTS_VALU x 64 / symbols "
                            "on the same kernel sources; the method fixes no operation count)",
                    "hbm": hbm}
    else:
        roofline = {"kernel": kern, "bound": "hbm", "launch_ms": round(kms, 4), **hbm, "valu": valu}

    result = {
        "metric": METRIC,
        "value": round(raw / (ms_per_step / 1000.0) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+u64",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "kv_heads": w.kv_heads, "tokens": w.tokens,
                   "head_dim": w.head_dim, "symbols": "bf16" if w.sym_fmt == 0 else "e4m3",
                   "mu": "bf16" if w.mu_fmt == 0 else "f32", "n_scalars": n, "calib_seqs": nseq,
                   "calib_tokens": w.calib_tokens, "chunk_tokens": 256, "lanes_per_chunk": 64,
                   "sigma": "channel x |mu| octave" if w.sigma_mode else "channel",
                   "p_hat": "adaptive (decayed counts per chunk)" if w.phat_mode else "calibrated histogram"},
        "encode_GBps": round(enc_gbps, 3),
        "decode_GBps": round(dec_gbps, 3),
        "encode_ms": round(enc_ms, 4),
        "decode_ms": round(dec_ms, 4),
        "encode_hbm_frac": round(enc_hbm / HBM_PEAK_GBPS, 5),
        "decode_hbm_frac": round(dec_hbm / HBM_PEAK_GBPS, 5),
        "bits_per_scalar": round(bits_per_scalar, 5),
        "compression_ratio": round(16.0 / bits_per_scalar if w.sym_fmt == 0 else 8.0 / bits_per_scalar, 4),
        "stream_bytes": nbytes,
        "roundtrip_exact": exact,
        "status": skv.status_string(status),
        "roofline": roofline,
        "kernel_ms": {k: round(v, 4) for k, v in sorted(kern_avg.items())},
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, mu, sigma, hist, buf, args.cpu_seconds)
    result["encode_status"] = skv.status_string(enc_status)
    result["decode_status"] = skv.status_string(dec_status)
    print(json.dumps(result), flush=True)
    if not exact or status != skv.OK:
        sys.exit(1)


def measured_copy_peak(torch, dev, reps=10):
    """HBM bandwidth of a plain device copy of 1 GiB (1 GiB read + 1 GiB
    written per copy), the median of `reps` timed copies, in GB/s."""
    src = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    times.sort()
    return 2.0 * (1 << 30) / (times[len(times) // 2] * 1e-3) / 1e9


def cpu_baseline(w, x, mu, sigma, hist, buf, seconds):
    """The CPU oracle, as it stands, on a bounded sample of chunks of the same
    cache; also checks those chunks' GPU bytes against it."""
    import numpy as np

    from oracle import skvref as R

    cores = max(1, min(os.cpu_count() or 1, 16))
    rsig = sigma.cpu().numpy()
    per_ch = R.OCT_STRIDE if w.sigma_mode == R.SIGMA_OCTAVE else 1
    rhist = hist.cpu().numpy().view(np.uint64)
    model = R.Model(w.sym_fmt, rhist)
    ntb = (w.tokens + 255) // 256
    rows_per_layer = 2 * w.kv_heads

    def sample(n_rows):
        # whole (layer, kv, head) rows from the front of the cache, all their chunks
        xs = x.reshape(-1, w.tokens, w.head_dim)[:n_rows].cpu().numpy()
        ms = mu.reshape(-1, w.tokens, w.head_dim)[:n_rows].cpu().numpy()
        xs = np.ascontiguousarray(xs.view(np.uint16 if w.sym_fmt == 0 else np.uint8))
        ms = np.ascontiguousarray(ms.view(np.uint16) if w.mu_fmt == 0 else ms)
        shp = (R.make_shape(1, n_rows // 2, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode, w.phat_mode)
               if n_rows % 2 == 0 else None)
        return xs, ms, shp

    def run(n_rows, threads=cores):
        xs, ms, shp = sample(n_rows)
        sig = np.ascontiguousarray(rsig[: n_rows * w.head_dim * per_ch])
        t0 = time.perf_counter()
        bits, offs = model.encode(shp, xs, ms, sig, nthreads=threads)
        t1 = time.perf_counter()
        dec, st = model.decode(shp, bits, offs, ms, sig, nthreads=threads)
        t2 = time.perf_counter()
        return xs, bits, offs, dec, st, t1 - t0, t2 - t1

    # one core on one (layer, kv) pair of rows
    xs1, _, _, dec1, st1, te1, td1 = run(2, threads=1)
    raw1 = xs1.size * w.sym_bytes
    single = {"encode_GBps": round(raw1 / te1 / 1e9, 5), "decode_GBps": round(raw1 / td1 / 1e9, 5),
              "value": round(raw1 / (te1 + td1) / 1e9, 5), "sample": f"2 rows, {xs1.size} scalars, 1 thread",
              "roundtrip_exact": bool(st1 == R.OK and np.array_equal(dec1, xs1))}
    # size the sample: one row pair first, then as many rows as fit the time budget
    _, _, _, _, _, te, td = run(2)
    per_row = (te + td) / 2
    n_rows = int(max(2, min(w.layers * rows_per_layer, seconds / max(per_row, 1e-6))))
    n_rows -= n_rows % 2
    xs, bits, offs, dec, st, te, td = run(n_rows)
    n = xs.size
    raw = n * w.sym_bytes
    # the sample's chunks are the GPU stream's first chunks: compare bytes
    nchunks = n_rows * ntb
    goffs = buf.offsets[: nchunks + 1].cpu().numpy().view(np.uint64)
    gbits = buf.bits[: int(goffs[-1])].cpu().numpy()
    same = bool(np.array_equal(goffs, offs) and np.array_equal(gbits, bits))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(raw / (te + td) / 1e9, 5),
        "unit": "GB/s",
        "cores": cores,
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"{n_rows} of {w.layers * rows_per_layer} (layer, kv, head) rows = {nchunks} chunks, "
                  f"{n} scalars, encode + decode",
        "encode_GBps": round(raw / te / 1e9, 5),
        "decode_GBps": round(raw / td / 1e9, 5),
        "seconds": round(te + td, 3),
        "single_core": single,
        "gpu_bytes_match_oracle": same,
        "oracle_roundtrip_exact": bool(st == R.OK and np.array_equal(dec, xs)),
    }


if __name__ == "__main__":
    main()
