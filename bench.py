"""Benchmark of the FibQuant hot path on one MI355X.

A step is one pass of the whole hot path over the GPT-2-small-shaped KV
workload (294,912 fp16 vectors = 12 layers x 12 heads x 1024 tokens x {K, V},
d = 64, codebook k = 4, N = 256, b = 2 bits per coordinate):

    fq_encode   all 294,912 vectors -> fixed-address codes + fp16 norms
    fq_decode   all codes -> fp16 reconstructions
    fq_attn_decode  one decode query per (layer, head) over the encoded cache
                (layers act as the batch, 12 query heads on 12 KV heads,
                T = 1024) straight from the codes

Inputs are resident in HBM before timing starts.  The metric is KV vectors per
second through the step (fp16-equivalent GB/s = vectors/s x 128 B).  Per-kernel
times come from HIP events on the stream the library launches on.  The
decode-attention workload (B=16, 32 query heads on 4 KV heads, T=32768) is
timed separately with L2 and the last-level cache evicted before every launch
(a 512 MiB read), and reported against the HBM roofline.  On the same cache a
decode loop is timed as well: per step the new token's K and V are encoded into
their slots (fq_encode_scatter) and attention runs over each sequence's valid
length (fq_attn_decode_varlen).  Along the rate axis (frozen initial codebooks
from b = 4 down to 0.22 bits per coordinate) the same tensor's encode, decode
and attention are timed as well, and so are prefill attention (64 causal
queries per head on the 32k cache) and the codebook construction
(fq_codebook_train) at larger shapes.  The CPU oracle is timed on a bounded sample
(rank 0, one GPU only).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV vectors/sec encode+decode (GB/s fp16-equiv) and fused-attn GB/s; % roofline"
HBM_PEAK_GBPS = 8000.0
# VALU lane-op rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s.  A
# three-input minimum resolves two comparisons per lane-op, so the search's
# compare work peaks at 78.6 T comparisons/s (the same figure as non-packed FMAs).
VALU_LANE_OPS = 256 * 64 * 2.4e9
CMP_PEAK_T = 2 * VALU_LANE_OPS / 1e12
D = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--attn-iters", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attn-workload", action="store_true")
    ap.add_argument("--no-decode-loop", action="store_true", help="skip the append + varlen attention timing")
    ap.add_argument("--no-rate-axis", action="store_true", help="skip the rate-axis timings")
    ap.add_argument("--no-build", action="store_true", help="skip the codebook-construction timings")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill attention timing")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload encode/decode timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def source_sha(name: str) -> str:
    p = os.path.join(ROOT, "universal_vector_quantization_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel: str, src: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(kernel)
    if not rec or rec.get("source_sha") != source_sha(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(budget_s: float = 12.0):
    """The oracle as it stands, on a bounded sample of the same step."""
    import workloads
    from oracle import attention as oatt
    from oracle import codec as oc

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    import universal_vector_quantization_amd as fq

    cw, rot = fq.load_artifact(4, 256)
    x = workloads.gpt2_small_kv()
    # size the sample from a 2048-vector calibration so the encode takes about budget_s
    t0 = time.perf_counter()
    oc.encode(x[:2048], rot, cw, np.float16)
    t_cal = time.perf_counter() - t0
    n_s = int(min(len(x), max(2048, 2048 * budget_s / max(t_cal, 1e-3))) // 2048 * 2048)
    # the whole tensor encodes in less than the budget on a many-core host: repeat the
    # timed encode (at most 5 times) until the budget is spent
    reps, t_enc = 0, 0.0
    while reps < 5 and (reps == 0 or t_enc < budget_s):
        t0 = time.perf_counter()
        enc = oc.encode(x[:n_s], rot, cw, np.float16)
        t_enc += time.perf_counter() - t0
        reps += 1
    t_enc /= reps
    t0 = time.perf_counter()
    oc.round_output(oc.decode(enc.codes, enc.norms, rot, cw), np.float16)
    t_dec = time.perf_counter() - t0
    # attention: one (layer, head) query over its 1024 keys and 1024 values
    T = workloads.GPT2_T
    kx = x[:T]
    vx = x[len(x) // 2: len(x) // 2 + T]
    ke = oc.encode(kx, rot, cw, np.float16)
    ve = oc.encode(vx, rot, cw, np.float16)
    q = workloads.gpt2_small_queries()[:1, :1]
    t0 = time.perf_counter()
    oatt.attention(q, ke.codes.reshape(1, 1, T, 16), ke.norms.reshape(1, 1, T), ve.codes.reshape(1, 1, T, 16),
                   ve.norms.reshape(1, 1, T), rot, cw, 0.125)
    t_att = time.perf_counter() - t0
    per_vec = t_enc / n_s + t_dec / n_s + t_att / (2 * T)
    return {"value": 1.0 / per_vec, "unit": "vectors/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle encode (x{reps}) + decode of the first {n_s} of the 294912 vectors plus attention "
                      f"of one (layer, head) query over its {T} keys/values; per-vector times summed "
                      f"(encode {t_enc:.2f}s per pass, decode {t_dec:.3f}s, attention {t_att:.3f}s)"}


# decoder kernel whose HBM bytes per launch (rocprofv3 counters) each workload reports
DECODE_TRAFFIC_KEYS = {"gpt2s_kv": "decode_stream_k4", "tinyllama_kv": "decode_stream_k8",
                       "fullvec_kv": "decode_full_k64"}


def workload_timings(fq, workloads, dev, stream, reps: int = 5):
    """Encode and decode time of every codec workload at full size (event-timed,
    median of ``reps`` launches; inputs resident, no cache flush)."""
    import torch

    out = {}
    gens = {"iid4096": lambda: workloads.iid_gaussian(4096, 101), "gpt2s_kv": workloads.gpt2_small_kv,
            "tinyllama_kv": workloads.tinyllama_kv, "fullvec_kv": workloads.fullvec_kv}
    for name, gen in gens.items():
        w = workloads.WORKLOADS[name]
        try:
            cb = fq.Codebook.from_artifact(w.k, w.N)
        except FileNotFoundError:
            out[name] = {"skipped": "codebook artifact missing"}
            continue
        x = torch.from_numpy(gen()).to(dev)
        n = x.shape[0]
        codes = torch.empty(cb.code_bytes(n), dtype=torch.uint8, device=dev)
        norms = torch.empty(n, dtype=torch.float16 if w.norm_dtype == "f16" else torch.float32, device=dev)
        xr = torch.empty_like(x)
        te, td = [], []
        for r in range(reps + 1):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            fq.fq_encode(cb.handle, x, codes, norms, stream)
            e[1].record(stream)
            fq.fq_decode(cb.handle, codes, norms, xr, stream)
            e[2].record(stream)
            torch.cuda.synchronize()
            if r:
                te.append(e[0].elapsed_time(e[1]))
                td.append(e[1].elapsed_time(e[2]))
        t_e, t_d = float(np.median(te)) / 1e3, float(np.median(td)) / 1e3
        vb = x.element_size() * D + norms.element_size() + cb.code_bytes(n) / n
        dk = DECODE_TRAFFIC_KEYS.get(name)
        out[name] = {"n": n, "k": w.k, "N": w.N, "encode_us": t_e * 1e6, "decode_us": t_d * 1e6,
                     "decode_traffic": measured_traffic(dk, "fq_decode_mfma.hip") if dk else None,
                     "encode_vec_per_s": n / t_e, "decode_vec_per_s": n / t_d,
                     "encode_GBps": n * vb / t_e / 1e9, "decode_GBps": n * vb / t_d / 1e9,
                     "decode_hbm_frac": n * vb / t_d / 1e9 / HBM_PEAK_GBPS,
                     "encode_cmp_frac": (D // w.k) * w.N * n / t_e / 1e12 / CMP_PEAK_T}
        cb.close()
        del x, codes, norms, xr
        torch.cuda.empty_cache()
    return out


# Rate-axis points (k, N) with frozen initial codebooks: b = log2(N) / k from 4 down to 0.22.
RATE_AXIS = [(1, 16), (2, 32), (2, 128), (4, 1024), (4, 16384), (16, 1024), (32, 512), (64, 16384)]


def rate_axis_timings(fq, workloads, dev, stream, reps: int = 3):
    """Encode, decode and decode-attention time along the rate axis on the
    GPT-2-small-shaped tensor (294,912 fp16 vectors; event-timed, median of
    ``reps``, inputs resident).  Attention: one query per (layer, head) over the
    just-encoded halves (B = 12, Hq = Hkv = 12, T = 1024), where the codebook fits
    in LDS."""
    import torch

    x = torch.from_numpy(workloads.gpt2_small_kv()).to(dev)
    n = x.shape[0]
    L, H, T = workloads.GPT2_L, workloads.GPT2_H, workloads.GPT2_T
    q = torch.from_numpy(workloads.gpt2_small_queries()).to(dev)
    ao = torch.empty((L, H, D), dtype=torch.float32, device=dev)
    out = {}

    def timed(fn):
        ts = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)) / 1e3

    for k, N in RATE_AXIS:
        try:
            cb = fq.Codebook.from_artifact(k, N, initial=True)
        except FileNotFoundError:
            out[f"k{k}_N{N}"] = {"skipped": "codebook artifact missing"}
            continue
        bits = N.bit_length() - 1
        codes = torch.empty(cb.code_bytes(n), dtype=torch.uint8, device=dev)
        norms = torch.empty(n, dtype=torch.float16, device=dev)
        xr = torch.empty_like(x)
        t_e = timed(lambda: fq.fq_encode(cb.handle, x, codes, norms, stream))
        t_d = timed(lambda: fq.fq_decode(cb.handle, codes, norms, xr, stream))
        dbytes = cb.code_bytes(n) + 2 * n + 2 * D * n  # codes + norms read, fp16 output written
        rec = {"b": bits / k, "record_bits": (D // k) * bits, "encode_us": t_e * 1e6, "encode_vec_per_s": n / t_e,
               "encode_cmp_frac": (D // k) * N * n / t_e / 1e12 / CMP_PEAK_T, "decode_us": t_d * 1e6,
               "decode_GBps": dbytes / t_d / 1e9, "decode_hbm_frac": dbytes / t_d / 1e9 / HBM_PEAK_GBPS}
        if k * N <= 16384:
            half = cb.code_bytes(n // 2)
            ws = torch.empty(max(fq.fq_attn_workspace_bytes(cb.handle, L, H, H, T), 16), dtype=torch.uint8,
                             device=dev)
            t_a = timed(lambda: fq.fq_attn_decode(cb.handle, q, codes[:half], norms[: n // 2], codes[half:],
                                                  norms[n // 2:], L, H, H, T, 0.125, ao, ws, stream))
            abytes = cb.code_bytes(n) + 2 * n + L * H * D * 6
            rec.update({"attention_us": t_a * 1e6, "attention_GBps": abytes / t_a / 1e9})
        out[f"k{k}_N{N}"] = rec
        cb.close()
        del codes, norms, xr
    return out


# Codebook-construction shapes: (k, N, training blocks); starts are the frozen initial codebooks.
BUILD_SHAPES = [(4, 1024, 262144), (4, 16384, 1048576), (64, 16384, 262144)]
FP64_VALU_PEAK_T = 78.6  # dense fp64 vector FLOP/s of the MI355X, in T
FP16_MFMA_PEAK_T = 2500.0  # dense fp16 matrix FLOP/s of the MI355X, in T


def build_timings(fq, workloads, dev, stream, iters: int = 5):
    """fq_codebook_train at larger shapes: `iters` Lloyd updates from the frozen
    initial codebook (rel_tol 0), 1024 validation blocks.  The assignment pass is
    the work: m N (2k + 2) fp64 flops (dot product, score, compare) per pass, and a
    call makes iters + 3 passes (one before the first update, one after each, two
    validations of 1024 blocks)."""
    import torch

    out = {}
    for k, N, m in BUILD_SHAPES:
        try:
            cw0, _ = fq.load_artifact(k, N, initial=True)
        except FileNotFoundError:
            out[f"k{k}_N{N}"] = {"skipped": "initial codebook artifact missing"}
            continue
        train = torch.from_numpy(workloads.canonical_blocks(D, k, m, 400 + k)).to(dev)
        valid = torch.from_numpy(workloads.canonical_blocks(D, k, 1024, 500 + k)).to(dev)
        starts = torch.from_numpy(cw0.astype(np.float64)[None]).to(dev)
        cw = torch.empty((N, k), dtype=torch.float32, device=dev)
        ws = torch.empty(fq.fq_codebook_train_workspace_bytes(k, N, m, 1024), dtype=torch.uint8, device=dev)
        fq.fq_codebook_train(train, valid, starts, 1, 0.0, cw, workspace=ws, stream=stream)  # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = fq.fq_codebook_train(train, valid, starts, iters, 0.0, cw, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        passes = len(res["history"])  # training assignments; validation passes are 1024 blocks each
        flops = passes * m * N * (2 * k + 2)
        out[f"k{k}_N{N}"] = {"training_blocks": m, "updates": passes - 1, "seconds": t,
                             "ms_per_update": t * 1e3 / max(passes - 1, 1),
                             "assign_TFLOPs": flops / t / 1e12,
                             "assign_frac_fp64_valu": flops / t / 1e12 / FP64_VALU_PEAK_T,
                             "train_mse_first_last": [res["history"][0], res["history"][-1]]}
        del train, valid, starts, cw, ws
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)
    import torch

    import universal_vector_quantization_amd as fq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale factor between counter readings and bytes moved.
        nbytes = 256 * 1024 * 1024
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)
        return

    # ---------------------------------------------------------------- headline workload
    w = workloads.WORKLOADS["gpt2s_kv"]
    cb = fq.Codebook.from_artifact(w.k, w.N)
    x_np = workloads.gpt2_small_kv(w.seed)
    n = len(x_np)
    x = torch.from_numpy(x_np).to(dev)
    codes = torch.empty(cb.code_bytes(n), dtype=torch.uint8, device=dev)
    norms = torch.empty(n, dtype=torch.float16, device=dev)
    xr = torch.empty_like(x)
    L, H, T = workloads.GPT2_L, workloads.GPT2_H, workloads.GPT2_T
    q = torch.from_numpy(workloads.gpt2_small_queries()).to(dev)
    half_bytes = cb.code_bytes(n // 2)
    k_codes, v_codes = codes[:half_bytes], codes[half_bytes:]
    k_norms, v_norms = norms[: n // 2], norms[n // 2:]
    attn_out = torch.empty((L, H, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fq.fq_attn_workspace_bytes(cb.handle, L, H, H, T), 16), dtype=torch.uint8, device=dev)

    ev = {k: [] for k in ("enc", "dec", "att")}

    def step(record: bool):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        fq.fq_encode(cb.handle, x, codes, norms, stream)
        if record:
            e[1].record(stream)
        fq.fq_decode(cb.handle, codes, norms, xr, stream)
        if record:
            e[2].record(stream)
        fq.fq_attn_decode(cb.handle, q, k_codes, k_norms, v_codes, v_norms, L, H, H, T, 0.125, attn_out, ws, stream)
        if record:
            e[3].record(stream)
            ev["enc"].append((e[0], e[1]))
            ev["dec"].append((e[1], e[2]))
            ev["att"].append((e[2], e[3]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    ms_step = elapsed * 1e3 / args.steps
    value = n * args.steps / elapsed

    # dominant kernel roofline: the encoder's nearest-codeword search; every
    # candidate score needs at least one comparison (two per three-input min)
    cmp_per_vec = (D // w.k) * w.N
    enc_s = ms["enc"] / 1e3
    achieved = cmp_per_vec * n / enc_s / 1e12
    enc_bytes = n * (D * 2 + 2) + cb.code_bytes(n)
    dec_bytes = enc_bytes
    att_bytes = 2 * cb.code_bytes(n // 2) + 2 * (n // 2) * 2 + L * H * D * 2 + L * H * D * 4
    traffic = measured_traffic("encode_h16_k4", "fq_encode_h16.hip")
    line = {
        "metric": METRIC, "value": value, "unit": "vectors/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "gpt2s_kv", "vectors": n, "layout": "[2 KV][12 layers][12 heads][1024 tokens][64]",
                   "input_dtype": "f16", "d": D, "k": w.k, "N": w.N, "bits_per_coordinate": np.log2(w.N) / w.k,
                   "step": "fq_encode + fq_decode + fq_attn_decode(B=12 layers, Hq=Hkv=12, T=1024)"},
        "fp16_equiv_GBps": value * D * 2 / 1e9,
        "breakdown_us": {"encode": ms["enc"] * 1e3, "decode": ms["dec"] * 1e3, "attention": ms["att"] * 1e3},
        "breakdown_GBps": {"encode": enc_bytes / (ms["enc"] / 1e3) / 1e9,
                           "decode": dec_bytes / (ms["dec"] / 1e3) / 1e9,
                           "attention": att_bytes / (ms["att"] / 1e3) / 1e9},
        "roofline": {"kernel": "encode_h16<k=4> (fq_encode, fp16 input)", "bound": "alu", "achieved": achieved,
                     "peak": CMP_PEAK_T, "unit": "TFLOP/s", "frac": achieved / CMP_PEAK_T,
                     "traffic": traffic,
                     "work": f"{cmp_per_vec} candidate-score comparisons per vector ((d/k) N) x {n} vectors; "
                             f"peak = 2 comparisons per VALU lane-op (three-input min) x 39.3 T lane-ops/s",
                     # the same time against the VALU-search model (k/2 + 1 lane-ops per score: packed
                     # FMAs plus a select), for comparison with designs that score on the VALU
                     "frac_vs_valu_search_model": cmp_per_vec * (w.k / 2 + 1) * n / VALU_LANE_OPS / enc_s},
    }

    # ---------------------------------------------------------------- decode-attention workload
    if not args.no_attn_workload:
        B, Hq, Hkv, Ta = workloads.ATTN_B, workloads.ATTN_HQ, workloads.ATTN_HKV, workloads.ATTN_T
        qa_np, kv_np = workloads.attention_inputs()
        kv = torch.from_numpy(kv_np.reshape(-1, D)).to(dev)
        na = B * Hkv * Ta
        ac = torch.empty(2 * cb.code_bytes(na), dtype=torch.uint8, device=dev)
        an = torch.empty(2 * na, dtype=torch.float16, device=dev)
        fq.fq_encode(cb.handle, kv, ac, an, stream)
        del kv
        qa = torch.from_numpy(qa_np).to(dev)
        ao = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        aws = torch.empty(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, Ta), dtype=torch.uint8, device=dev)
        kcs, vcs = ac[: cb.code_bytes(na)], ac[cb.code_bytes(na):]
        kns, vns = an[:na], an[na:]
        # Eviction between launches READS a 512 MiB buffer, leaving L2 and the 256 MB
        # last-level cache full of clean lines of it; a write-based fill would leave
        # dirty lines whose write-back lands inside the timed launch.
        flush = torch.ones(128 * 1024 * 1024, dtype=torch.int32, device=dev)
        times = []
        for it in range(args.attn_iters + 3):
            flush.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fq.fq_attn_decode(cb.handle, qa, kcs, kns, vcs, vns, B, Hq, Hkv, Ta, 0.125, ao, aws, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if it >= 3:
                times.append(e0.elapsed_time(e1))
        t_att = float(np.median(times)) / 1e3
        abytes = 2 * cb.code_bytes(na) + 2 * na * 2 + B * Hq * D * 2 + B * Hq * D * 4
        line["attn_b16_t32k"] = {
            "workload": "B=16, Hq=32, Hkv=4, T=32768, k=4, N=256 codes + fp16 norms, caches evicted (512 MiB read) "
                        "before every launch",
            "us_per_step": t_att * 1e6, "hbm_bytes": abytes, "GBps": abytes / t_att / 1e9,
            "fp16_equiv_GBps": 2 * na * D * 2 / t_att / 1e9,
            "roofline": {"kernel": "attn_k4b8 (+ attn_combine: the events bracket the whole fq_attn_decode call)",
                         "bound": "hbm", "achieved": abytes / t_att / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": abytes / t_att / 1e9 / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("attn_k4b8", "fq_attn.hip")},
        }

        # ------------------------------------------------------------ prefill over the same cache
        # 64 causal queries per head (a 64-token chunk appended to the 32k cache): useful
        # work 4 * 64 flops per (query, visible key) pair (QK and PV); the kernel issues
        # 1.5x that on the matrix core (the query enters as fp16 hi + lo).
        if not args.no_prefill:
            Sq = 64
            qp = torch.from_numpy(np.random.default_rng(107).standard_normal((B, Hq, Sq, D)).astype(np.float16)).to(dev)
            po = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device=dev)
            pws = torch.empty(fq.fq_attn_prefill_workspace_bytes(cb.handle, B, Hq, Hkv, Sq, Ta), dtype=torch.uint8,
                              device=dev)
            flush = torch.ones(128 * 1024 * 1024, dtype=torch.int32, device=dev)
            tp = []
            for it in range(args.attn_iters + 3):
                flush.max()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fq.fq_attn_prefill(cb.handle, qp, kcs, kns, vcs, vns, B, Hq, Hkv, Sq, Ta, True, 0.125, po, pws,
                                   stream)
                e1.record(stream)
                torch.cuda.synchronize()
                if it >= 3:
                    tp.append(e0.elapsed_time(e1))
            t_p = float(np.median(tp)) / 1e3
            pairs = B * Hq * sum(Ta - Sq + i + 1 for i in range(Sq))
            useful = 4.0 * D * pairs
            line["prefill_b16_t32k_q64"] = {
                "workload": "B=16, Hq=32, Hkv=4, T=32768, 64 causal queries per head (the last 64 positions), "
                            "k=4, N=256 codes + fp16 norms, caches evicted before every launch",
                "us_per_step": t_p * 1e6, "query_key_pairs": pairs,
                "roofline": {"kernel": "attn_prefill_k4b8 (+ attn_combine)", "bound": "mfma",
                             "achieved": useful / t_p / 1e12, "peak": FP16_MFMA_PEAK_T, "unit": "TFLOP/s",
                             "frac": useful / t_p / 1e12 / FP16_MFMA_PEAK_T, "traffic": None,
                             "issued_TFLOPs": 1.5 * useful / t_p / 1e12},
            }
            del flush

        # ------------------------------------------------------------ decode loop over the same cache
        # One decode step per sequence: the new token's K and V go to slot len_b of their
        # (batch, KV head) slab (fq_encode_scatter), then attention runs over len_b + 1
        # keys (fq_attn_decode_varlen).  Lengths start spread over [T/2, T - iters) and
        # grow by one per step; slots and lengths of every step are on the device
        # before timing, and the caches are evicted before every step.
        if not args.no_decode_loop:
            iters = args.attn_iters
            rng = np.random.default_rng(106)
            len0 = rng.integers(Ta // 2, Ta - iters - 4, size=B)
            base = (np.arange(B)[:, None] * Hkv + np.arange(Hkv)[None, :]) * Ta  # [B, Hkv] slab starts
            # K and V caches are the two halves of one store (records [0, na) and [na, 2 na)),
            # so one call appends both
            slots_all = torch.from_numpy(np.stack([np.concatenate([(base + (len0 + it)[:, None]).reshape(-1)] * 2)
                                                   + np.repeat([0, na], B * Hkv)
                                                   for it in range(iters + 3)]).astype(np.int64)).to(dev)
            lens_all = torch.from_numpy(np.stack([len0 + it + 1 for it in range(iters + 3)]).astype(np.int32)).to(dev)
            newkv = torch.from_numpy(np.ascontiguousarray(kv_np[:, :, :, :iters + 3].transpose(3, 0, 1, 2, 4))
                                     .reshape(iters + 3, 2 * B * Hkv, D)).to(dev)
            flush = torch.ones(128 * 1024 * 1024, dtype=torch.int32, device=dev)
            t_app, t_var = [], []
            for it in range(iters + 3):
                flush.max()
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record(stream)
                fq.fq_encode_scatter(cb.handle, newkv[it], slots_all[it], 2 * na, ac, an, stream)
                e[1].record(stream)
                fq.fq_attn_decode_varlen(cb.handle, qa, kcs, kns, vcs, vns, lens_all[it], B, Hq, Hkv, Ta, 0.125, ao,
                                         aws, stream)
                e[2].record(stream)
                torch.cuda.synchronize()
                if it >= 3:
                    t_app.append(e[0].elapsed_time(e[1]))
                    t_var.append(e[1].elapsed_time(e[2]))
            t_a, t_v = float(np.median(t_app)) / 1e3, float(np.median(t_var)) / 1e3
            # The same step captured once as a HIP graph: every replay reads this step's new
            # vectors, slots and lengths from fixed device buffers, refreshed before replay.
            x_buf, s_buf, l_buf = newkv[0].clone(), slots_all[0].clone(), lens_all[0].clone()
            gs = torch.cuda.Stream()
            gs.wait_stream(stream)
            with torch.cuda.stream(gs):  # warm-up on the capture stream
                fq.fq_encode_scatter(cb.handle, x_buf, s_buf, 2 * na, ac, an, gs)
                fq.fq_attn_decode_varlen(cb.handle, qa, kcs, kns, vcs, vns, l_buf, B, Hq, Hkv, Ta, 0.125, ao, aws, gs)
            stream.wait_stream(gs)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                cs = torch.cuda.current_stream()
                fq.fq_encode_scatter(cb.handle, x_buf, s_buf, 2 * na, ac, an, cs)
                fq.fq_attn_decode_varlen(cb.handle, qa, kcs, kns, vcs, vns, l_buf, B, Hq, Hkv, Ta, 0.125, ao, aws, cs)
            t_graph = []
            for it in range(iters + 3):
                x_buf.copy_(newkv[it])
                s_buf.copy_(slots_all[it])
                l_buf.copy_(lens_all[it])
                flush.max()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                if it >= 3:
                    t_graph.append(e0.elapsed_time(e1))
            t_g = float(np.median(t_graph)) / 1e3
            del graph
            keys = int(lens_all[3:].sum().item()) * Hkv / iters  # keys read per step, all slabs
            vbytes = keys * (16 + 16 + 2 + 2) + B * Hq * D * 2 + B * Hq * D * 4
            line["decode_loop_b16_t32k"] = {
                "workload": "B=16, Hq=32, Hkv=4, cache capacity T=32768, per-batch lengths uniform in [T/2, T); per "
                            "step: 64 new K and 64 new V vectors encoded into their slots (one call), then attention "
                            "over each "
                            "batch's valid keys; caches evicted before every step",
                "us_per_step": (t_a + t_v) * 1e6, "breakdown_us": {"append": t_a * 1e6, "attention": t_v * 1e6},
                "us_per_step_graph": t_g * 1e6,
                "keys_per_step": keys, "hbm_bytes_attention": vbytes,
                "roofline": {"kernel": "attn_k4b8 with per-batch lengths (+ attn_combine)", "bound": "hbm",
                             "achieved": vbytes / t_v / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": vbytes / t_v / 1e9 / HBM_PEAK_GBPS, "traffic": None},
            }
            del flush

    if not args.no_workloads:
        line["workloads"] = workload_timings(fq, workloads, dev, stream)
    if not args.no_rate_axis:
        line["rate_axis"] = rate_axis_timings(fq, workloads, dev, stream)
    if not args.no_build:
        line["codebook_build"] = build_timings(fq, workloads, dev, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    cb.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
