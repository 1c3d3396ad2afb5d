#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet hot path on one MI355X.

Headline (the decode leg): one step = one gdn_decode launch over B=256
single-token sequences (Hk=16, Hv=32, Dk=Dv=128, bf16 q/k/v/out, gate and
q/k L2-norm fused) updating fp32 states in place in a 1024-slot pool.  Launches
rotate over four disjoint 256-slot subsets of the pool, so every launch reads
and writes 512 MiB of state that the previous three launches did not touch.
value = algorithmic bytes per step / time per step, in GB/s.

Second leg (same JSON line, "prefill"): gdn_gate + gdn_prefill_varlen over 8
sequences with lengths U(1,8192) summing to 32768 tokens (Hk=8, Hv=24, D=128,
fp16, initial states from a 64-slot pool), reported in tokens/s; and
("prefill_t4096") the same over one sequence of 4096 tokens (Hk=16, Hv=32,
bf16, zero initial state).

Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  The CPU oracle is timed on the host's cores (a thread per
independent (sequence, v-head) unit, whole workloads) as a baseline, not a
target.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
METRIC = "GDN decode state GB/s (% HBM peak) @B=256; varlen prefill tokens/s"
PREFILL_WARM_S = 0.3           # least warm-up of the prefill legs, in seconds of calls


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(B, hk, hv, dk, dv, in_bytes, out_bytes, alpha_bytes=4, state_bytes=4):
    """Algorithmic HBM bytes of one decode step: the state is read and written
    once per live (row, v-head); q/k once per (row, q/k head); v and out once;
    alpha, beta per (row, v-head); dt_bias, ssm_a per v-head; the slot index."""
    state = 2 * B * hv * dv * dk * state_bytes
    qk = 2 * B * hk * dk * in_bytes
    vo = B * hv * dv * (in_bytes + out_bytes)
    gate = B * hv * (alpha_bytes + 4) + 2 * hv * 4 + B * 4
    return state + qk + vo + gate


DECODE_SOURCES = ("linear_attention_recurrence_gdn_amd/csrc/gdn_recurrent.hip",
                  "linear_attention_recurrence_gdn_amd/csrc/gdn_device.h")
TRAFFIC_PROFILE = "profiles/decode_B256_hbm_traffic.md"


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed PMC summary (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy's counters), or None when the summary is
    missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":", 1)[0].strip() in (
                    "source_sha256", "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                v = v.split()
                fields[k.strip()] = v[0].strip("`") if v else ""
    if fields.get("source_sha256") != decode_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


PREFILL_SOURCES = ("linear_attention_recurrence_gdn_amd/csrc/gdn_chunked.hip",
                   "linear_attention_recurrence_gdn_amd/csrc/gdn_prefill_gate.h",
                   "linear_attention_recurrence_gdn_amd/csrc/gdn_launch.h",
                   "linear_attention_recurrence_gdn_amd/csrc/gdn_device.h")
WALK_COUNTERS_PROFILE = "profiles/prefill_varlen8_walk_sq_counters.md"


def prefill_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in PREFILL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def walk_mfma_busy():
    """MFMA busy fraction of the varlen walk on the SIMDs it occupies, from the
    committed SQ counter summary, or None when it is missing or was taken on
    different kernel sources."""
    path = os.path.join(ROOT, WALK_COUNTERS_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":", 1)[0].strip() in (
                    "source_sha256", "walk_mfma_busy_frac"):
                k, v = line.split(":", 1)
                v = v.split()
                fields[k.strip()] = v[0].strip("`") if v else ""
    if fields.get("source_sha256") != prefill_source_hash():
        return None
    try:
        return float(fields["walk_mfma_busy_frac"])
    except (KeyError, ValueError):
        return None


def prefill_bytes(T, N, hk, hv, dk, dv, in_bytes, out_bytes, n_init=None):
    """Algorithmic HBM bytes of the varlen prefill with the gate fused: q/k/v
    read once, out written once, alpha (f32) and beta read once per (token,
    v-head), the initial state of each of the n_init sequences that have one
    read once and every final state written once."""
    n_init = N if n_init is None else n_init
    qkv = T * (2 * hk * dk + hv * dv) * in_bytes
    out = T * hv * dv * out_bytes
    gate = T * hv * 4 * 2          # alpha and beta read
    state = (n_init + N) * hv * dv * dk * 4
    return qkv + out + gate + state


def prefill_flops(T, hv, dk, dv, C=64):
    """Flops of the chunked form per (token, v-head) at chunk size C:
    2 [C (3 Dk + 2 Dv) + 3 Dk Dv + C^2 / 6]."""
    return 2.0 * T * hv * (C * (3 * dk + 2 * dv) + 3 * dk * dv + C * C / 6.0)


def schedule_of(ws, N, lengths):
    """The schedule a chunked prefill call chose, from the per-call metadata it
    leaves at the front of its workspace: int32 cs[N+1], order[N], ocs[N+1],
    then the split rank k, the number of split sequences ks, their segment
    count S and segment lengths (chunks)."""
    import torch
    words = ws[:4 * (3 * N + 7)].view(torch.int32).cpu().numpy()
    k, ks, S = (int(x) for x in words[3 * N + 2:3 * N + 5])
    order = [int(x) for x in words[N + 1:2 * N + 1]]
    return {
        "split_rank": k,
        "walked_early": [lengths[s] for s in order[:k]],
        "split_sequences": [lengths[s] for s in order[:ks]],
        "segments": S if ks else 1,
        "note": "the records of the k longest sequences are formed first and their walks "
                "start at once, the other sequences' records and walks beside them on a second "
                "stream; each split sequence is walked in S segments: first its segment-0 "
                "state and each middle segment's local state and transition, then every "
                "segment with outputs from its exact entry state",
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of each CPU-oracle baseline leg")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-t4096", action="store_true",
                    help="skip the single-sequence T=4096 prefill leg")
    ap.add_argument("--no-state16", action="store_true",
                    help="skip the decode leg with a bf16 state pool")
    ap.add_argument("--no-norm", action="store_true",
                    help="skip the gated-RMSNorm legs (fused decode, norm after prefill)")
    ap.add_argument("--no-conv", action="store_true", help="skip the conv1d legs")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the B=1024 packed decode over the 4096-slot pool")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scale factor for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--only", default="",
                    help="comma list of legs to time (profiling runs): decode, decode_bf16, "
                         "decode_norm, decode_b1024, conv_update, prefill, t4096, conv_fwd, "
                         "post_conv, rmsnorm, prefill_norm, cpu; default all")
    args = ap.parse_args()
    only = {x for x in args.only.split(",") if x}

    def want(leg):
        return not only or leg in only
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.exit("bench.py: one GPU only (the decode and prefill kernels "
                 "shard by sequence with no exchange); run with --gpus 1")

    import torch
    import workloads as W
    import linear_attention_recurrence_gdn_amd as gdn

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 28
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n,
                                               "launches": 5}}), flush=True)
        return
    t_setup = time.time()

    # ---------------- decode leg ----------------
    case = W.decode_b256()
    B, hk, hv, dk, dv = case.batch, case.hk, case.hv, case.dk, case.dv
    to_dev = lambda a: torch.from_numpy(a).to(dev)
    qb = to_dev(case.q.buf.view(np.int16)).view(torch.bfloat16).view(B, hk, dk)
    kb = to_dev(case.k.buf.view(np.int16)).view(torch.bfloat16).view(B, hk, dk)
    vb = to_dev(case.v.buf.view(np.int16)).view(torch.bfloat16).view(B, hv, dv)
    alpha, dt_bias, ssm_a, beta = (to_dev(case.alpha), to_dev(case.dt_bias),
                                   to_dev(case.ssm_a), to_dev(case.beta))
    pool = to_dev(case.pool)
    perm = np.random.default_rng([202, 0xB]).permutation(case.num_slots).astype(np.int32)
    subsets = [to_dev(np.ascontiguousarray(perm[i * B:(i + 1) * B])) for i in range(4)]
    out = torch.empty((B, hv, dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"decode setup {time.time() - t_setup:.1f}s")

    def timed(step, warmup, steps, warm_s=0.0):
        """Wall seconds over `steps` launches after `warmup` (the timed region:
        nothing but the launches between two synchronisations), then each
        launch's duration (ms) from HIP events recorded on the launch stream
        around `steps` further launches.  The events are kept out of the wall
        region because their markers add a gap between launches.  warm_s
        extends the warm-up to at least that many seconds of launches: after
        the host has prepared a leg's inputs the GPU's clocks take a few tens
        of calls of the compute-bound prefill to come back up (the first 20
        calls after an idle second run about 10 % slower), while the
        memory-bound decode shows no such ramp."""
        n = 0
        t_w = time.perf_counter()
        while n < warmup or time.perf_counter() - t_w < warm_s:
            step(n)
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(n + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            step(n + steps + i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return wall, np.array([a.elapsed_time(b) for a, b in ev])

    def decode_step(i):
        gdn.decode(qb, kb, vb, alpha, dt_bias, ssm_a, beta, pool, subsets[i % 4],
                   scale=case.scale, out=out, stream=stream)

    step_bytes = decode_bytes(B, hk, hv, dk, dv, 2, 2)
    if want("decode"):
        wall, kernel_ms = timed(decode_step, args.warmup, args.steps)
    else:   # a profiling run of other legs only: the headline is not measured
        wall, kernel_ms = float("nan"), np.array([float("nan")])
    ms_per_step = wall * 1e3 / args.steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    kavg = float(kernel_ms.mean())
    k_gbs = step_bytes / (kavg * 1e-3) / 1e9
    log(f"decode: {ms_per_step * 1e3:.1f} us/step wall, kernel avg {kavg * 1e3:.1f} us "
        f"(min {kernel_ms.min() * 1e3:.1f}, median {np.median(kernel_ms) * 1e3:.1f}) "
        f"-> {k_gbs:.0f} GB/s = {k_gbs / HBM_PEAK_GBS * 100:.1f}% of peak")

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode B=256 x 1 token, Hk=16, Hv=32, Dk=Dv=128, bf16 q/k/v/out, "
                        "fp32 state pool of 1024 slots (4 rotating 256-slot subsets), gate and "
                        "q/k L2-norm fused",
            "global_batch": B, "seq_len": 1, "parallelism": "none (1 GPU)",
            "algorithmic_bytes_per_step": step_bytes,
            "pct_hbm_peak": round(gbs / HBM_PEAK_GBS * 100, 2),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated)",
            "kernel": "gdn::decode_kernel (Dk=128, 8 state loads/lane, nontemporal)",
            "kernel_avg_us": round(kavg * 1e3, 2),
        },
    }

    # ---------------- decode with the pool stored as bf16 ----------------
    if want("decode_bf16") and not args.no_state16:
        pool16 = to_dev(W.encode(case.pool, W.BF16).view(np.int16)).view(torch.bfloat16)

        def decode16_step(i):
            gdn.decode(qb, kb, vb, alpha, dt_bias, ssm_a, beta, pool16, subsets[i % 4],
                       scale=case.scale, out=out, stream=stream)

        wall16, k16 = timed(decode16_step, args.warmup, args.steps)
        bytes16 = decode_bytes(B, hk, hv, dk, dv, 2, 2, state_bytes=2)
        ms16 = wall16 * 1e3 / args.steps
        kavg16 = float(k16.mean())
        result["decode_state_bf16"] = {
            "workload": "the same decode with the 1024-slot state pool stored as bf16 "
                        "(widened to f32 for the step, rounded on store)",
            "ms_per_step": round(ms16, 5),
            "tokens_per_s": round(B / (ms16 * 1e-3), 1),
            "algorithmic_bytes_per_step": bytes16,
            "kernel_avg_us": round(kavg16 * 1e3, 2),
            "achieved_GBs": round(bytes16 / (kavg16 * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes16 / (kavg16 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "speedup_vs_f32_state": round(kavg / kavg16, 3),
        }
        del pool16
        log(f"decode bf16 state: kernel avg {kavg16 * 1e3:.1f} us -> "
            f"{bytes16 / (kavg16 * 1e-3) / 1e9:.0f} GB/s")

    # ---------------- decode with the gated RMSNorm fused ----------------
    if want("decode_norm") and not args.no_norm:
        nrm = W.norm_inputs(202, B, hv, dv, W.BF16)
        zb = to_dev(nrm.z.buf.view(np.int16)).view(torch.bfloat16).view(B, hv, dv)
        wb = to_dev(nrm.w.view(np.int16)).view(torch.bfloat16)

        def decode_norm_step(i):
            gdn.decode_gated_norm(qb, kb, vb, alpha, dt_bias, ssm_a, beta, pool, subsets[i % 4],
                                  zb, wb, scale=case.scale, norm_eps=nrm.eps, out=out,
                                  stream=stream)

        wall_n, kn = timed(decode_norm_step, args.warmup, args.steps)
        bytes_n = step_bytes + B * hv * dv * 2 + dv * 2
        kavg_n = float(kn.mean())
        result["decode_gated_norm"] = {
            "workload": "the same decode with the gated RMSNorm (silu gate, bf16 z and w) "
                        "fused into the output store",
            "ms_per_step": round(wall_n * 1e3 / args.steps, 5),
            "algorithmic_bytes_per_step": bytes_n,
            "kernel_avg_us": round(kavg_n * 1e3, 2),
            "achieved_GBs": round(bytes_n / (kavg_n * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes_n / (kavg_n * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "overhead_vs_plain_decode": round(kavg_n / kavg - 1.0, 4),
        }
        log(f"decode + gated norm: kernel avg {kavg_n * 1e3:.1f} us")

    # ---------------- large decode from row-strided packed input ----------------
    if want("decode_b1024") and not args.no_large:
        big = W.decode_packed_b1024(with_pool=False)
        B5, hk5, hv5, dk5, dv5 = big.batch, big.hk, big.hv, big.dk, big.dv
        slots5 = 4096
        pbuf = to_dev(np.ascontiguousarray(big.q.buf)).reshape(-1)  # fp16 [B, 8448]
        stride5 = big.q.row_stride
        q5 = pbuf.as_strided((B5, hk5, dk5), (stride5, dk5, 1), big.q.offset)
        k5 = pbuf.as_strided((B5, hk5, dk5), (stride5, dk5, 1), big.k.offset)
        v5 = pbuf.as_strided((B5, hv5, dv5), (stride5, dv5, 1), big.v.offset)
        a5, dt5, sa5, b5 = (to_dev(big.alpha), to_dev(big.dt_bias), to_dev(big.ssm_a),
                            to_dev(big.beta))
        # the 8.6 GB state pool is drawn on the device (same N(0, 0.05^2) recipe, seeded)
        gen5 = torch.Generator(device=dev)
        gen5.manual_seed(505)
        pool5 = torch.empty((slots5, hv5, dv5, dk5), dtype=torch.float32, device=dev)
        pool5.normal_(0.0, 0.05, generator=gen5)
        perm5 = np.random.default_rng([505, 0xB]).permutation(slots5).astype(np.int32)
        subsets5 = [to_dev(np.ascontiguousarray(perm5[i * B5:(i + 1) * B5])) for i in range(4)]
        out5 = torch.empty((B5, hv5, dv5), dtype=torch.float16, device=dev)

        def decode5_step(i):
            gdn.decode(q5, k5, v5, a5, dt5, sa5, b5, pool5, subsets5[i % 4],
                       scale=big.scale, out=out5, stream=stream)

        steps5 = max(4, args.steps // 2)
        wall5, k5ms = timed(decode5_step, max(4, args.warmup // 2), steps5)
        bytes5 = decode_bytes(B5, hk5, hv5, dk5, dv5, 2, 2)
        kavg5 = float(k5ms.mean())
        result["decode_b1024_packed"] = {
            "workload": "decode B=1024 x 1 token from one packed fp16 q|k|v row per sequence "
                        "(row stride 8448, 256 padding columns), Hk=16, Hv=32, Dk=Dv=128, "
                        "fp16 out, fp32 state pool of 4096 slots (4 rotating 1024-slot subsets)",
            "ms_per_step": round(wall5 * 1e3 / steps5, 5),
            "algorithmic_bytes_per_step": bytes5,
            "kernel_avg_us": round(kavg5 * 1e3, 2),
            "kernel_median_us": round(float(np.median(k5ms)) * 1e3, 2),
            "achieved_GBs": round(bytes5 / (kavg5 * 1e-3) / 1e9, 1),
            "hbm_frac": round(bytes5 / (kavg5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        log(f"decode B=1024 packed: kernel avg {kavg5 * 1e3:.1f} us -> "
            f"{bytes5 / (kavg5 * 1e-3) / 1e9:.0f} GB/s")
        del pool5, pbuf, q5, k5, v5

    # ---------------- conv1d update at the decode batch ----------------
    if want("conv_update") and not args.no_conv:
        C, K = 2 * hk * dk + hv * dv, 4
        crng = np.random.default_rng([202, 0xC0])
        ux = to_dev(W.encode(crng.normal(size=(B, C)).astype(np.float32), W.BF16).view(np.int16)
                    ).view(torch.bfloat16)
        uw = to_dev(W.encode(crng.uniform(-1, 1, size=(C, K)), W.BF16).view(np.int16)
                    ).view(torch.bfloat16)
        ust = torch.zeros((case.num_slots, C, K - 1), dtype=torch.bfloat16, device=dev)
        uout = torch.empty_like(ux)

        def conv_upd_step(i):
            gdn.conv1d_update(ux, uw, None, ust, state_idx=subsets[i % 4], out=uout,
                              stream=stream)

        _, uk = timed(conv_upd_step, args.warmup, args.steps)
        ubytes = 2 * B * C * 2 + 2 * B * C * (K - 1) * 2 + C * K * 2 + B * 4
        uavg = float(uk.mean())
        result["conv1d_update"] = {
            "workload": f"conv1d update (K=4, silu) for the B=256 decode batch, {C} bf16 "
                        f"channels, bf16 state rows from the 1024-slot cache",
            "kernel_avg_us": round(uavg * 1e3, 2),
            "algorithmic_bytes": ubytes,
            "achieved_GBs": round(ubytes / (uavg * 1e-3) / 1e9, 1),
            "hbm_frac": round(ubytes / (uavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        log(f"conv1d_update: kernel avg {uavg * 1e3:.1f} us")
        del ust

    # ---------------- prefill leg ----------------
    if not args.no_prefill:
        pre = W.prefill_varlen_gqa3()
        T, N = pre.total_tokens, pre.num_seqs
        qp = to_dev(pre.q.buf).view(T, pre.hk, pre.dk)
        kp = to_dev(pre.k.buf).view(T, pre.hk, pre.dk)
        vp = to_dev(pre.v.buf).view(T, pre.hv, pre.dv)
        pa, pdt, pssm, pbeta = (to_dev(pre.alpha), to_dev(pre.dt_bias), to_dev(pre.ssm_a),
                                to_dev(pre.beta))
        ppool = to_dev(pre.pool)
        pcu, pidx, phi = to_dev(pre.cu_seqlens), to_dev(pre.idx), to_dev(pre.has_init)
        pout = torch.empty((T, pre.hv, pre.dv), dtype=torch.float16, device=dev)
        ws_n = gdn.prefill_workspace_size(T, N, pre.hk, pre.hv, pre.dk, pre.dv, torch.float16)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        aux = torch.cuda.Stream()   # the second stream of the split schedule

        def prefill_step():
            gdn.prefill_varlen_gated(qp, kp, vp, pa, pdt, pssm, pbeta, ppool, pcu,
                                     scale=pre.scale, state_idx=pidx, has_initial_state=phi,
                                     out=pout, workspace=ws, stream=stream, aux_stream=aux)

        if want("prefill"):
            pwall, pms = timed(lambda i: prefill_step(), 8, args.prefill_steps, PREFILL_WARM_S)
            p_ms_step = pwall * 1e3 / args.prefill_steps
            pbytes = prefill_bytes(T, N, pre.hk, pre.hv, pre.dk, pre.dv, 2, 2,
                                   int(pre.has_init.sum()))
            pflops = prefill_flops(T, pre.hv, pre.dk, pre.dv)
            pavg = float(pms.mean())
            result["prefill"] = {
                "workload": "varlen prefill, 8 sequences, lengths U(1,8192) summing to 32768, "
                            "Hk=8, Hv=24 (GQA 3), D=128, fp16 q/k/v/out, fp32 states from a "
                            "64-slot pool; gate fused into the recurrence "
                            "(gdn_prefill_varlen_gated)",
                "lengths": pre.meta["lengths"],
                "tokens_per_s": round(T / (p_ms_step * 1e-3), 1),
                "ms_per_step": round(p_ms_step, 4),
                "kernel_avg_ms": round(pavg, 4),
                "achieved_GBs": round(pbytes / (pavg * 1e-3) / 1e9, 1),
                "hbm_frac": round(pbytes / (pavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "chunked_flops_per_step": pflops,
                "mfma_frac_algorithmic": round(pflops / (pavg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "walk_mfma_busy": walk_mfma_busy(),
                "walk_mfma_busy_source": WALK_COUNTERS_PROFILE + " (SQ_VALU_MFMA_BUSY_CYCLES "
                                         "over the SIMDs the longest walk occupies; null when "
                                         "taken on other kernel sources)",
                "path": "chunked" if ws_n > 0 else "token-sequential",
            }
            if ws_n > 0:
                result["prefill"]["schedule"] = schedule_of(ws, N, pre.meta["lengths"])
            log(f"prefill: {p_ms_step:.3f} ms/step -> {T / (p_ms_step * 1e-3) / 1e6:.2f} M tokens/s")

        # the single long sequence: T=4096, Hk=16, Hv=32, bf16, zero initial state
        if want("t4096") and not args.no_t4096:
            p3 = W.prefill_t4096()
            T3 = p3.total_tokens
            q3 = to_dev(p3.q.buf.view(np.int16)).view(torch.bfloat16).view(T3, p3.hk, p3.dk)
            k3 = to_dev(p3.k.buf.view(np.int16)).view(torch.bfloat16).view(T3, p3.hk, p3.dk)
            v3 = to_dev(p3.v.buf.view(np.int16)).view(torch.bfloat16).view(T3, p3.hv, p3.dv)
            a3, dt3, sa3, b3 = (to_dev(p3.alpha), to_dev(p3.dt_bias), to_dev(p3.ssm_a),
                                to_dev(p3.beta))
            pool3 = to_dev(p3.pool)
            cu3, idx3, hi3 = to_dev(p3.cu_seqlens), to_dev(p3.idx), to_dev(p3.has_init)
            out3 = torch.empty((T3, p3.hv, p3.dv), dtype=torch.bfloat16, device=dev)
            ws3_n = gdn.prefill_workspace_size(T3, 1, p3.hk, p3.hv, p3.dk, p3.dv,
                                               torch.bfloat16)
            ws3 = torch.empty(max(ws3_n, 1), dtype=torch.uint8, device=dev)

            def t4096_step(i):
                gdn.prefill_varlen_gated(q3, k3, v3, a3, dt3, sa3, b3, pool3, cu3,
                                         scale=p3.scale, state_idx=idx3, has_initial_state=hi3,
                                         out=out3, workspace=ws3, stream=stream,
                                         aux_stream=aux)

            w3, k3ms = timed(t4096_step, 8, args.prefill_steps, PREFILL_WARM_S)
            ms3 = w3 * 1e3 / args.prefill_steps
            avg3 = float(k3ms.mean())
            bytes3 = prefill_bytes(T3, 1, p3.hk, p3.hv, p3.dk, p3.dv, 2, 2, 0)
            flops3 = prefill_flops(T3, p3.hv, p3.dk, p3.dv)
            result["prefill_t4096"] = {
                "workload": "single-sequence prefill T=4096, Hk=16, Hv=32, D=128, bf16 q/k/v/out, "
                            "zero initial state (slot never read), fp32 final state; "
                            "gate fused into the recurrence (gdn_prefill_varlen_gated)",
                "tokens_per_s": round(T3 / (ms3 * 1e-3), 1),
                "ms_per_step": round(ms3, 4),
                "kernel_avg_ms": round(avg3, 4),
                "algorithmic_bytes_per_step": bytes3,
                "achieved_GBs": round(bytes3 / (avg3 * 1e-3) / 1e9, 1),
                "hbm_frac": round(bytes3 / (avg3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "chunked_flops_per_step": flops3,
                "mfma_frac_algorithmic": round(flops3 / (avg3 * 1e-3) / 1e12 /
                                               MFMA_BF16_PEAK_TFLOPS, 4),
                "path": "chunked" if ws3_n > 0 else "token-sequential",
                "schedule": schedule_of(ws3, 1, [T3]) if ws3_n > 0 else None,
            }
            log(f"prefill T=4096: {ms3:.3f} ms/step -> {T3 / (ms3 * 1e-3) / 1e6:.2f} M tokens/s")
            del q3, k3, v3, out3, ws3, pool3

        # the causal conv1d before the front-end, over the same tokens
        if want("conv_fwd") and not args.no_conv:
            C, K = 2 * pre.hk * pre.dk + pre.hv * pre.dv, 4
            crng = np.random.default_rng([404, 0xC0])
            cx = to_dev(W.encode(crng.normal(size=(T, C)).astype(np.float32), W.F16))
            cw = to_dev(W.encode(crng.uniform(-1, 1, size=(C, K)), W.F16))
            cst = torch.zeros((64, C, K - 1), dtype=torch.float16, device=dev)
            cout = torch.empty_like(cx)

            def conv_step(i):
                gdn.conv1d_fwd(cx, cw, None, cst, pcu, state_idx=pidx, has_initial_state=phi,
                               out=cout, stream=stream)

            cwall, ck = timed(conv_step, 3, args.prefill_steps)
            cbytes = 2 * T * C * 2 + 2 * N * C * (K - 1) * 2 + C * K * 2
            cavg = float(ck.mean())
            result.setdefault("prefill", {})["conv1d_fwd"] = {
                "workload": f"depthwise causal conv1d (K=4, silu) over the 32768 packed tokens, "
                            f"{C} fp16 channels (q|k|v), fp16 state from the 64-slot cache",
                "kernel_avg_us": round(cavg * 1e3, 2),
                "algorithmic_bytes": cbytes,
                "achieved_GBs": round(cbytes / (cavg * 1e-3) / 1e9, 1),
                "hbm_frac": round(cbytes / (cavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
            log(f"prefill conv1d_fwd: kernel avg {cavg * 1e3:.1f} us")
            del cx, cout

        # the gated RMSNorm over the prefill output (a separate HBM pass)
        if want("post_conv") and not args.no_conv:
            # the front-end after the conv, materialising q, k (normalised), v, g and beta
            # from the conv rows and one merged fp16 b | a row per token
            C = 2 * pre.hk * pre.dk + pre.hv * pre.dv
            frng = np.random.default_rng([505, 0xC0])
            fx = to_dev(W.encode(frng.uniform(-1.5, 1.5, size=(T, C)), W.F16))
            fba = to_dev(W.encode(frng.uniform(-2, 2, size=(T, 2 * pre.hv)), W.F16))
            fb, fa = fba[:, :pre.hv], fba[:, pre.hv:]

            def post_conv_step(i):
                gdn.post_conv(fx, fa, fb, pdt, pssm, hk=pre.hk, dk=pre.dk, dv=pre.dv,
                              stream=stream)

            _, fk = timed(post_conv_step, 3, args.prefill_steps)
            fbytes = 2 * T * C * 2 + T * pre.hv * (2 * 2 + 2 * 4)
            favg = float(fk.mean())
            result.setdefault("prefill", {})["post_conv"] = {
                "workload": f"post-conv front-end over the 32768 packed tokens: {C} fp16 "
                            f"channels in and out (q, k L2-normalised), g and beta in f32 "
                            f"from a merged fp16 b | a row (two kernels)",
                "kernel_avg_us": round(favg * 1e3, 2),
                "algorithmic_bytes": fbytes,
                "achieved_GBs": round(fbytes / (favg * 1e-3) / 1e9, 1),
                "hbm_frac": round(fbytes / (favg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
            log(f"prefill post_conv: kernel avg {favg * 1e3:.1f} us")
            del fx, fba, fa, fb

        if want("rmsnorm") and not args.no_norm:
            pn = W.norm_inputs(404, T, pre.hv, pre.dv, W.F16)
            pz = to_dev(pn.z.buf).view(T, pre.hv, pre.dv)
            pw = to_dev(pn.w)
            nout = torch.empty_like(pout)

            def norm_step(i):
                gdn.rmsnorm_gated(pout, pz, pw, eps=pn.eps, out=nout, stream=stream)

            nwall, nk = timed(norm_step, 3, args.prefill_steps)
            nbytes = 3 * T * pre.hv * pre.dv * 2 + pre.dv * 2
            navg = float(nk.mean())
            result.setdefault("prefill", {})["rmsnorm_gated"] = {
                "workload": "gated RMSNorm (silu) over the [32768, 24, 128] fp16 prefill output "
                            "with an fp16 gate and weight",
                "kernel_avg_us": round(navg * 1e3, 2),
                "algorithmic_bytes": nbytes,
                "achieved_GBs": round(nbytes / (navg * 1e-3) / 1e9, 1),
                "hbm_frac": round(nbytes / (navg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
            log(f"prefill gated norm: kernel avg {navg * 1e3:.1f} us")

        if want("prefill_norm") and not args.no_norm:
            gn = W.norm_inputs(404, T, pre.hv, pre.dv, W.F16)
            gz = to_dev(gn.z.buf).view(T, pre.hv, pre.dv)
            gw = to_dev(gn.w)

            def prefill_norm_step(i):
                gdn.prefill_varlen_gated_norm(qp, kp, vp, pa, pdt, pssm, pbeta, ppool, pcu, gz,
                                              gw, scale=pre.scale, norm_eps=gn.eps,
                                              state_idx=pidx, has_initial_state=phi, out=pout,
                                              workspace=ws, stream=stream, aux_stream=aux)

            gwall, gk = timed(prefill_norm_step, 4, args.prefill_steps, PREFILL_WARM_S)
            g_ms = gwall * 1e3 / args.prefill_steps
            result.setdefault("prefill", {})["with_gated_norm"] = {
                "workload": "the same varlen prefill followed by the gated RMSNorm (silu, fp16 "
                            "gate and weight) over its output in place, one call "
                            "(gdn_prefill_varlen_gated_norm: the walks, then the norm pass)",
                "ms_per_step": round(g_ms, 4),
                "tokens_per_s": round(T / (g_ms * 1e-3), 1),
                "kernel_avg_ms": round(float(gk.mean()), 4),
            }
            log(f"prefill + gated norm: {g_ms:.3f} ms/step -> "
                f"{T / (g_ms * 1e-3) / 1e6:.2f} M tokens/s")
            del gz, gw

    # ---------------- CPU oracle baseline ----------------
    if want("cpu") and not args.no_cpu:
        import oracle
        nthr = oracle.default_threads()
        oracle.set_threads(nthr)
        model, host_cpus = cpu_model(), os.cpu_count()
        where = (f"{nthr} threads over independent (sequence, v-head) units on {model} "
                 f"({host_cpus} logical CPUs on the host)")
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.decode_case(case)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        cpu_t = time.perf_counter() - t0
        cpu_gbs = step_bytes * reps / cpu_t / 1e9
        result["cpu_baseline"] = {
            "value": round(cpu_gbs, 4), "unit": "GB/s", "cores": nthr, "kind": "oracle",
            "sample": f"{reps} whole decode step(s) of the B=256 workload (gate + step in f64) "
                      f"in {cpu_t:.1f} s; {where}",
            "cpu_model": model, "host_cpus": host_cpus,
        }
        log(f"cpu oracle decode: {cpu_gbs:.3f} GB/s over {reps} step(s), {nthr} threads")
        if "prefill" in result:
            t0 = time.perf_counter()
            oracle.prefill_case(pre)
            pt = time.perf_counter() - t0
            result["prefill"]["cpu_baseline"] = {
                "value": round(pre.total_tokens / pt, 2), "unit": "tokens/s", "cores": nthr,
                "kind": "oracle",
                "sample": f"the whole varlen workload ({pre.total_tokens} tokens, all "
                          f"{pre.hv} v-heads, gate + recurrence in f64) in {pt:.1f} s; {where}",
            }
            log(f"cpu oracle prefill: {pre.total_tokens / pt:.1f} tokens/s")
            if "prefill_t4096" in result:
                p3 = W.prefill_t4096()
                t0 = time.perf_counter()
                oracle.prefill_case(p3)
                pt3 = time.perf_counter() - t0
                result["prefill_t4096"]["cpu_baseline"] = {
                    "value": round(p3.total_tokens / pt3, 2), "unit": "tokens/s",
                    "cores": nthr, "kind": "oracle",
                    "sample": f"the whole T=4096 workload (all {p3.hv} v-heads) in "
                              f"{pt3:.1f} s; {where}",
                }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
