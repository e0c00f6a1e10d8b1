"""Benchmark of the attention hot path on one MI355X.

One step = one causal MHA prefill (B=2, Hq=Hkv=32, Sq=Sk=4096, d=128, bf16 out)
followed by one paged GQA decode (64 sequences, Hq=64, Hkv=8, d=128, lengths
U{1024..32768}, 64-token blocks placed by a random block table: split kernel +
combine). Inputs are seeded synthetic tensors resident in HBM before timing.

The JSON line's `value` is prefill TFLOP/s (algorithmic flops: only the
visible causal pairs, 4*d flops each), timed with HIP events on the stream the
kernels run on; the decode half of the metric (algorithmic KV bytes per
second) is in `decode`. Other workloads (GQA d=256 with and without
causal+softcap+sinks, single-head d=16) are timed after the step loop and
reported under `other`. `cpu_baseline` times the fp64 CPU oracle on a bounded
sample of the prefill workload.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--no-other] [--gpus 1]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "prefill attention TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"

# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE passes (read counter
# scaled x2, write x1 against a 1 GiB plain copy; see profiles/hbm_traffic_bench.md), valid
# only while the kernel sources hash to the values they were measured on.
MEASURED_TRAFFIC = {
    "prefill_c2": {"sources": ("prefill.hip", "attn_device.hpp", "../build.py"), "sha256_16": "0faed732a068c308", "bytes": 653849049},
    "decode_c4": {"sources": ("decode.hip", "attn_device.hpp", "../build.py"), "sha256_16": "4ca49410d0a34b75", "bytes": 5035204832},
    "decode_c5": {"sources": ("decode.hip", "attn_device.hpp", "../build.py"), "sha256_16": "4ca49410d0a34b75", "bytes": 123606018},
}


def measured_traffic(key):
    """The recorded traffic if the kernel sources and build options (build.py) are unchanged
    since the counters were taken."""
    import hashlib
    e = MEASURED_TRAFFIC[key]
    m = hashlib.sha256()
    for f in e["sources"]:
        with open(os.path.join(ROOT, "attention_flash_attn_amd", "csrc", f), "rb") as fh:
            m.update(fh.read())
    return e["bytes"] if m.hexdigest()[:16] == e["sha256_16"] else None


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def prefill_flops(c):
    """Algorithmic flops: 2*(dk+dv) per visible (query, key) pair."""
    B, Sq, Sk, Hq = c["B"], c["Sq"], c["Sk"], c["Hq"]
    if c["causal"]:
        shift = Sk - Sq
        pairs = sum(max(0, min(Sk, i + shift + 1)) for i in range(Sq))
    else:
        pairs = Sq * Sk
    return 2.0 * (c["dk"] + c["dv"]) * pairs * B * Hq


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=0.2,
                    help="seconds of untimed steps run before the warm-up steps, so the GPU clock reaches its "
                         "steady state whatever --warmup is (0 = none); reported as settle_s")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-other", action="store_true", help="skip the extra workloads")
    ap.add_argument("--cpu-heads", type=int, default=64, help="(batch, head) pairs in the CPU sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (a plain copy kernel of known size, "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (the kernels would shard "
              "over (batch, KV head) with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from attention_flash_attn_amd import binding, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---------------- inputs (seeded, synthetic), resident in HBM
    c2 = synth.CONFIGS["c2_causal_mha_d128"]
    log("generating prefill inputs")
    pc = synth.prefill_case(c2["seed"], c2["B"], c2["Sq"], c2["Sk"], c2["Hq"], c2["Hkv"], c2["dk"], c2["dv"],
                            std=c2["std"])
    q2, k2, v2 = to_dev(pc["q"]), to_dev(pc["k"]), to_dev(pc["v"])
    o2 = torch.empty((c2["B"], c2["Sq"], c2["Hq"], c2["dv"]), device=dev, dtype=torch.bfloat16)
    del pc

    c4 = synth.CONFIGS["c4_paged_gqa_decode"]
    log("generating paged decode inputs")
    dc = synth.paged_case(c4["seed"], c4["B"], c4["Hq"], c4["Hkv"], c4["dk"], c4["dv"], c4["len_lo"],
                          c4["len_hi"], block_size=c4["block_size"])
    lens_host = dc["seq_lens"].astype(np.int64)
    q4 = to_dev(dc["q"])
    kc4, vc4 = to_dev(dc["k_cache"]), to_dev(dc["v_cache"])
    table4 = torch.from_numpy(dc["block_table"]).to(dev)
    lens4 = torch.from_numpy(dc["seq_lens"]).to(dev)
    del dc
    o4 = torch.empty((c4["B"], 1, c4["Hq"], c4["dv"]), device=dev, dtype=torch.bfloat16)
    ws_bytes = binding.attn_decode_workspace_bytes(c4["B"], c4["Hq"], c4["Hkv"], 1, c4["len_hi"], c4["dk"],
                                                   c4["dv"])
    ws4 = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)

    flops2 = prefill_flops(c2)
    kv_bytes4 = float(lens_host.sum()) * c4["Hkv"] * (c4["dk"] + c4["dv"]) * 2
    io_bytes4 = (q4.numel() + o4.numel()) * 2 + table4.numel() * 4 + lens4.numel() * 4
    bytes4 = kv_bytes4 + io_bytes4

    def prefill():
        binding.attn_prefill_fwd(q2, k2, v2, o2, None, scale=c2["scale"], causal=True)

    def decode():
        binding.attn_decode_fwd(q4, kc4, vc4, o4, ws4, scale=c4["scale"], Sk_max=c4["len_hi"],
                                block_table=table4, seq_lens=lens4)

    stream = torch.cuda.current_stream()
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB in %.1f us (%.0f GB/s read+write)" %
            (c0.elapsed_time(c1) * 1e3, 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9))
        del src, dst
    # clock settle: under this load the GPU clock needs ~0.1 s to reach its steady state, longer
    # than a few warm-up steps take, so full steps run untimed for a fixed time first
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(10):
            prefill()
            decode()
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pre = [ev[i][0].elapsed_time(ev[i][1]) * 1e-3 for i in range(K)]
    t_dec = [ev[i][1].elapsed_time(ev[i][2]) * 1e-3 for i in range(K)]
    avg_pre = sum(t_pre) / K
    avg_dec = sum(t_dec) / K
    tflops = flops2 / avg_pre / 1e12
    dec_gbs = bytes4 / avg_dec / 1e9
    log("prefill c2: %.1f us/launch, %.1f TFLOP/s (%.1f%% of peak)" % (avg_pre * 1e6, tflops,
                                                                        100 * tflops / PEAK_BF16_TFLOPS))
    # the same prefill launched back to back (no decode in between): sustained MFMA load
    # lowers the clock, so this is reported beside the in-step figure
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        prefill()
    e1.record(stream)
    torch.cuda.synchronize()
    t_b2b = e0.elapsed_time(e1) * 1e-3 / K
    log("prefill c2 back to back: %.1f us/launch, %.1f TFLOP/s" % (t_b2b * 1e6, flops2 / t_b2b / 1e12))
    log("decode c4: %.1f us/call, %.1f GB/s (%.1f%% of peak)" % (avg_dec * 1e6, dec_gbs, 100 * dec_gbs / PEAK_HBM_GBS))

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_s": round(settle_s, 3),
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal MHA prefill B=2 Hq=Hkv=32 Sq=Sk=4096 dk=dv=128 bf16 out (value) + paged GQA "
                        "decode B=64 Hq=64 Hkv=8 d=128 lengths U{1024..32768} 64-token blocks (decode)",
            "prefill_flops_per_launch": flops2,
            "decode_kv_bytes_per_call": bytes4,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "prefill_kernel<128,128,64,8,2,causal,bf16 out>",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill_c2"),
            "avg_launch_us": round(avg_pre * 1e6, 2),
            "back_to_back_TFLOP/s": round(flops2 / t_b2b / 1e12, 2),
            "back_to_back_us": round(t_b2b * 1e6, 2),
        },
        "decode": {
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "us_per_call": round(avg_dec * 1e6, 2),
            "roofline": {"kernel": "decode_paged_split_kernel<128,128> + decode_combine_kernel", "bound": "hbm",
                         "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode_c4")},
        },
    }

    # ---------------- gathered-row decode (MLA shape), timed cold: 8 copies of the row
    # cache rotate so the selected rows (37.7 MB per call) cannot stay in the 256 MB MALL
    c5 = synth.CONFIGS["c5_gathered_mla_decode"]
    log("generating gathered decode inputs")
    gc = synth.gathered_case(c5["seed"], c5["T"], c5["Hq"], c5["dk"], c5["dv"], c5["n_rows"], c5["n_sel"],
                             row_dim=c5["row_dim"])
    ncopy = 8
    kv5 = [to_dev(gc["kv"]) for _ in range(ncopy)]
    q5 = to_dev(gc["q"]).view(c5["T"], 1, c5["Hq"], c5["dk"])
    ri5 = torch.from_numpy(gc["row_index"]).to(dev)
    kp5 = torch.from_numpy(gc["key_pos"]).to(dev)
    qp5 = torch.from_numpy(gc["q_pos"]).to(dev)
    o5 = torch.empty((c5["T"], 1, c5["Hq"], c5["dv"]), device=dev, dtype=torch.bfloat16)
    ws5 = torch.empty(binding.attn_decode_workspace_bytes(c5["T"], c5["Hq"], 1, 1, c5["n_sel"], c5["dk"], c5["dv"]),
                      device=dev, dtype=torch.uint8)
    bytes5 = (c5["T"] * c5["n_sel"] * c5["row_dim"] * 2 + ri5.numel() * 4 + kp5.numel() * 4 + qp5.numel() * 4 +
              q5.numel() * 2 + o5.numel() * 2)
    flops5 = 2.0 * c5["T"] * c5["Hq"] * c5["n_sel"] * (c5["dk"] + c5["dv"])

    def gathered(i):
        kv = kv5[i % ncopy]
        binding.attn_decode_fwd(q5, kv[:, :c5["dk"]], kv[:, :c5["dv"]], o5, ws5, scale=c5["scale"],
                                Sk_max=c5["n_sel"], causal=True, row_index=ri5, key_pos=kp5, q_pos=qp5)
    for i in range(ncopy):
        gathered(i)
    reps = 8 * ncopy
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        gathered(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t5 = e0.elapsed_time(e1) * 1e-3 / reps
    log("gathered decode c5: %.2f us/call, %.1f GB/s (%.1f%% of HBM peak), %.1f TFLOP/s" %
        (t5 * 1e6, bytes5 / t5 / 1e9, 100 * bytes5 / t5 / 1e9 / PEAK_HBM_GBS, flops5 / t5 / 1e12))
    result["decode_gathered"] = {
        "workload": "16 tokens x 128 heads, 2048 gathered rows of 576 (key) / first 512 (value), "
                    "65536-row cache in permuted 64-row blocks, causal on position, bf16 out, cold (8 rotated "
                    "cache copies)",
        "value": round(bytes5 / t5 / 1e9, 1), "unit": "GB/s", "us_per_call": round(t5 * 1e6, 2),
        "bytes_per_call": bytes5, "flops_per_call": flops5,
        "roofline": {"kernel": "decode_gathered_split_kernel<576,512,4> + decode_combine_kernel", "bound": "hbm",
                     "achieved": round(bytes5 / t5 / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(bytes5 / t5 / 1e9 / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode_c5"),
                     "mfma_frac": round(flops5 / t5 / 1e12 / PEAK_BF16_TFLOPS, 4)},
    }
    del kv5, gc

    # ---------------- other workloads (own timing, after the step loop)
    if not args.no_other:
        other = {}
        for name in ("c3a_gqa_d256", "c3b_gqa_d256_causal_softcap", "c1_single_head_d16"):
            c = synth.CONFIGS[name]
            log("generating %s" % name)
            cc = synth.prefill_case(c["seed"], c["B"], c["Sq"], c["Sk"], c["Hq"], c["Hkv"], c["dk"], c["dv"],
                                    std=c["std"], sinks=c["sinks"])
            q, k, v = to_dev(cc["q"]), to_dev(cc["k"]), to_dev(cc["v"])
            sk = torch.from_numpy(cc["sinks"]).to(dev) if cc["sinks"] is not None else None
            o = torch.empty((c["B"], c["Sq"], c["Hq"], c["dv"]), device=dev,
                            dtype=torch.float32 if c["o_dtype"] == "f32" else torch.bfloat16)

            def run(q=q, k=k, v=v, o=o, sk=sk, c=c):
                binding.attn_prefill_fwd(q, k, v, o, None, scale=c["scale"], causal=c["causal"],
                                         softcap=c["softcap"], sinks=sk)
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.1:  # at least 100 ms of warm work: steady clocks
                run()
                torch.cuda.synchronize()
            reps = 50
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / reps
            f = prefill_flops(c)
            other[name] = {"us": round(t * 1e6, 2), "TFLOP/s": round(f / t / 1e12, 2),
                           "frac_bf16_peak": round(f / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
            log("%s: %.1f us, %.1f TFLOP/s" % (name, t * 1e6, f / t / 1e12))
            del q, k, v, o, cc
        result["other"] = other

        # the widened operations at the same workload shapes (own timing)
        def timed(fn, reps=10):
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.025:  # at least 25 ms of warm work: steady clocks
                fn()
                torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            z.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(z) * 1e-3 / reps

        variants = {}
        log("variants: ALiBi mask, fp16 K/V, multi-token decode, q8_0 pre-pass")
        mask2 = torch.from_numpy(synth.mask_case(2, 1, 1, c2["Sq"], c2["Sk"], kind="distance")).to(dev)
        t = timed(lambda: binding.attn_prefill_fwd_ex(q2, k2, v2, o2, scale=c2["scale"], causal=True, mask=mask2,
                                                      max_bias=8.0))
        variants["prefill_c2_alibi"] = {"workload": "config 2 + fp16 distance mask [1,1,4096,4096], max_bias 8",
                                        "us": round(t * 1e6, 1), "TFLOP/s": round(flops2 / t / 1e12, 1)}
        del mask2
        q2f, k2h, v2h = q2.float(), k2.half(), v2.half()
        t = timed(lambda: binding.attn_prefill_fwd_ex(q2f, k2h, v2h, o2, scale=c2["scale"], causal=True))
        variants["prefill_c2_f16kv_f32q"] = {"workload": "config 2 with fp16 K/V and an fp32 Q",
                                             "us": round(t * 1e6, 1), "TFLOP/s": round(flops2 / t / 1e12, 1)}
        del q2f, k2h, v2h
        kc4h, vc4h = kc4.half(), vc4.half()
        t = timed(lambda: binding.attn_decode_fwd(q4, kc4h, vc4h, o4, ws4, scale=c4["scale"], Sk_max=c4["len_hi"],
                                                  block_table=table4, seq_lens=lens4))
        variants["decode_c4_f16"] = {"workload": "config 4 with fp16 caches", "us": round(t * 1e6, 1),
                                     "GB/s": round(bytes4 / t / 1e9, 1)}
        del kc4h, vc4h
        q4s = torch.randn((c4["B"], 4, c4["Hq"], c4["dk"]), device=dev).to(torch.bfloat16)
        o4s = torch.empty((c4["B"], 4, c4["Hq"], c4["dv"]), device=dev, dtype=torch.bfloat16)
        ws4s = torch.empty(binding.attn_decode_workspace_bytes(c4["B"], c4["Hq"], c4["Hkv"], 4, c4["len_hi"],
                                                               c4["dk"], c4["dv"]), device=dev, dtype=torch.uint8)
        t = timed(lambda: binding.attn_decode_fwd(q4s, kc4, vc4, o4s, ws4s, scale=c4["scale"], Sk_max=c4["len_hi"],
                                                  causal=True, block_table=table4, seq_lens=lens4))
        variants["decode_c4_4tokens"] = {"workload": "config 4 with 4 causal draft tokens per sequence "
                                                     "(32 query columns per KV head)",
                                         "us": round(t * 1e6, 1), "GB/s": round(bytes4 / t / 1e9, 1)}
        del q4s, o4s, ws4s
        nblk = 1 << 24
        src = torch.randint(0, 256, (nblk * 34,), device=dev, dtype=torch.uint8)
        dst = torch.empty(nblk * 32, device=dev, dtype=torch.float16)
        t = timed(lambda: binding.attn_dequant_fp16(src, "q8_0", dst))
        variants["dequant_q8_0"] = {"workload": "2^24 q8_0 blocks (571 MB) to fp16 (1074 MB)",
                                    "us": round(t * 1e6, 1),
                                    "GB/s": round((src.numel() + dst.numel() * 2) / t / 1e9, 1)}
        del src, dst
        # MLA decode tail after config 5: out-absorb + o-projection for its 16 tokens x 128 heads;
        # two weight copies alternate so the 252 MB of weights come from HBM each call
        tc = synth.MLA_TAIL
        T_, H_, R_, DV_, N_ = tc["T"], tc["H"], tc["R"], tc["DV"], tc["N"]
        ol = torch.randn((T_, H_, R_), device=dev).to(torch.bfloat16)
        was = [(torch.randn((H_, DV_, R_), device=dev) * R_ ** -0.5).to(torch.bfloat16) for _ in range(2)]
        wos = [(torch.randn((H_ * DV_, N_), device=dev) * (H_ * DV_) ** -0.5).to(torch.bfloat16) for _ in range(2)]
        yt = torch.empty((T_, N_), device=dev, dtype=torch.bfloat16)
        wst = torch.empty(binding.attn_mla_tail_workspace_bytes(T_, H_, R_, DV_, N_), device=dev, dtype=torch.uint8)
        it = [0]

        def tail_call():
            i = it[0] = (it[0] + 1) % 2
            binding.attn_mla_tail(ol, was[i], wos[i], yt, wst)
        t = timed(tail_call, reps=20)
        tail_bytes = (H_ * DV_ * R_ + H_ * DV_ * N_ + T_ * H_ * R_ + T_ * N_) * 2
        tail_flops = 2.0 * T_ * H_ * DV_ * (R_ + N_)
        variants["mla_tail"] = {"workload": "MLA tail after config 5: 16 tokens, 128 heads, latent 512, "
                                            "v_head_dim 128, hidden 7168 (252 MB of bf16 weights, cold)",
                                "us": round(t * 1e6, 1), "GB/s": round(tail_bytes / t / 1e9, 1),
                                "TFLOP/s": round(tail_flops / t / 1e12, 2)}
        del ol, was, wos, yt, wst
        for k, v in variants.items():
            log("%s: %s" % (k, ", ".join("%s %s" % (a, b) for a, b in v.items() if a != "workload")))
        result["variants"] = variants

    # ---------------- CPU baseline: the oracle on a bounded sample of the prefill workload
    if not args.no_cpu:
        import oracle
        log("CPU oracle baseline")
        pc = synth.prefill_case(c2["seed"], c2["B"], c2["Sq"], c2["Sk"], c2["Hq"], c2["Hkv"], c2["dk"], c2["dv"],
                                std=c2["std"])
        pairs = [(b, h) for b in range(c2["B"]) for h in range(c2["Hq"])][:args.cpu_heads]
        t0 = time.perf_counter()
        for b, h in pairs:
            oracle.prefill(pc["q"], pc["k"], pc["v"], c2["scale"], causal=True, heads=[h], batches=[b])
        tc = time.perf_counter() - t0
        try:  # BLAS threads the oracle's matrix products ran on
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
        except Exception:
            cores = os.cpu_count() or 1
        f = prefill_flops(c2) / (c2["B"] * c2["Hq"]) * len(pairs)
        result["cpu_baseline"] = {"value": round(f / tc / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
                                  "kind": "oracle",
                                  "sample": "%d of the 64 (batch, head) pairs of the causal MHA prefill "
                                            "(4096 x 4096, d=128), fp64 numpy, %.1f s" % (len(pairs), tc)}
        log("oracle: %.1f s for %d heads -> %.4f TFLOP/s" % (tc, len(pairs), f / tc / 1e12))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
