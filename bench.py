#!/usr/bin/env python3
"""Benchmark of the prefill attention-unit path on one MI355X.

One step = the whole path on one batch of synthetic input, on one HIP stream:
  qkv_proj (fused QKV GEMM) -> prefill_attention (causal GQA flash attention,
  reading Q/K/V as strided views of the projection output) -> kv_cache_write
  (paged scatter into 16-token pages).
Inputs are seeded draws (``workloads``) already resident in HBM before timing.

Printed: one JSON line.  ``value`` is the attention throughput in TFLOP/s
(causal FLOPs counted as 2*2*s^2*head_dim*n_head/2, summed over sequences)
over the attention kernel's average duration inside the timed steps, measured
with HIP events on the stream the kernels run on; ``ms_per_step`` is the wall
time of a whole step.  ``roofline`` describes the attention kernel against the
bf16 dense MFMA peak, ``kernels`` every kernel, ``cpu_baseline`` the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (published)
KV_SETS = 8                    # rotating buffer sets for the cold KV-write timing
METRIC = "prefill attention TFLOPS + % bf16 MFMA peak, s=8192 GQA 32q/8kv hd128"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed steps first (the clocks settle over the first ~0.3 s of load)")
    ap.add_argument("--workload", default="gqa_s8192",
                    help="gqa_s8192 (default), mha_s2048, varlen16_gqa, long_gqa_s32768_fp8kv")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle sample time")
    ap.add_argument("--kv-cold-reps", type=int, default=20)
    ap.add_argument("--extra-reps", type=int, default=20,
                    help="reps of the extra measurements (fused GEMM + KV write, paged chunk attention); 0 skips")
    ap.add_argument("--split-reps", type=int, default=100,
                    help="reps of the split-key-range side measurement (s=2048, one pass against split); 0 skips")
    ap.add_argument("--clock-seconds", type=float, default=1.0,
                    help="seconds of back-to-back attention launches while the GPU clocks and socket power are "
                         "sampled; 0 skips")
    ap.add_argument("--splitkv-only", action="store_true",
                    help="only run the split-key-range side measurement (--split-reps launches of each kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM byte counters)")
    return ap.parse_args()


def source_sha(name):
    p = os.path.join(ROOT, "prefill_causal_attention_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("attn_fwd_sha") != source_sha("attn_fwd.hip"):
        return None
    return t.get("hbm_bytes_per_launch")


def memory_clock_mhz():
    """HBM clock as amdsmi reports it (MHz), or None."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        try:
            h = amdsmi.amdsmi_get_processor_handles()[0]
            return float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)["clk"])
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception:
        return None


class PowerSampler:
    """Socket power (W) and its cap from amdsmi, sampled every 20 ms in a
    thread while GPU work runs; the first 0.5 s are left out (the reading
    trails the load by about that much).  Silent (None) where amdsmi is
    missing or refuses."""

    def __init__(self):
        import threading
        self.samples, self.cap, self._h = [], None, None
        self._stop = threading.Event()
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            cap = amdsmi.amdsmi_get_power_cap_info(self._h).get("power_cap")
            self.cap = cap / 1e6 if isinstance(cap, (int, float)) else None   # reported in microwatts
        except Exception:
            self._h = None
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        t0 = time.time()
        while not self._stop.is_set():
            try:
                pw = self._smi.amdsmi_get_power_info(self._h).get("current_socket_power")
                if isinstance(pw, (int, float)) and time.time() - t0 >= 0.5:
                    self.samples.append(float(pw))
            except Exception:
                pass
            time.sleep(0.02)

    def __enter__(self):
        if self._h is not None:
            self._t.start()
        return self

    def __exit__(self, *exc):
        if self._h is not None:
            self._stop.set()
            self._t.join()
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass

    def result(self):
        return {"socket_power_w": sum(self.samples) / len(self.samples) if self.samples else None,
                "power_cap_w": self.cap, "power_samples": len(self.samples)}


def sample_clocks(pca, torch, launch, seconds):
    """Average shader clock of each XCD while `launch` runs back to back for
    about `seconds`, from the GPU's own counters (two pca.clock_stamp calls on
    the same stream around the launches); the median over the XCDs is
    sclk_mhz."""
    if seconds <= 0:
        return {"sclk_mhz": None, "note": "not sampled (--clock-seconds 0)"}
    dev = torch.device("cuda:0")
    a = torch.zeros(pca.CLOCK_STAMP_WORDS, dtype=torch.int64, device=dev)
    b = torch.zeros_like(a)
    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launch()
    e1.record()
    torch.cuda.synchronize()
    n = max(1, int(seconds * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
    with PowerSampler() as pw:
        pca.clock_stamp(a)
        for _ in range(n):
            launch()
        pca.clock_stamp(b)
        torch.cuda.synchronize()
    per_xcd = pca.shader_clock_mhz(a.cpu().numpy(), b.cpu().numpy())
    vals = sorted(per_xcd.values())
    return {"sclk_mhz": vals[len(vals) // 2] if vals else None, "sclk_per_xcd_mhz": per_xcd,
            "mclk_mhz": memory_clock_mhz(), **pw.result(),
            "note": f"shader clock = s_memtime cycles / s_memrealtime (100 MHz) on each CU's own counters over {n} "
                    "back-to-back attention launches after the timed steps, per XCD the median over its CUs, "
                    "sclk_mhz the median over XCDs; mclk from amdsmi; socket_power_w: amdsmi's socket power "
                    "averaged over those launches after their first 0.5 s, power_cap_w the board's cap"}


def cpu_baseline(w, target_s):
    """Time the fp64 oracle's attention on a sample of query rows (all heads)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads
    from oracle import attention as A

    buf, *_ = workloads.qkv_inputs(w)
    b = buf.view(__import__("torch").int16).numpy().view(np.uint16)
    q, k, v = A.head_split(b, w.n_head, w.n_kv_head, w.head_dim)
    cu = workloads.cu_seqlens(w)
    rng = np.random.default_rng(12345)

    def run(n):
        rows = np.sort(rng.choice(w.total_tokens, size=n, replace=False))
        t0 = time.perf_counter()
        A.varlen_causal_attention(q, k, v, cu, rows=rows)
        dt = time.perf_counter() - t0
        seq = np.searchsorted(cu, rows, side="right") - 1
        pos = rows - cu[seq]
        flops = float(np.sum(4.0 * (pos + 1) * w.head_dim * w.n_head))   # causal work of these rows
        return dt, flops

    run(32)                      # first call pays numpy/BLAS start-up
    dt, _ = run(128)
    n = int(min(w.total_tokens, max(128, 128 * target_s / max(dt, 1e-3))))
    dt, flops = run(n)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} query rows drawn uniformly from {w.total_tokens}, all {w.n_head} heads, "
                      f"fp64 numpy oracle (full-width masked score rows, two-pass softmax); "
                      f"causal FLOPs of those rows / {dt:.1f} s; BLAS threads={threads}, host cpus={os.cpu_count()}"}


def splitkv_side(pca, torch, dev, reps):
    """One 2048-token sequence, hd 128, MHA (32/32) then GQA (32/8): the
    one-pass attention kernel against the split entry point, each `reps`
    launches after 3 untimed ones, HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev)
    out = {}
    for H, Hk in ((32, 32), (32, 8)):
        S, hd = 2048, 128
        gen.manual_seed(9005)
        q = torch.randn((S, H * hd), generator=gen, device=dev).to(torch.bfloat16)
        kv = torch.randn((S, 2 * Hk * hd), generator=gen, device=dev).to(torch.bfloat16)
        k, v = kv[:, :Hk * hd], kv[:, Hk * hd:]
        o = torch.empty_like(q)
        ws = torch.zeros(pca.prefill_attention_splitkv_workspace(1, S, H, Hk, hd), dtype=torch.uint8, device=dev)
        times = []
        for fn in (lambda: pca.prefill_attention(q, k, v, o, H, Hk, hd),
                   lambda: pca.prefill_attention_splitkv(q, k, v, o, ws, H, Hk, hd)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / reps)
        flop = 2.0 * 2.0 * S * S * hd * H / 2
        out[f"s2048_h{H}_kv{Hk}"] = {"one_pass_ms": times[0], "split_ms": times[1],
                                     "tflops_one_pass": flop / (times[0] * 1e-3) / 1e12,
                                     "tflops_split": flop / (times[1] * 1e-3) / 1e12}
        del q, kv, k, v, o, ws
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path has no multi-GPU form.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import prefill_causal_attention_amd as pca
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pca.load()
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "reps": 5}), flush=True)
        return
    if args.splitkv_only:
        print(json.dumps({"prefill_attention_splitkv": splitkv_side(pca, torch, torch.device("cuda:0"),
                                                                   max(1, args.split_reps))}), flush=True)
        return
    w = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    T, nk = w.total_tokens, w.n_kv_head * w.head_dim
    lay = pca.kv_layout(w.n_head, w.n_kv_head, w.head_dim, 16, "fp8_e4m3" if w.cache == "fp8" else "bf16")

    x, wq = workloads.projection_inputs(w)
    x = x.to(dev)
    wt = wq.t().contiguous().to(dev)          # weight pre-transposed once, untimed
    del wq
    y = torch.empty((T, lay["qkv_ld"]), dtype=torch.bfloat16, device=dev)
    o = torch.empty((T, w.n_head * w.head_dim), dtype=torch.bfloat16, device=dev)
    cu = torch.from_numpy(workloads.cu_seqlens(w)).to(dev)
    bt_h = workloads.block_table(w)
    bt = torch.from_numpy(np.where(bt_h < 0, 0, bt_h).astype(np.int32)).to(dev)
    shape = (w.num_pages, 16, w.n_kv_head, w.head_dim)
    fp8 = w.cache == "fp8"
    kc = torch.zeros(shape, dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    ks = torch.zeros(shape[:3], dtype=torch.float32, device=dev) if fp8 else None
    vs = torch.zeros_like(ks) if fp8 else None
    q = y[:, lay["q_off"]:lay["q_off"] + w.n_head * w.head_dim]
    k = y[:, lay["k_off"]:lay["k_off"] + nk]
    v = y[:, lay["v_off"]:lay["v_off"] + nk]
    cache_dtype = "fp8_e4m3" if fp8 else "bf16"
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pca.qkv_proj(x, wt, y)
        if ev is not None:
            ev[1].record(stream)
        pca.prefill_attention(q, k, v, o, w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                              max_seqlen=w.max_seqlen)
        if ev is not None:
            ev[2].record(stream)
        pca.kv_cache_write(k, v, bt, kc, vc, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                           cache_dtype=cache_dtype, k_scale=ks, v_scale=vs)
        if ev is not None:
            ev[3].record(stream)


    step()                       # one pass first, so y holds real K/V for the side measurements
    torch.cuda.synchronize()

    # cold KV write: KV_SETS independent (K/V source, page pool) sets written
    # back to back between two events, so a set's lines were last touched
    # KV_SETS - 1 launches (>= 448 MiB of other traffic at s=8192) earlier and
    # no longer sit in L2 or the 256 MB MALL; per-launch time = span / KV_SETS
    # (no event overhead per launch)
    sets = []
    for _ in range(KV_SETS):
        ys = torch.empty_like(y)
        ys[:, lay["k_off"]:].copy_(y[:, lay["k_off"]:])
        kcs, vcs = torch.zeros_like(kc), torch.zeros_like(vc)
        kss = torch.zeros_like(ks) if fp8 else None
        vss = torch.zeros_like(vs) if fp8 else None
        sets.append((ys[:, lay["k_off"]:lay["k_off"] + nk], ys[:, lay["v_off"]:lay["v_off"] + nk], kcs, vcs, kss, vss))

    def kv_round():
        for ks_, vs_, kc_, vc_, ksc, vsc in sets:
            pca.kv_cache_write(ks_, vs_, bt, kc_, vc_, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                               cache_dtype=cache_dtype, k_scale=ksc, v_scale=vsc)

    kv_round()
    torch.cuda.synchronize()
    cold = []
    for _ in range(args.kv_cold_reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kv_round()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) / KV_SETS)
    del sets
    t_kv_cold = np.array(cold)

    # the same box's plain-copy ceiling for those bytes: KV_SETS (source,
    # destination) pairs of the K+V byte count, copied back to back, cold in
    # the same way; bytes moved = read + write
    kv_payload = 2 * T * nk * 2
    pairs = [(torch.ones(kv_payload // 8, dtype=torch.int64, device=dev),
              torch.empty(kv_payload // 8, dtype=torch.int64, device=dev)) for _ in range(KV_SETS)]

    def copy_round():
        for src, dst in pairs:
            dst.copy_(src)

    copy_round()
    torch.cuda.synchronize()
    cold_copy = []
    for _ in range(args.kv_cold_reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        copy_round()
        e1.record(stream)
        torch.cuda.synchronize()
        cold_copy.append(e0.elapsed_time(e1) / KV_SETS)
    del pairs
    t_copy_cold = np.array(cold_copy)

    extras = {}
    if args.extra_reps > 0:
        def timed(fn, reps):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        # the KV-cache write done by the GEMM epilogue, against GEMM + separate write
        def fused():
            pca.qkv_proj_kv_write(x, wt, y, bt, kc, vc, w.n_head, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                                  cache_dtype=cache_dtype, k_scale=ks, v_scale=vs)

        def separate():
            pca.qkv_proj(x, wt, y)
            pca.kv_cache_write(k, v, bt, kc, vc, w.n_kv_head, w.head_dim, cu_seqlens=cu,
                               cache_dtype=cache_dtype, k_scale=ks, v_scale=vs)
        t_sep = timed(separate, args.extra_reps)
        t_fused = timed(fused, args.extra_reps)
        extras["qkv_proj_kv_write"] = {"fused_ms": t_fused, "separate_ms": t_sep,
                                       "gemm_tflops_fused": w.gemm_flops() / (t_fused * 1e-3) / 1e12}

        # chunked prefill: 8 sequences, each a 512-row chunk over a 7680-key cached
        # prefix (bf16 pages, GQA as the workload), the chunk's K/V already paged
        nseq, P, Lq = 8, 7680, 512
        ctx = P + Lq
        npg = ctx // 16
        rng = np.random.default_rng(9001)
        pbt = torch.from_numpy(rng.permutation(nseq * npg).reshape(nseq, npg).astype(np.int32)).to(dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(9002)
        pk = torch.randn((nseq * npg, 16, w.n_kv_head, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        pv = torch.randn((nseq * npg, 16, w.n_kv_head, w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        pq = torch.randn((nseq * Lq, w.n_head * w.head_dim), generator=gen, device=dev).to(torch.bfloat16)
        po = torch.empty_like(pq)
        pcu = torch.arange(0, (nseq + 1) * Lq, Lq, dtype=torch.int32, device=dev)
        pctx = torch.full((nseq,), ctx, dtype=torch.int32, device=dev)

        def paged():
            pca.prefill_attention_paged(pq, po, pk, pv, pbt, pctx, w.n_head, w.n_kv_head, w.head_dim,
                                        cu_seqlens=pcu, max_seqlen=Lq, max_ctx=ctx)
        t_paged = timed(paged, args.extra_reps)
        pflop = 4.0 * w.head_dim * w.n_head * nseq * (Lq * P + Lq * (Lq + 1) / 2)
        extras["prefill_attention_paged"] = {
            "case": f"{nseq} sequences x {Lq}-row chunk over a {P}-key cached prefix, bf16 pages",
            "ms": t_paged, "flop": pflop, "tflops": pflop / (t_paged * 1e-3) / 1e12,
            "flop_count": "exact causal pairs, 4*hd*n_head per (query, visible key)"}
        # the same chunks with a 1024-key sliding window over the key positions
        W = 1024

        def paged_window():
            pca.prefill_attention_paged(pq, po, pk, pv, pbt, pctx, w.n_head, w.n_kv_head, w.head_dim,
                                        cu_seqlens=pcu, max_seqlen=Lq, max_ctx=ctx, window=W)
        t_pw = timed(paged_window, args.extra_reps)
        pwflop = 4.0 * w.head_dim * w.n_head * nseq * Lq * W        # every chunk row sees exactly W keys here
        extras["prefill_attention_paged_window"] = {
            "case": f"{nseq} sequences x {Lq}-row chunk over a {P}-key cached prefix, bf16 pages, window {W}",
            "ms": t_pw, "flop": pwflop, "tflops": pwflop / (t_pw * 1e-3) / 1e12,
            "flop_count": "exact visible pairs, 4*hd*n_head per (query, key in its window)"}
        del pk, pv, pq, po

        if args.split_reps > 0:
            extras["prefill_attention_splitkv"] = splitkv_side(pca, torch, dev, args.split_reps)

        # the two ends of the attention unit: RMSNorm folded into the QKV GEMM
        # (row statistics + scaled epilogue), and W_o with the residual add
        inv_rms = torch.empty((T,), dtype=torch.float32, device=dev)
        t_rms = timed(lambda: pca.rms_norm_qkv_proj(x, wt, y, inv_rms, eps=1e-6), args.extra_reps)
        t_plain = timed(lambda: pca.qkv_proj(x, wt, y), args.extra_reps)
        extras["rms_norm_qkv_proj"] = {"ms": t_rms, "qkv_proj_ms": t_plain,
                                       "gemm_tflops": w.gemm_flops() / (t_rms * 1e-3) / 1e12}
        gen.manual_seed(9003)
        nq = w.n_head * w.head_dim
        w_o = (torch.randn((w.h, nq), generator=gen, device=dev) * nq ** -0.5).to(torch.bfloat16)
        res = torch.randn((T, w.h), generator=gen, device=dev).to(torch.bfloat16)
        t_op = timed(lambda: pca.out_proj_residual(o, w_o, res, res), args.extra_reps)
        oflop = 2.0 * T * nq * w.h
        extras["out_proj_residual"] = {"ms": t_op, "flop": oflop, "tflops": oflop / (t_op * 1e-3) / 1e12,
                                       "case": f"({T}, {nq}) @ W_o ({nq}, {w.h}) + residual, in place"}
        del w_o, res, inv_rms

        # fp8 operands for the projection: W^T quantised once (load time),
        # X quantised per step, then the GEMM on the fp8 matrix cores
        xq = torch.empty((T, w.h), dtype=torch.uint8, device=dev)
        sx = torch.empty((T,), dtype=torch.float32, device=dev)
        wq = torch.empty((w.n_qkv, w.h), dtype=torch.uint8, device=dev)
        sw = torch.empty((w.n_qkv,), dtype=torch.float32, device=dev)
        pca.quantize_rows_fp8(wt, wq, sw)
        t_q = timed(lambda: pca.quantize_rows_fp8(x, xq, sx), args.extra_reps)
        t_g8 = timed(lambda: pca.qkv_proj_fp8(xq, sx, wq, sw, y), args.extra_reps)
        g8 = w.gemm_flops() / (t_g8 * 1e-3) / 1e12
        extras["qkv_proj_fp8"] = {"quantize_x_ms": t_q, "gemm_ms": t_g8, "gemm_tflops": g8,
                                  "frac_fp8_peak": g8 / PEAK_FP8_TFLOPS}
        del xq, sx, wq, sw

        # fp8 operands for the scores: K quantised per (token, kv head) with
        # power-of-two scales (once per step, timed apart), Q inside the kernel
        k8 = torch.empty((T, nk), dtype=torch.uint8, device=dev)
        kex = torch.empty((T, (w.n_kv_head + 3) // 4 * 4), dtype=torch.uint8, device=dev)
        kex_v = kex[:, :w.n_kv_head]
        t_kq = timed(lambda: pca.quantize_heads_fp8(k, k8, kex_v, w.n_kv_head, w.head_dim), args.extra_reps)
        t_a8 = timed(lambda: pca.prefill_attention_fp8qk(q, k8, kex_v, v, o, w.n_head, w.n_kv_head, w.head_dim,
                                                         cu_seqlens=cu, max_seqlen=w.max_seqlen), args.extra_reps)
        # half of the FLOPs (Q.K^T) at the fp8 rate, half (P.V) at the bf16 rate
        mixed_peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
        a8 = w.attention_flops() / (t_a8 * 1e-3) / 1e12
        extras["prefill_attention_fp8qk"] = {
            "case": "same workload, fp8 E4M3 Q.K^T operands with power-of-two row scales, bf16 P.V",
            "ms": t_a8, "tflops": a8, "frac_bf16_peak": a8 / PEAK_BF16_TFLOPS,
            "frac_mixed_peak": a8 / mixed_peak, "mixed_peak_tflops": mixed_peak, "quantize_k_ms": t_kq}
        del k8, kex, kex_v

        # the fp8 KV write at the long-context shape (s=32768, 40 q / 8 kv heads,
        # hd 128, permuted pages), K and V read as column slices of the fused
        # projection output as on the path; cold: 4 independent (output, pools)
        # sets written back to back, per-launch time = span / 4
        w5 = workloads.BY_NAME["long_gqa_s32768_fp8kv"]
        T5, nk5 = w5.total_tokens, w5.n_kv_head * w5.head_dim
        lay5 = pca.kv_layout(w5.n_head, w5.n_kv_head, w5.head_dim, 16, "fp8_e4m3")
        k5o, v5o = lay5["k_off"], lay5["v_off"]
        bt5h = workloads.block_table(w5)
        bt5 = torch.from_numpy(np.where(bt5h < 0, 0, bt5h).astype(np.int32)).to(dev)
        shape5 = (w5.num_pages, 16, w5.n_kv_head, w5.head_dim)
        gen.manual_seed(9004)
        sets5 = []
        for _ in range(4):
            y5 = torch.zeros((T5, lay5["qkv_ld"]), dtype=torch.bfloat16, device=dev)
            y5[:, k5o:v5o + nk5] = torch.randn((T5, v5o + nk5 - k5o), generator=gen, device=dev).to(torch.bfloat16)
            sets5.append((y5[:, k5o:k5o + nk5], y5[:, v5o:v5o + nk5], torch.empty(shape5, dtype=torch.uint8, device=dev),
                          torch.empty(shape5, dtype=torch.uint8, device=dev),
                          torch.empty(shape5[:3], dtype=torch.float32, device=dev),
                          torch.empty(shape5[:3], dtype=torch.float32, device=dev)))

        def kv5_round():
            for k5, v5, kc5, vc5, ks5, vs5 in sets5:
                pca.kv_cache_write(k5, v5, bt5, kc5, vc5, w5.n_kv_head, w5.head_dim, cache_dtype="fp8_e4m3",
                                   k_scale=ks5, v_scale=vs5)
        t5 = timed(kv5_round, max(2, args.extra_reps // 4)) / len(sets5)
        b5 = 2 * T5 * nk5 * 2 + 2 * T5 * nk5 + 2 * T5 * w5.n_kv_head * 4 + 4 * T5 // 16
        extras["kv_cache_write_fp8"] = {
            "case": f"s={T5}, {w5.n_kv_head} kv heads x {w5.head_dim} (slices of the ({T5}, {lay5['qkv_ld']}) "
                    "projection output), fp8 E4M3 pages, cold",
            "ms": t5, "algorithmic_bytes": b5, "gbs": b5 / (t5 * 1e-3) / 1e9,
            "frac_hbm": b5 / (t5 * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del sets5

    # The headline steps run after the side measurements above, so they see the
    # clock the chip holds under sustained load rather than its ramp from idle.
    print(f"[bench] workload={w.name} T={T} warmup={args.warmup} steps={args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    stamp_a = torch.zeros(pca.CLOCK_STAMP_WORDS, dtype=torch.int64, device=dev)
    stamp_b = torch.zeros_like(stamp_a)
    pca.clock_stamp(stamp_a)           # outside the wall-clock window and the events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pca.clock_stamp(stamp_b)
    ms_step = wall * 1e3 / args.steps
    t_gemm = np.array([e[0].elapsed_time(e[1]) for e in events])
    t_attn = np.array([e[1].elapsed_time(e[2]) for e in events])
    t_kv = np.array([e[2].elapsed_time(e[3]) for e in events])
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    clocks = sample_clocks(pca, torch, lambda: pca.prefill_attention(q, k, v, o, w.n_head, w.n_kv_head, w.head_dim,
                                                                      cu_seqlens=cu, max_seqlen=w.max_seqlen),
                           args.clock_seconds)
    steps_clock = pca.shader_clock_mhz(stamp_a.cpu().numpy(), stamp_b.cpu().numpy())
    if steps_clock:
        v_ = sorted(steps_clock.values())
        clocks["sclk_mhz_timed_steps"] = v_[len(v_) // 2]

    att_flops = w.attention_flops()
    gemm_flops = w.gemm_flops()
    eb = 1 if fp8 else 2
    kv_bytes = 2 * T * nk * 2 + 2 * T * nk * eb + (2 * T * w.n_kv_head * 4 if fp8 else 0) + 4 * T // 16
    attn_bytes = 2 * T * w.head_dim * (2 * w.n_head + 2 * w.n_kv_head)
    a_ms = float(t_attn.mean())
    tflops = att_flops / (a_ms * 1e-3) / 1e12

    def kstat(t):
        return {"mean_ms": float(t.mean()), "median_ms": float(np.median(t)),
                "p10_ms": float(np.percentile(t, 10)), "p90_ms": float(np.percentile(t, 90))}

    kernels = {
        "prefill_attention": dict(kstat(t_attn), tflops=tflops, frac_bf16_peak=tflops / PEAK_BF16_TFLOPS,
                                  flop=att_flops, algorithmic_bytes=attn_bytes),
        "qkv_proj": dict(kstat(t_gemm), tflops=gemm_flops / (t_gemm.mean() * 1e-3) / 1e12,
                         frac_bf16_peak=gemm_flops / (t_gemm.mean() * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         flop=gemm_flops),
        "kv_cache_write": dict(kstat(t_kv), algorithmic_bytes=kv_bytes,
                               gbs_in_step=kv_bytes / (t_kv.mean() * 1e-3) / 1e9,
                               cold_mean_ms=float(t_kv_cold.mean()),
                               cold_median_ms=float(np.median(t_kv_cold)),
                               gbs_cold=kv_bytes / (np.median(t_kv_cold) * 1e-3) / 1e9,
                               frac_hbm_cold=kv_bytes / (np.median(t_kv_cold) * 1e-3) / 1e9 / PEAK_HBM_GBS,
                               copy_ceiling_gbs_cold=2 * kv_payload / (np.median(t_copy_cold) * 1e-3) / 1e9,
                               frac_of_copy_ceiling=(kv_bytes / np.median(t_kv_cold)) /
                               (2 * kv_payload / np.median(t_copy_cold)),
                               copy_ceiling_case=f"plain device copy of the same {kv_payload} K+V bytes "
                                                 f"(torch copy_, {KV_SETS} rotating pairs, cold)"),
    }
    traffic = measured_traffic(w.name)
    roofline = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": f"attn_fwd_kernel<{w.head_dim}, 0, false, false>",
                "flop_per_launch": att_flops, "avg_launch_ms": a_ms,
                "traffic_source": (f"profiles/attn_fwd_{w.name}_traffic.json: rocprofv3 --pmc FETCH_SIZE and "
                                   "WRITE_SIZE of this kernel source (sha-matched), scaled by a plain 1 GiB copy; "
                                   "not measured in this run") if traffic is not None else None,
                "clock": clocks}
    if clocks.get("sclk_mhz"):
        # the published peak assumes 2.4 GHz; at the observed shader clock the same units peak lower
        peak_at_clock = PEAK_BF16_TFLOPS * clocks["sclk_mhz"] / 2400.0
        roofline["peak_at_observed_sclk"] = peak_at_clock
        roofline["frac_at_observed_sclk"] = tflops / peak_at_clock
    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/h) weights, bf16)",
        "config": {"workload": w.name, "seq_lens": list(w.seqlens) if w.num_seqs <= 16 else w.num_seqs,
                   "total_tokens": T, "h": w.h, "n_head": w.n_head, "n_kv_head": w.n_kv_head,
                   "head_dim": w.head_dim, "page_size": 16, "kv_cache": w.cache,
                   "block_table": w.block_table},
        "roofline": roofline,
        "kernels": kernels,
        "path_tflops": (att_flops + gemm_flops) / (ms_step * 1e-3) / 1e12,
        "extras": extras,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
