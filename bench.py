"""KDA operator benchmark on one MI355X.

One step = the whole hot path once:
  * chunked prefill, bf16 q/k/v, fp32 alpha/beta/state/o:
    B=1, H=32, T=8192, d_k=d_v=128, chunk 64, zero initial state
  * one recurrent decode step: 256 sequences x 32 heads, d=128, fp32 state
    (256x32x128x128) updated in place, bf16 q/k/v; the states are prefill
    end-states of 64 seeded tokens per (sequence, head).
Inputs are seeded synthetic data resident in HBM before timing starts.

Prints ONE JSON line.  `value` is prefill tokens/s (tokens of the 8192-token
sequence per second of prefill-kernel time); decode us/step is reported next
to it.  Kernel times come from HIP events recorded on the stream the kernels
are launched on (torch's current stream), averaged over the timed steps.
The line also carries: `parity` (the timed launches' outputs against the
fp64 oracle: prefill o and state on heads 0 and 31, o on every head for the
tokens the cpu_baseline leg ran, the decode step on three sequences),
`more_configs` (the packed 64-sequence prefill and the 1M-token prefill with
1024 decode steps after it: times, HBM fractions, sampled parity), and `run`
(GPU, software versions, commit or kernel-source hash).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense


def prefill_algorithmic_bytes(T, H, DK, DV, state_in, state_out):
    """q, k, v (bf16) + alpha (fp32) + beta (fp32) + o (fp32) per token-head,
    plus the fp32 states read/written once per (sequence, head)."""
    per_tok_head = 2 * DK + 2 * DK + 2 * DV + 4 * DK + 4 + 4 * DV
    st = 4 * DK * DV * H * (int(state_in) + int(state_out))
    return T * H * per_tok_head + st


def decode_algorithmic_bytes(N, H, DK, DV):
    """fp32 state read + write, bf16 q, k, v, fp32 alpha, beta and o."""
    return N * H * (2 * 4 * DK * DV + 2 * DK + 2 * DK + 2 * DV + 4 * DK + 4 + 4 * DV)


def prefill_algorithmic_flops(T, H, DK, DV, C=64):
    """Triangle-aware plain-product FLOPs per token-head of the chunk form:
    6 DK DV (state products) + (3C+1) DK + 2 (C+1) DV + C^2/3."""
    return T * H * (6 * DK * DV + (3 * C + 1) * DK + 2 * (C + 1) * DV + C * C / 3)


def cpu_baseline(seconds, q, k, v, a, b):
    """The fp64 oracle (as it stands) on the same seeded prefill arrays the GPU
    gets: all heads, the sequence's tokens in order, until `seconds` elapse."""
    from threadpoolctl import threadpool_limits

    from oracle import kda_recurrent

    B, T, H, D = q.shape
    step = 256
    done, t_used, S = 0, 0.0, None
    outs = []
    with threadpool_limits(limits=1):
        while t_used < seconds and done < T:
            sl = slice(done, min(done + step, T))
            t0 = time.perf_counter()
            o, S = kda_recurrent(q[:, sl], k[:, sl], v[:, sl], a[:, sl], b[:, sl], S)
            t_used += time.perf_counter() - t0
            outs.append(o)
            done = sl.stop
    return np.concatenate(outs, axis=1), {
        "value": done / t_used,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"fp64 numpy token recurrence on the benchmark's own inputs: all {H} heads, "
                  f"first {done} of {T} tokens ({t_used:.1f} s, BLAS limited to 1 thread); "
                  f"host {platform.machine()}, {len(os.sched_getaffinity(0))} cores visible",
    }


def source_blob_ids(here):
    """Git blob ids (what `git hash-object FILE` prints, 12 hex digits) of the
    measured code: they identify the committed files also where the tree runs
    without its history (git_commit null)."""
    import hashlib

    csrc = os.path.join(here, "gated_delta_rule_diag_amd", "csrc")
    blobs = {}
    for rel in ["bench.py", "include/kda.h", "gated_delta_rule_diag_amd/kda.py"] + \
            [f"gated_delta_rule_diag_amd/csrc/{n}" for n in sorted(os.listdir(csrc))]:
        with open(os.path.join(here, rel), "rb") as f:
            data = f.read()
        blobs[rel] = hashlib.sha1(b"blob %d\0" % len(data) + data).hexdigest()[:12]
    return blobs


def run_info(torch):
    """What the evaluation pages ask a measurement to state besides the
    numbers: hardware, software versions and the code measured ("Kimi Linear、
    独自の土俵でFull Attentionを上回る" (remio.ai), section "オープンコードにより
    主張は検証可能になる…")."""
    import hashlib
    import subprocess

    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    csrc = os.path.join(here, "gated_delta_rule_diag_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    try:
        commit = subprocess.run(["git", "-C", here, "rev-parse", "HEAD"], capture_output=True,
                                text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        commit = None
    blobs = source_blob_ids(here)
    props = torch.cuda.get_device_properties(0)
    return {
        "gpu": torch.cuda.get_device_name(0),
        "gpu_arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "torch": torch.__version__,
        "hip": torch.version.hip,
        "git_commit": commit,
        "kernel_source_sha256_16": h.hexdigest()[:16],
        "git_blob_ids": blobs,
        "host_cpu": platform.processor() or platform.machine(),
    }


def extra_configs(torch, kda, I, reps=3):
    """The packed-sequence prefill (64 sequences, lengths ~U{512..16384},
    H=32, d=128) and the 1M-token prefill followed by 1024 decode steps
    (B=1, H=32, d=128): times, rates, HBM fractions, and parity of a sample of
    their outputs against the oracle.  Inputs are drawn on the device with the
    recipe's distributions (normalisation in fp32)."""
    from oracle import kda_recurrent, max_rel_err

    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    H, D = 32, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(I.SEED + 34)

    def draw(shape):
        q = torch.randn(shape + (D,), generator=gen, device=dev)
        q = (q / q.norm(dim=-1, keepdim=True)).to(bf)
        k = torch.randn(shape + (D,), generator=gen, device=dev)
        k = (k / k.norm(dim=-1, keepdim=True)).to(bf)
        v = torch.randn(shape + (D,), generator=gen, device=dev).to(bf)
        b = torch.sigmoid(torch.randn(shape, generator=gen, device=dev))
        a = torch.exp(-torch.exp(torch.rand(shape + (D,), generator=gen, device=dev) * 4 - 5))
        return q, k, v, a, b

    def timed(fn, n):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(n):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / n * 1e3   # us per call

    host = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    res = {}
    # ---- packed sequences ----
    lengths = I.varlen_lengths(3, 64, 512, 16384)
    Tt = int(lengths.sum())
    cu_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu = torch.from_numpy(cu_h).to(dev)
    q, k, v, a, b = draw((Tt, H))
    o = torch.empty((Tt, H, D), device=dev, dtype=torch.float32)
    S = torch.empty((64, H, D, D), device=dev, dtype=torch.float32)
    us = timed(lambda: kda.chunk_prefill_varlen(q, k, v, a, b, cu, None, True, 64, o, S), reps)
    nbytes = prefill_algorithmic_bytes(Tt, H, D, D, False, False) + 64 * H * D * D * 4
    n = int(np.argmin(lengths))   # the shortest sequence, head 0, through the oracle
    s0, s1 = int(cu_h[n]), int(cu_h[n + 1])
    sl = lambda t: host(t[s0:s1, 0])[None, :, None]  # noqa: E731
    ro, rS = kda_recurrent(sl(q), sl(k), sl(v), sl(a), host(b[s0:s1, 0])[None, :, None])
    res["varlen_n64_h32_d128"] = {
        "tokens": Tt, "us": us, "tokens_per_s": Tt / (us * 1e-6),
        "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
        "parity": {"sample": f"sequence {n} ({s1 - s0} tokens), head 0",
                   "o": max_rel_err(host(o[s0:s1, 0]), ro[0, :, 0]),
                   "state": max_rel_err(host(S[n, 0]), rS[0, 0])},
    }
    del q, k, v, a, b, o, S, cu
    torch.cuda.empty_cache()
    # ---- 1M-token prefill, then 1024 decode steps from its state ----
    T = 1 << 20
    q, k, v, a, b = draw((1, T, H))
    o = torch.empty((1, T, H, D), device=dev, dtype=torch.float32)
    S = torch.empty((1, H, D, D), device=dev, dtype=torch.float32)
    ws = torch.empty(max(kda.lib().kda_chunk_prefill_workspace_size(1, T, H, D, D, 64), 1),
                     device=dev, dtype=torch.uint8)
    us = timed(lambda: kda.chunk_prefill(q, k, v, a, b, None, True, 64, o, S, ws), 2)
    nbytes = prefill_algorithmic_bytes(T, H, D, D, False, True)
    P = 2048   # the first P tokens of head 0 through the oracle
    sl = lambda t: host(t[:, :P, 0])[:, :, None]  # noqa: E731
    ro, _ = kda_recurrent(sl(q), sl(k), sl(v), sl(a), host(b[:, :P, 0])[:, :, None])
    par = {"sample": f"head 0, the first {P} of {T} tokens (o)",
           "o": max_rel_err(host(o[:, :P, 0]), ro[:, :, 0])}
    del q, k, v, a, o, ws
    torch.cuda.empty_cache()
    dq, dk, dv, da, db = draw((1, H))
    od = torch.empty((1, H, D), device=dev, dtype=torch.float32)
    step = lambda: kda.decode_step(dq, dk, dv, da, db, S, od)  # noqa: E731
    eager = timed(step, 1024)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(16):
            step()
    in_graph = timed(graph.replay, 64) / 16
    res["long_context_t1m_h32_d128"] = {
        "tokens": T, "prefill_us": us, "prefill_tokens_per_s": T / (us * 1e-6),
        "prefill_hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
        "decode_1024_steps_us_per_step_eager": eager,
        "decode_us_per_step_hip_graph_16_steps": in_graph,
        "parity": par,
    }
    del graph, S, dq, dk, dv, da, db, od, b
    torch.cuda.empty_cache()
    return res


def long_context(torch):
    """Decode (B=1, H=32, d=128) from the end state of a prefill of T tokens,
    T = 4K, 64K, 1M: the state does not grow with T, so neither does the step.
    Prints one JSON line with the per-step times (eager, and with 16 steps in
    one HIP graph) and the prefill times."""
    from gated_delta_rule_diag_amd import kda

    dev = torch.device("cuda:0")
    H, D = 32, 128
    g = torch.Generator(device=dev)
    g.manual_seed(4)

    def inputs(T):
        q = torch.randn(1, T, H, D, device=dev, generator=g)
        q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        k = torch.randn(1, T, H, D, device=dev, generator=g)
        k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        v = torch.randn(1, T, H, D, device=dev, generator=g).to(torch.bfloat16)
        a = torch.exp(-torch.exp(torch.rand(1, T, H, D, device=dev, generator=g) * 4 - 5))
        b = torch.sigmoid(torch.randn(1, T, H, device=dev, generator=g))
        return q, k, v, a, b

    def elapsed_us(fn, reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    dq, dk, dv, da, db = (t[:, 0].contiguous() for t in inputs(1))
    o1 = torch.empty((1, H, D), device=dev, dtype=torch.float32)
    rows = []
    for T in (4096, 65536, 1 << 20):
        x = inputs(T)
        kda.chunk_prefill(*x)
        torch.cuda.synchronize()
        pre_us = elapsed_us(lambda: kda.chunk_prefill(*x), 2)
        _, S = kda.chunk_prefill(*x)
        del x
        kda.decode_step(dq, dk, dv, da, db, S, o1)
        torch.cuda.synchronize()
        eager = elapsed_us(lambda: kda.decode_step(dq, dk, dv, da, db, S, o1), 1024)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            kda.decode_step(dq, dk, dv, da, db, S, o1)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(16):
                kda.decode_step(dq, dk, dv, da, db, S, o1)
        graph.replay()
        torch.cuda.synchronize()
        in_graph = elapsed_us(graph.replay, 64) / 16
        rows.append({"T": T, "prefill_us": pre_us, "prefill_tokens_per_s": T / (pre_us * 1e-6),
                     "decode_us_per_step_eager": eager, "decode_us_per_step_hip_graph": in_graph})
        del graph, S
        torch.cuda.empty_cache()
    print(json.dumps({"long_context": {"workload": "B=1 H=32 d=128 bf16 prefill of T tokens, then "
                                                   "decode steps from its end state", "runs": rows}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 30 untimed steps (about 20 ms of sustained work): with 3 the first timed
    # steps still ran at the GPU's ramp-up clocks (prefill 485 us against 457 us
    # from 30 warm-up steps on, the same with 100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the serving variants timed after the steps (profiled runs)")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the packed-sequence and 1M-token workloads timed after the steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 512 MiB device-to-device copy before the timed region "
                         "(reference for HBM byte counters)")
    ap.add_argument("--long-context", action="store_true",
                    help="instead of the step: decode B=1 H=32 d=128 from the end states of "
                         "prefills of 4K, 64K and 1M tokens (per-step time flat in T)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA operator here runs on a single MI355X "
              "(multi-GPU sharding is not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.long_context:
        long_context(torch)
        return

    from gated_delta_rule_diag_amd import inputs as I
    from gated_delta_rule_diag_amd import kda

    dev = torch.device("cuda:0")
    B, T, H, D = 1, 8192, 32, 128
    ND = 256

    # ---- prefill workload (seeded, host-generated, copied to HBM once) ----
    q, k, v, a, b = I.batch_inputs(1, B, T, H, D, D, "bf16")
    bf = torch.bfloat16
    to = lambda x, dt=torch.float32: torch.from_numpy(x).to(dev).to(dt).contiguous()  # noqa: E731
    pq, pk, pv, pa, pb = to(q, bf), to(k, bf), to(v, bf), to(a), to(b)
    po = torch.empty((B, T, H, D), device=dev, dtype=torch.float32)
    pst = torch.empty((B, H, D, D), device=dev, dtype=torch.float32)
    wsz = kda.lib().kda_chunk_prefill_workspace_size(B, T, H, D, D, 64)
    pws = torch.empty(max(wsz, 1), device=dev, dtype=torch.uint8)

    # ---- decode workload ----
    dq, dk_, dv_, da, db = I.decode_inputs(2, ND, H, D, D, "bf16")
    dq, dk_, dv_, da, db = to(dq, bf), to(dk_, bf), to(dv_, bf), to(da), to(db)
    # start states: prefill end-states of 64 seeded tokens per (sequence, head)
    L0 = 64
    gen = torch.Generator(device=dev)
    gen.manual_seed(I.SEED + 2)
    x = torch.randn((ND, L0, H, D), generator=gen, device=dev)
    wq = x / x.norm(dim=-1, keepdim=True)
    x = torch.randn((ND, L0, H, D), generator=gen, device=dev)
    wk = x / x.norm(dim=-1, keepdim=True)
    wv = torch.randn((ND, L0, H, D), generator=gen, device=dev)
    wa = torch.exp(-torch.exp(torch.rand((ND, L0, H, D), generator=gen, device=dev) * 4 - 5))
    wb = torch.sigmoid(torch.randn((ND, L0, H), generator=gen, device=dev))
    _, dstate = kda.chunk_prefill(wq.to(bf), wk.to(bf), wv.to(bf), wa.contiguous(), wb.contiguous())
    del x, wq, wk, wv, wa, wb
    do = torch.empty((ND, H, D), device=dev, dtype=torch.float32)
    dstate0 = dstate.clone()   # the decode's parity is taken from this copy after timing
    if args.copy_calibration:
        src = torch.ones(512 << 18, device=dev, dtype=torch.float32)  # 512 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        kda.chunk_prefill(pq, pk, pv, pa, pb, None, True, 64, po, pst, pws)
        if ev is not None:
            ev[1].record()
        kda.decode_step(dq, dk_, dv_, da, db, dstate, do)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    # ---- parity of the timed launches (same kernels, same launch shapes) ----
    # prefill: po / pst of the last timed step (checked before anything else
    # writes them); decode: one step from the saved start states, checked for
    # sequences 0, 97 and 255 (all heads).
    from oracle import kda_decode_step, kda_recurrent, max_rel_err

    sel = [0, 97, 255]
    d_o = torch.empty_like(do)
    st = dstate0.clone()
    kda.decode_step(dq, dk_, dv_, da, db, st, d_o)
    torch.cuda.synchronize()
    hostf = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    s0h = hostf(dstate0[sel])
    xs = [hostf(t[sel]) for t in (dq, dk_, dv_, da, db)]
    ro_d, rS_d = kda_decode_step(*xs, s0h)
    parity = {
        "tolerance": 2e-3,
        "decode_o": max_rel_err(hostf(d_o[sel]), ro_d),
        "decode_state": max_rel_err(hostf(st[sel]), rS_d),
        "decode_sample": "sequences 0, 97, 255, all 32 heads, the first step from the timed start states",
    }
    del st, d_o, dstate0
    hp = [0, 31]
    ro_p, rS_p = kda_recurrent(q[:, :, hp], k[:, :, hp], v[:, :, hp], a[:, :, hp], b[:, :, hp])
    parity["prefill_o_heads_0_31"] = max_rel_err(hostf(po[:, :, hp]), ro_p)
    parity["prefill_state_heads_0_31"] = max_rel_err(hostf(pst[:, hp]), rS_p)
    po_first = hostf(po)   # compared with the cpu_baseline leg (the oracle) below


    # ---- the serving variants, timed after (and outside) the steps above ----
    def time_call(fn, reps=max(args.steps, 5)):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps * 1e3   # us per call

    dec_bytes = decode_algorithmic_bytes(ND, H, D, D)
    variants = None
    if not args.no_variants:
        hbm = lambda us: dec_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS  # noqa: E731
        # decode steps back to back (no prefill in between: the previous
        # step's writes are not drained while HBM idles)
        b2b_us = time_call(lambda: kda.decode_step(dq, dk_, dv_, da, db, dstate, do))
        snaps = torch.empty((B, T // (64 * 16), H, D, D), device=dev, dtype=torch.float32)
        snap_us = time_call(lambda: kda.chunk_prefill_snapshots(
            pq, pk, pv, pa, pb, 16, None, True, 64, po, pst, snaps, pws))
        del snaps
        pg = pa[..., 0].contiguous()   # one gate per token and head (Gated DeltaNet)
        gate_us = time_call(lambda: kda.chunk_prefill(pq, pk, pv, pg, pb, None, True, 64, po, pst,
                                                      pws))
        del pg
        P = 2 * ND
        gen_p = torch.Generator()
        gen_p.manual_seed(I.SEED + 5)
        slots = torch.randperm(P, generator=gen_p)[:ND].to(torch.int32).to(dev)
        pool = torch.zeros((P, H, D, D), device=dev, dtype=torch.float32)
        pool[slots.long()] = dstate
        pool1_us = time_call(lambda: kda.decode_pool(dq[:, None], dk_[:, None], dv_[:, None],
                                                     da[:, None], db[:, None], pool, slots,
                                                     out=do[:, None]))
        L4 = 4
        rq, rk, rv = (x[:, None].expand(ND, L4, H, D).contiguous() for x in (dq, dk_, dv_))
        ra = da[:, None].expand(ND, L4, H, D).contiguous()
        rb = db[:, None].expand(ND, L4, H).contiguous()
        o4 = torch.empty((ND, L4, H, D), device=dev, dtype=torch.float32)
        pool4_us = time_call(lambda: kda.decode_pool(rq, rk, rv, ra, rb, pool, slots, out=o4))
        del pool, rq, rk, rv, ra, rb, o4
        # one sequence x 32 heads: launch-bound; eager calls vs 16 steps in one HIP graph
        x1 = [t[:1].contiguous() for t in (dq, dk_, dv_, da, db)]
        s1 = dstate[:1].clone()
        o1 = torch.empty((1, H, D), device=dev, dtype=torch.float32)
        n1_eager_us = time_call(lambda: kda.decode_step(*x1, s1, o1), reps=200)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            kda.decode_step(*x1, s1, o1)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(16):
                kda.decode_step(*x1, s1, o1)
        n1_graph_us = time_call(graph.replay, reps=20) / 16
        del graph, x1, s1, o1
        # backward pass (training) of the same prefill workload
        d_o = torch.randn((B, T, H, D), device=dev, dtype=torch.float32)
        bws = torch.empty(kda.lib().kda_chunk_backward_workspace_size(B, T, H, D, D, 64),
                          device=dev, dtype=torch.uint8)
        bwd_us = time_call(lambda: kda.chunk_backward(pq, pk, pv, pa, pb, d_o, workspace=bws),
                           reps=3)
        pg = pa[..., 0].contiguous()
        bwd_sg_us = time_call(lambda: kda.chunk_backward(pq, pk, pv, pg, pb, d_o, workspace=bws),
                              reps=3)
        del d_o, bws, pg
        variants = {
            "decode_back_to_back_us_per_step": b2b_us,
            "decode_back_to_back_hbm_frac": hbm(b2b_us),
            "prefill_with_snapshots_every_1024_tokens_us": snap_us,
            "prefill_scalar_gate_us": gate_us,
            "decode_pool_512_slots_L1_us": pool1_us,
            "decode_pool_512_slots_L1_hbm_frac": hbm(pool1_us),
            "decode_pool_512_slots_L4_us": pool4_us,
            "decode_pool_512_slots_L4_us_per_token": pool4_us / L4,
            "backward_b1_h32_t8192_us": bwd_us,
            # algorithmic bytes of a backward call: q, k, v (bf16), alpha, beta,
            # d_o in; dq, dk, dalpha, dv, dbeta out (3,848 B per token-head at d=128)
            "backward_b1_h32_t8192_hbm_frac": B * T * H * (3 * D * 2 + 4 * D + 4 + 4 * D
                                                           + 3 * 4 * D + 4 * D + 4)
            / (bwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "backward_scalar_gate_b1_h32_t8192_us": bwd_sg_us,
            "decode_n1_h32_eager_us_per_step": n1_eager_us,
            "decode_n1_h32_hip_graph_us_per_step": n1_graph_us,
        }

    extra = None
    if not args.no_extra_configs:
        del pq, pk, pv, pa, pb, pws, dq, dk_, dv_, da, db, dstate, do
        torch.cuda.empty_cache()
        extra = extra_configs(torch, kda, I)

    pre_bytes = prefill_algorithmic_bytes(T, H, D, D, False, True)
    pre_gbs = pre_bytes / (pre_ms * 1e-3) / 1e9
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    pre_tflops = prefill_algorithmic_flops(T, H, D, D) / (pre_ms * 1e-3) / 1e12

    # HBM traffic measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE,
    # scaled by a plain-copy calibration), used only while the kernel source
    # is the one the counters were taken on.
    traffic, traffic_dec = None, None
    here = os.path.dirname(os.path.abspath(__file__))
    tfile = os.path.join(here, "profiles", "traffic.json")
    if os.path.exists(tfile):
        import hashlib

        with open(tfile) as f:
            tj = json.load(f)
        csrc = os.path.join(here, "gated_delta_rule_diag_amd", "csrc")

        def sha16(name):
            with open(os.path.join(csrc, name), "rb") as f:
                return hashlib.sha256(f.read()).hexdigest()[:16]

        if tj.get("prefill_kernel_source_sha256_16") == sha16("kda_prefill.hip"):
            traffic = tj.get("prefill_bytes_per_call")
        if tj.get("decode_kernel_source_sha256_16") == sha16("kda_decode.hip"):
            traffic_dec = tj.get("decode_bytes_per_launch")

    # Which prefill form the library takes for this shape (the same rule as in
    # the library: the staged two-kernel form below 128 (sequence, head) pairs).
    staged = B * H < 128 and T > 64
    stage_name = "kda_stage2_kernel" if D == 128 else "kda_stage_kernel"
    pre_kernels = (f"{stage_name} + kda_chain_kernel (staged form: one pair of launches per "
                   "segment of chunks)"
                   if staged else "kda_prefill_kernel")
    out = {
        "metric": "KDA prefill tokens/s + decode us/step (B=256); % of MFMA / HBM peak",
        "value": T / (pre_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "KDA chunked prefill B=1 H=32 T=8192 d=128 bf16 (chunk 64, zero initial "
                        "state) + one decode step 256 seq x 32 heads d=128 (fp32 state in place)",
            "prefill": {"B": B, "T": T, "H": H, "d_k": D, "d_v": D, "chunk": 64},
            "decode": {"N": ND, "H": H, "d_k": D, "d_v": D},
        },
        "prefill_us": pre_ms * 1e3,
        "decode_us_per_step": dec_ms * 1e3,
        "prefill_form": "staged" if staged else "fused",
        "roofline": {
            "bound": "hbm",
            "kernel": pre_kernels,
            "achieved": pre_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": pre_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes": pre_bytes,
            "algorithmic_tflops": pre_tflops,
            "mfma_frac_algorithmic": pre_tflops / BF16_MFMA_PEAK_TFLOPS,
        },
        "parity": parity,
        "more_configs": extra,
        "serving_variants": variants,
        "run": run_info(torch),
        "roofline_decode": {
            "bound": "hbm",
            "kernel": "kda_decode_kernel",
            "achieved": dec_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS,
            "traffic": traffic_dec,
            "algorithmic_bytes": dec_bytes,
        },
    }
    if not args.no_cpu_baseline:
        ro_c, out["cpu_baseline"] = cpu_baseline(args.cpu_seconds, q, k, v, a, b)
        n_c = ro_c.shape[1]
        n_c = min(n_c, po_first.shape[1])
        parity["prefill_o_all_heads_first_tokens"] = max_rel_err(po_first[:, :n_c], ro_c[:, :n_c])
        parity["prefill_o_all_heads_first_tokens_sample"] = f"all {H} heads, tokens 0..{n_c - 1}"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
