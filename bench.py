"""Benchmark: attention-backward TFLOP/s on kept blocks, 8K block-sparse (keep 0.25).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--algo split_ds|split|loopk|loopq] [--no-cpu-baseline] [--no-compare]

One step = one pass of the whole hot path over one batch of synthetic input:
block presence -> Q->K / K->Q CSR on the GPU, then the backward call (delta
preprocess, the main kernel(s), and for LoopK/LoopQ the fp32 -> bf16
postprocess).  The default algorithm is SPLIT_DS (dK/dV pass storing dS,
then dQ = dS K).  Inputs are resident in HBM before the timed region.  FLOP are
counted over computed blocks only: 2 * (3*Dqk + 2*Dv) per (query, key) pair of
every kept block, whatever the algorithm executes.

The backward's O and LSE come from the GPU forward (`attn_fwd`) on the same
mask, run once before timing.

Printed on stdout: one JSON line.  Progress goes to stderr.  Besides the
contract fields it carries the per-step median / min / P90, the mask
conversion alone as GB/s (`converter`), the forward alone (`forward`), the
index producer alone (`indexer_topk`: top-k of a 16K packed-causal score
matrix), the
pre/postprocess GB/s, the main kernels' TFLOP/s and, unless --no-compare, the
other algorithms' step times.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "blocksparse_mha_s8k_d128"
METRIC = "attn-bwd TFLOP/s on kept blocks, 8K block-sparse 0.75; % bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2500.0          # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
# kernels of each algorithm: (name, timer stage, algorithmic FLOP per pair, executed FLOP per pair)
def main_kernels(algo, dqk, dv):
    full = 2 * (3 * dqk + 2 * dv)
    if algo == "loopk":
        return [("k_bwd_loopk", 1, full, full)]
    if algo == "loopq":
        return [("k_bwd_loopq", 1, full, full)]
    if algo == "split_ds":
        # the dK/dV pass (first) also stores dS; the dQ pass streams it back (dQ GEMM only)
        return [("k_bwd_dkdv", 1, 2 * (2 * dqk + 2 * dv), 2 * (2 * dqk + 2 * dv)),
                ("k_bwd_dq_ds", 2, 2 * dqk, 2 * dqk)]
    # split: the dQ pass (first) does dQ plus a recompute of S and dP; the dK/dV pass does S, dP, dV, dK
    return [("k_bwd_dq", 1, 2 * dqk, 2 * (2 * dqk + dv)),
            ("k_bwd_dkdv", 2, 2 * (2 * dqk + 2 * dv), 2 * (2 * dqk + 2 * dv))]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kept_blocks(w, presence=None, indices_presence=None):
    """Computed (b, head, qb, kb) blocks: mask blocks with at least one visible pair."""
    n_qb, n_kb = w.n_qb, w.n_kb
    if w.mask in ("block", "index"):
        p = presence if presence is not None else indices_presence
        Hm = p.shape[1]
        cnt = 0
        if w.causal:
            qb = np.arange(n_qb)[:, None]
            kb = np.arange(n_kb)[None, :]
            last = np.minimum((qb + 1) * 128, w.seqlen_q) - 1
            vis = kb * 128 <= last + w.seqlen_k - w.seqlen_q
            cnt = int(((p != 0) & vis[None, None]).sum())
        else:
            cnt = int((p != 0).sum())
        return cnt * (w.heads_q // Hm)
    per_head = 0
    for qb in range(n_qb):
        if w.causal:
            last = min((qb + 1) * 128, w.seqlen_q) - 1
            lim = last + w.seqlen_k - w.seqlen_q
            per_head += 0 if lim < 0 else min(n_kb, lim // 128 + 1)
        else:
            per_head += n_kb
    return per_head * w.batch * w.heads_q


def flop_per_step(w, kept):
    return kept * 128 * 128 * 2 * (3 * w.dim_qk + 2 * w.dim_v)


def file_sha(path):
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(kernel_key):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            t = json.load(f).get(kernel_key)
        if not t or t.get("source_sha256") != file_sha(t["source"]):
            return None
        return float(t["hbm_bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(w, data, budget_s=20.0, max_slices=64):
    """The fp64 oracle backward (K order) on a bounded sample of the workload:
    whole (batch b, query head h) slices, in order, added until about budget_s
    of CPU time (or max_slices)."""
    import oracle
    cores = len(os.sched_getaffinity(0))            # host cores this process may run on
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = cores
    total_flop, total_s, slices = 0, 0.0, []
    for b in range(w.batch):
        q = oracle.bf16_to_f64(data["q"][b:b + 1])
        k = oracle.bf16_to_f64(data["k"][b:b + 1])
        v = oracle.bf16_to_f64(data["v"][b:b + 1])
        do = oracle.bf16_to_f64(data["do"][b:b + 1])
        if w.mask == "block":
            pres = data["presence"][b:b + 1]
            omask = oracle.block_mask_from_csr(pres.shape[1], *oracle.presence_to_csr(pres))
        elif w.mask == "index":
            rows = data["indices"][b * w.seqlen_q:(b + 1) * w.seqlen_q]
            pres = oracle.indices_to_presence(rows, 1, w.seqlen_q, w.seqlen_k)
            omask = oracle.block_mask_from_csr(pres.shape[1], *oracle.presence_to_csr(pres))
        else:
            omask = oracle.dense_mask()
        for h in range(w.heads_q):
            O, L = oracle.attn_fwd(q, k, v, omask, w.causal, w.scale, heads=[h])
            O = oracle.bf16_to_f64(oracle.round_to_bf16(O))
            L = oracle.round_to_f32(L).astype(np.float64)
            t0 = time.perf_counter()
            oracle.attn_bwd(q, k, v, O, do, L, omask, w.causal, w.scale, order="K", heads=[h])
            total_s += time.perf_counter() - t0
            total_flop += _head_flop(omask, w, h)
            slices.append((b, h))
            log(f"  cpu baseline: batch {b} head {h}: {total_s:.1f} s so far")
            if total_s >= budget_s or len(slices) >= max_slices:
                break
        if total_s >= budget_s or len(slices) >= max_slices:
            break
    return {
        "value": total_flop / total_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(min(cores, threads)),
        "affinity_cores": int(cores),
        "blas_threads": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle backward (K order) of {len(slices)} whole (batch, query head) "
                   f"slices of {w.name}, first {slices[0]} .. last {slices[-1]}: "
                   f"{total_flop / 1e9:.1f} GFLOP in {total_s:.1f} s"),
    }


def cpu_converter(w, data):
    """The oracle's mask conversion on the host (NumPy), for the GPU
    converter's comparison: presence -> CSR (block masks) or indices ->
    presence -> CSR (index masks), whole workload, one run."""
    import oracle
    if w.mask == "block":
        t0 = time.perf_counter()
        oracle.presence_to_csr(data["presence"])
        what = "presence -> CSR"
    elif w.mask == "index":
        t0 = time.perf_counter()
        oracle.presence_to_csr(oracle.indices_to_presence(data["indices"], w.batch, w.seqlen_q, w.seqlen_k))
        what = "indices -> presence -> CSR"
    else:
        return None
    return {"ms": round((time.perf_counter() - t0) * 1e3, 2), "what": what, "kind": "oracle"}


def _head_flop(omask, w, h):
    """FLOP of one (batch, query head) slice over its computed blocks, with the
    convention of the GPU figure (whole 128x128 blocks, ragged edges cut)."""
    per_pair = 2 * (3 * w.dim_qk + 2 * w.dim_v)
    n_qb, n_kb = w.n_qb, w.n_kb
    tot = 0
    for qb in range(n_qb):
        last = min((qb + 1) * 128, w.seqlen_q) - 1
        if omask.kind == "dense":
            kbs = range(n_kb)
        else:
            hm = h * omask.heads // w.heads_q
            r = hm * n_qb + qb
            kbs = omask.q2k_col[omask.q2k_row_ptr[r]:omask.q2k_row_ptr[r + 1]]
        for kb in kbs:
            if w.causal and kb * 128 > last + w.seqlen_k - w.seqlen_q:
                continue
            tot += (last + 1 - qb * 128) * (min((kb + 1) * 128, w.seqlen_k) - kb * 128) * per_pair
    return tot


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--algo", default="split_ds", choices=["split", "split_ds", "loopk", "loopq"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true", help="skip timing the other loop order")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by batch/head with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import index_sparse_attention_amd as isa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    isa.load_library()

    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.name}: generating inputs")
    data = synth.make_workload_inputs(w)
    presence = data.get("presence")
    idx_presence = None
    if w.mask == "index":
        # kept-block count for the FLOP figure comes from the GPU-built CSR below
        pass
    dev = torch.device("cuda:0")
    t = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, do = t(data["q"]), t(data["k"]), t(data["v"]), t(data["do"])

    # mask on the device (once, to size things and count kept blocks)
    if w.mask == "block":
        pres_dev = torch.from_numpy(presence).to(dev)
        mk = lambda: isa.block_mask_to_csr(pres_dev)
    elif w.mask == "index":
        idx_dev = torch.from_numpy(data["indices"]).to(dev)
        mk = lambda: isa.index_to_block_sparse(idx_dev, w.batch, w.seqlen_q, w.seqlen_k)
    else:
        mk = lambda: None
    m0 = mk()
    nnz0 = m0.nnz() if m0 is not None else None    # kept mask blocks (one read; every step's mask has the same)
    if w.mask == "index":
        qp = m0.q2k_row_ptr.cpu().numpy()
        qc = m0.q2k_col[:int(qp[-1])].cpu().numpy()
        idx_presence = np.zeros((w.batch, w.heads_k, w.n_qb, w.n_kb), dtype=np.uint8)
        rows = np.repeat(np.arange(len(qp) - 1), np.diff(qp))
        idx_presence.reshape(-1, w.n_kb)[rows, qc] = 1
    kept = kept_blocks(w, presence, idx_presence)
    flop = flop_per_step(w, kept)
    # the backward's O and LSE come from the GPU forward on the same mask
    o, lse = isa.attn_fwd(q, k, v, mask=m0, causal=w.causal, softmax_scale=w.scale)
    torch.cuda.synchronize()
    log(f"kept blocks {kept}, {flop / 1e9:.1f} GFLOP per step")

    def time_forward(reps=20):
        """The forward alone (not part of the backward step): O and LSE from Q,
        K, V and the mask; FLOP = 2 GEMMs per kept pair."""
        for _ in range(3):
            isa.attn_fwd(q, k, v, mask=m0, causal=w.causal, softmax_scale=w.scale, o=o, lse=lse)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            isa.attn_fwd(q, k, v, mask=m0, causal=w.causal, softmax_scale=w.scale, o=o, lse=lse)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        fwd_flop = kept * 128 * 128 * 2 * (w.dim_qk + w.dim_v)
        tf = fwd_flop / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "tflops": round(tf, 3), "pct_bf16_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2),
                "flop": fwd_flop}

    def run(algo, steps, warmup):
        # the workspace holds SPLIT_DS's dS tiles for the kept blocks only
        ws = torch.empty(isa.attn_bwd_workspace_bytes(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_k,
                                                      w.dim_qk, w.dim_v, algo, mask=m0, causal=w.causal),
                         dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        timer = isa.Timer(capacity=max(steps, 1))

        def step(tm):
            m = mk()
            if m is not None:
                m.nnz_host = nnz0
            isa.attn_bwd(q, k, v, o, do, lse, mask=m, causal=w.causal, softmax_scale=w.scale, algo=algo,
                         dq=dq, dk=dk, dv=dv, workspace=ws, timer=tm)

        for _ in range(warmup):
            step(None)
        torch.cuda.synchronize()
        timer.reset()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            step(timer)
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = ev[0].elapsed_time(ev[-1])
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
        n, stage = timer.read()
        timer.close()
        return {"ms_per_step": ev_ms / steps, "wall_ms_per_step": wall * 1e3 / steps,
                "step_ms": {"median": float(np.median(per)), "min": float(per.min()),
                            "p90": float(np.percentile(per, 90))},
                "stage_ms": [s / max(n, 1) for s in stage], "n_timed": n}

    def time_converter(reps=20):
        """The mask conversion alone (it is also inside every step), as GB/s
        over the bytes it must read: the presence matrix (block masks) or the
        index tensor (index masks)."""
        if w.mask not in ("block", "index"):
            return None
        for _ in range(3):
            mk()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            mk()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        nbytes = int(pres_dev.numel()) if w.mask == "block" else int(idx_dev.numel()) * 4
        return {"ms": round(ms, 4), "bytes_read": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "what": "presence -> CSR" if w.mask == "block" else "indices -> presence -> CSR"}

    def time_topk(pack=16384, nseq=4, k=2048, reps=5):
        """The index producer alone (not part of the backward step): top-k of a
        packed-causal fp32 score matrix (pack x pack, nseq sequences, each row
        limited to its causal range in its sequence), k positions per row."""
        g = torch.Generator(device=dev).manual_seed(7)
        x = torch.randn(pack, pack, device=dev, dtype=torch.float32, generator=g)
        seg = pack // nseq
        st = torch.tensor(np.repeat(np.arange(nseq) * seg, seg), dtype=torch.int32, device=dev)
        en = torch.tensor(np.concatenate([np.arange(seg) + 1 + i * seg for i in range(nseq)]), dtype=torch.int32,
                          device=dev)
        out = isa.topk_select(x, k, st, en)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            isa.topk_select(x, k, st, en, out=out)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        valid = int((en - st).sum().item())
        del x
        return {"ms": round(ms, 4), "pack": pack, "sequences": nseq, "topk": k,
                "valid_score_gbs": round(valid * 4 / (ms * 1e-3) / 1e9, 1)}

    if args.algo == "split_ds" and isa.choose_algo(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_k, w.dim_qk,
                                                   w.dim_v, mask=m0, causal=w.causal, device=dev) != "split_ds":
        log("split_ds: the dS store does not fit the free device memory; timing split instead")
        args.algo = "split"
    def time_atomic_ceiling(n_add=1 << 27, n_dst=1 << 24, reps=5):
        """fp32 global atomic adds per second of a plain library kernel (torch
        index_add_: one atomic add per source element, consecutive elements to
        consecutive destinations), the reference rate for the atomic
        reductions of LoopK (dK/dV) and LoopQ (dQ)."""
        dst = torch.zeros(n_dst, dtype=torch.float32, device=dev)
        src = torch.ones(n_add, dtype=torch.float32, device=dev)
        idx = torch.arange(n_add, dtype=torch.int64, device=dev) % n_dst
        dst.index_add_(0, idx, src)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dst.index_add_(0, idx, src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        del dst, src, idx
        return {"g_atomics_per_s": round(n_add / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4),
                "adds": n_add, "dst_elems": n_dst, "what": "torch index_add_ fp32"}

    log(f"timing {args.algo}: {args.warmup} warmup + {args.steps} steps")
    r = run(args.algo, args.steps, args.warmup)
    pairs = kept * 128 * 128
    value = flop / (r["ms_per_step"] * 1e-3) / 1e12
    kern = []
    for name, stage, alg_pp, exe_pp in main_kernels(args.algo, w.dim_qk, w.dim_v):
        ms = r["stage_ms"][stage]
        kern.append({"kernel": name, "avg_launch_ms": round(ms, 4),
                     "algorithmic_tflops": round(pairs * alg_pp / (ms * 1e-3) / 1e12, 3),
                     "executed_mfma_tflops": round(pairs * exe_pp / (ms * 1e-3) / 1e12, 3)})
        if name == "k_bwd_dq_ds":                  # streams 2 bytes of stored dS per pair
            kern[-1]["ds_read_gbs"] = round(pairs * 2 / (ms * 1e-3) / 1e9, 1)
        if name in ("k_bwd_loopk", "k_bwd_loopq"):  # fp32 atomic adds: dK+dV per key (LoopK), dQ per query (LoopQ)
            per_pair = (w.dim_qk + w.dim_v) / 128 if name == "k_bwd_loopk" else w.dim_qk / 128
            kern[-1]["g_atomics_per_s"] = round(pairs * per_pair / (ms * 1e-3) / 1e9, 1)
    dom = max(kern, key=lambda k: k["avg_launch_ms"])
    traffic = load_traffic(f"{dom['kernel']}:{args.algo}:{w.name}")
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_k": w.heads_k,
                   "seqlen_q": w.seqlen_q, "seqlen_k": w.seqlen_k, "dim_qk": w.dim_qk, "dim_v": w.dim_v,
                   "causal": w.causal, "mask": w.mask, "block": 128, "keep_prob": w.keep_prob,
                   "topk": w.topk, "kept_blocks": kept, "algo": args.algo, "seed": w.seed},
        "pct_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": dom["algorithmic_tflops"], "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom["algorithmic_tflops"] / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": dom["kernel"], "avg_launch_ms": dom["avg_launch_ms"],
                     "executed_mfma_tflops": dom["executed_mfma_tflops"]},
        "kernels": kern,
        "stages_ms": {"pre": round(r["stage_ms"][0], 4), "main_a": round(r["stage_ms"][1], 4),
                      "main_b": round(r["stage_ms"][2], 4), "post": round(r["stage_ms"][3], 4)},
        "step_ms": {k: round(v, 4) for k, v in r["step_ms"].items()},
        "converter": time_converter(),
        "forward": time_forward(),
        "indexer_topk": time_topk(),
        "atomic_ceiling": time_atomic_ceiling(),
    }
    rows_q = w.batch * w.seqlen_q * w.heads_q
    rows_k = w.batch * w.seqlen_k * w.heads_k
    pre_bytes = rows_q * w.dim_v * 2 * 2 + rows_q * 4
    post_bytes = 0
    if args.algo == "loopk":
        pre_bytes += rows_k * (w.dim_qk + w.dim_v) * 4
        post_bytes = rows_k * (w.dim_qk + w.dim_v) * (4 + 2)
    elif args.algo == "loopq":
        pre_bytes += rows_q * w.dim_qk * 4
        post_bytes = rows_q * w.dim_qk * (4 + 2)
    elif args.algo == "split_ds":
        pre_bytes += rows_q * 4 * 2                # lse read, lse * log2(e) written
    out["prepost_gbs"] = {"pre": round(pre_bytes / (r["stage_ms"][0] * 1e-3) / 1e9, 1),
                          "post": (round(post_bytes / (r["stage_ms"][3] * 1e-3) / 1e9, 1)
                                   if post_bytes else None),
                          "peak": HBM_PEAK_GBS}
    if not args.no_compare:
        out["compare"] = []
        for other in [a for a in ("split", "split_ds", "loopk", "loopq") if a != args.algo]:
            log(f"timing {other} for comparison")
            torch.cuda.synchronize()
            torch.cuda.empty_cache()                # the previous run's workspace back to the device first
            r2 = run(other, max(10, args.steps // 2), 3)
            out["compare"].append({"algo": other, "ms_per_step": round(r2["ms_per_step"], 4),
                                   "value": round(flop / (r2["ms_per_step"] * 1e-3) / 1e12, 3),
                                   "stages_ms": [round(x, 4) for x in r2["stage_ms"]],
                                   "step_ms": {k: round(v, 4) for k, v in r2["step_ms"].items()}})
            if other in ("loopk", "loopq"):           # fp32 atomic adds per second of the main kernel
                n_at = pairs * ((w.dim_qk + w.dim_v) if other == "loopk" else w.dim_qk) / 128
                out["compare"][-1]["g_atomics_per_s"] = round(n_at / (r2["stage_ms"][1] * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, data)
        out["converter_cpu"] = cpu_converter(w, data)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
