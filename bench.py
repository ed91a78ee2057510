"""Prefill benchmark of token-level sparse attention (select + sparse layers) on one MI355X.

One step = one hybrid module over the whole prompt: hs2_prefill_block, i.e. the
full layer's token selection (row statistics, group scores, top-K + forced
recent window, index rows) followed by every sparse layer reusing K/V and the
index rows (from one shared-gather plan of the rows where that pays: two or more
layers, or rows up to 32768 tokens). Inputs are seeded synthetic bf16 tensors
already resident in HBM.

Default workload: B=1, L=32768, Hq=32, Hkv=8, d=128, K=1024, W=128, needle keys,
1 select + 3 sparse layers. Prints one JSON line.

--decode NAME measures the decode step instead (one new token per sequence
against its KV cache: hs2_decode_select + every sparse layer's
hs2_decode_sparse_attn) and prints its own JSON line.
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "prefill tokens/sec (select+sparse attn) at L=32k; % MFMA peak, % HBM BW"


def algorithmic_work(lengths, Hq, Hkv, d, K, W, elem_bytes=2):
    """Selection MFMA flops (two QK^T passes) and sparse-layer bytes per layer
    (K/V elements of elem_bytes: 2 for bf16, 1 for the FP8 cache)."""
    KW = K + W
    pairs = sum(L * (L + 1) // 2 for L in lengths)
    f_sel = 4 * d * Hq * pairs
    n_sum = 0
    for L in lengths:
        m = min(L, KW)
        n_sum += m * (m + 1) // 2 + (L - m) * KW  # sum_t min(t+1, KW)
    T = sum(lengths)
    gathered = Hkv * n_sum * 2 * d * elem_bytes  # K and V rows, once per (t, g)
    idx_bytes = T * Hkv * KW * 4
    qo_bytes = 2 * T * Hq * d * 2
    return f_sel, gathered + idx_bytes + qo_bytes, n_sum


def kernel_source_hash(name):
    with open(os.path.join(ROOT, "token_level_sparse_hs2_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_profile(workload, key, source):
    """A committed rocprofv3 record (profiles/counters.json) for `key`, if it was taken on
    the current source of its kernel file (else None: the counters describe older code)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(workload, {}).get(key)
    if not e or e.get("source_sha256_16") != kernel_source_hash(source):
        return None
    return e


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def compulsory_bytes(lengths, Hq, Hkv, d, K, W, elem_bytes=2):
    """Bytes one sparse layer cannot avoid moving: every K/V row once, the index rows,
    the layer's queries in and its output out."""
    T = sum(lengths)
    return 2 * T * Hkv * d * elem_bytes + T * Hkv * (K + W) * 4 + 2 * T * Hq * d * 2


def read_counters(db_path):
    """{kernel name: {counter: [value per dispatch]}} from a rocprofv3 --pmc database
    (counters summed over the hardware instances of each dispatch)."""
    import collections
    import sqlite3
    con = sqlite3.connect(db_path)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for disp, kname, cname, val in con.execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        per[(kname, disp)][cname] += val
    con.close()
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (k, _), cs in sorted(per.items(), key=lambda kv: kv[0][1]):
        for c, v in cs.items():
            out[k][c].append(v)
    return out


def summarize_profiles(prof_dir, workload, G, keys=None):
    """Write profiles/counters.json entries for `workload` from the rocprofv3 databases under
    prof_dir (subdirectories fetch*/write*: FETCH_SIZE / WRITE_SIZE with --copy-calibration;
    sq*: SQ counters with GRBM_GUI_ACTIVE; tcc*: TCC hit/miss). Each entry records the
    source hash of its kernel file, so bench.py ignores it once that source changes."""
    import glob
    def db(prefix):
        hits = sorted(glob.glob(os.path.join(prof_dir, prefix + "*", "*_results.db")))
        return read_counters(hits[0]) if hits else {}
    fetch, write, sq, tcc = db("fetch"), db("write"), db("sq"), db("tcc")
    avg = lambda xs: sum(xs) / len(xs)
    # counter scaling from the 1 GiB device copy (--copy-calibration): the copy dispatch
    # (the runtime's blit kernel or torch's copy) with the most bytes
    copies = [k for k in fetch if "copy" in k.lower()]
    ck = max(copies, key=lambda k: max(fetch[k]["FETCH_SIZE"]))
    i = fetch[ck]["FETCH_SIZE"].index(max(fetch[ck]["FETCH_SIZE"]))
    f_factor = (1 << 30) / (fetch[ck]["FETCH_SIZE"][i] * 1024)
    w_factor = (1 << 30) / (max(write[ck]["WRITE_SIZE"]) * 1024)
    kernels = {
        "sparse_planned": (f"sparse_attn_kernel<{G}, false, false, 32, true>", "sparse_attn.hip"),
        "sparse_per_token": (f"sparse_attn_kernel<{G}, false, false, 32, false>", "sparse_attn.hip"),
        "sparse_planned_fp8": (f"sparse_attn_kernel<{G}, false, true, 16, true>", "sparse_attn.hip"),
        "sparse_plan": (f"sparse_plan_kernel<{min(16 // G, 8)}>", "sparse_attn.hip"),
        "scores": (f"scores_kernel<{G}, false>", "select_scores.hip"),
        "topk": ("topk_kernel<", "select_topk.hip"),
        "full_out": (f"full_out_kernel<{G}, false>", "full_out.hip"),
    }
    path = os.path.join(ROOT, "profiles", "counters.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    ent = rec.setdefault(workload, {})
    for key, (pat, src) in kernels.items():
        if keys and key not in keys:
            continue
        name = next((k for k in fetch if pat in k), None)
        if name is None:
            continue
        e = {"kernel": name, "source_sha256_16": kernel_source_hash(src),
             "dispatches": len(fetch[name]["FETCH_SIZE"]),
             "fetch_kib": avg(fetch[name]["FETCH_SIZE"]),
             "write_kib": avg(write[name]["WRITE_SIZE"]) if name in write else None,
             "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4)}
        e["read_bytes"] = int(e["fetch_kib"] * 1024 * f_factor)
        e["write_bytes"] = int((e["write_kib"] or 0) * 1024 * w_factor)
        e["hbm_bytes_per_launch"] = e["read_bytes"] + e["write_bytes"]
        if name in tcc:
            hit, miss = avg(tcc[name]["TCC_HIT_sum"]), avg(tcc[name]["TCC_MISS_sum"])
            e.update({"tcc_hit": hit, "tcc_miss": miss, "l2_hit_rate": round(hit / (hit + miss), 4),
                      "tcc_ea0_rdreq": avg(tcc[name]["TCC_EA0_RDREQ_sum"]),
                      "tcc_ea0_rdreq_dram": avg(tcc[name]["TCC_EA0_RDREQ_DRAM_sum"])})
        if name in sq:
            c = {k: avg(v) for k, v in sq[name].items()}
            e["sq"] = c
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
                # GRBM_GUI_ACTIVE sums the 8 XCDs; 1024 SIMDs each carry one matrix core
                e["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                       (1024 * c["GRBM_GUI_ACTIVE"] / 8), 4)
            if c.get("SQ_INSTS_MFMA"):
                e["valu_per_mfma"] = round(c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"], 3)
                if "SQ_INSTS_VALU_TRANS_F32" in c:
                    e["trans_per_mfma"] = round(c["SQ_INSTS_VALU_TRANS_F32"] / c["SQ_INSTS_MFMA"], 3)
        ent[key] = e
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(ent, indent=1))


def cpu_baseline(inp, w, n_tokens, threads):
    """The oracle (select for every group + every sparse layer) on a uniform token sample."""
    import numpy as np
    import oracle
    T = w.total
    toks = np.unique(np.linspace(0, T - 1, n_tokens).round().astype(np.int64))
    rows = (toks[:, None] * w.Hkv + np.arange(w.Hkv)[None, :]).ravel()
    t0 = time.perf_counter()
    o_idx, _ = oracle.select(inp["q_full"], inp["k"], inp["cu_seqlens"], w.Hq, w.Hkv, w.K, w.W,
                             scale=w.scale, rows=rows, nthreads=threads)
    full_idx = np.full((T, w.Hkv, w.K + w.W), -1, dtype=np.int32)
    full_idx[toks] = o_idx.reshape(len(toks), w.Hkv, -1)
    for qs in inp["q_sparse"]:
        oracle.sparse_attn(qs, inp["k"], inp["v"], inp["cu_seqlens"], w.Hq, w.Hkv, full_idx,
                           scale=w.scale, tokens=toks, nthreads=threads, want_bf16=False)
    dt = time.perf_counter() - t0
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(toks)} tokens evenly spaced over the {T}-token prompt (every KV group, "
                      f"select + {len(inp['q_sparse'])} sparse layers), fp64 C oracle, "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="32k", choices=["tiny", "8k", "32k", "128k", "varlen"])
    ap.add_argument("--cpu-tokens", type=int, default=640)  # about 10 s of oracle work at 32k
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=5)
    ap.add_argument("--no-side", action="store_true",
                    help="skip the side figures (selection variants, FP8 cache, full output, "
                         "exact path): the step and its own kernels only")
    ap.add_argument("--block", action="store_true",
                    help="64-token block selection (the pages' ablation baseline) instead of tokens")
    ap.add_argument("--decode", default=None, choices=["decode-32k", "decode-varlen"],
                    help="time the decode step on this cache workload instead of prefill")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device-to-device copy (known bytes) for counter scaling")
    ap.add_argument("--summarize-profiles", default=None, metavar="DIR",
                    help="write profiles/counters.json entries for --workload from the rocprofv3 "
                         "counter databases under DIR (no GPU needed)")
    ap.add_argument("--summarize-keys", default=None,
                    help="comma-separated entries to write (default: every kernel found)")
    args = ap.parse_args()
    if args.summarize_profiles:
        import synthgen
        w = synthgen.workload(args.workload)
        keys = args.summarize_keys.split(",") if args.summarize_keys else None
        return summarize_profiles(args.summarize_profiles, args.workload, w.Hq // w.Hkv, keys)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the work would shard by KV group, with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    if args.decode:
        return main_decode(args)

    import numpy as np
    import torch
    import synthgen
    import token_level_sparse_hs2_amd as hs2
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from hs2_testlib import GpuCase

    w = synthgen.workload(args.workload)
    t_in = time.perf_counter()
    inp = synthgen.make_inputs(w)
    case = GpuCase(w, inp, flags=hs2.HS2_FLAG_BLOCK_SELECT if args.block else 0)
    gen_s = time.perf_counter() - t_in
    T, Hq, Hkv, d, K, W = w.total, w.Hq, w.Hkv, w.d, w.K, w.W
    n_layers = len(case.q_sparse)
    outs = [torch.empty((T, Hq, d), dtype=torch.bfloat16, device="cuda") for _ in case.q_sparse]
    idx = case.new_idx()
    stream = torch.cuda.current_stream()

    def step():
        hs2.hs2_prefill_block(case.dims, case.varlen, case.q_full, case.k, case.v, case.q_sparse,
                              outs, idx, hs2.HS2_OUT_BF16, case.workspace, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms_per_step = wall * 1e3 / args.steps
    p50, p99 = float(np.percentile(per_step, 50)), float(np.percentile(per_step, 99))

    # per-kernel launch durations with HIP events on the launch stream
    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = args.kernel_reps
    sel_ms = timed(lambda: hs2.hs2_select(case.dims, case.varlen, case.q_full, case.k, idx, None,
                                          case.workspace, stream=stream), reps)
    # the step's sparse layers run from one shared-gather plan of idx
    plan = torch.empty(hs2.hs2_workspace_size(case.dims, case.varlen, hs2.HS2_OP_SPARSE_PLAN),
                       dtype=torch.uint8, device="cuda")
    plan_ms = timed(lambda: hs2.hs2_sparse_plan(case.dims, case.varlen, idx, plan, stream=stream),
                    reps)
    sp_ms = timed(lambda: hs2.hs2_sparse_attn_planned(case.dims, case.varlen, case.q_sparse[0],
                                                      case.k, case.v, plan, outs[0],
                                                      hs2.HS2_OUT_BF16, stream=stream), reps)
    sp_tok_ms = timed(lambda: hs2.hs2_sparse_attn(case.dims, case.varlen, case.q_sparse[0], case.k,
                                                  case.v, idx, outs[0], hs2.HS2_OUT_BF16,
                                                  stream=stream), reps)
    union_rows, pair_rows = plan_rows(plan, case.T, Hq // Hkv, Hkv, K + W, idx)
    f_sel, b_sp, n_sum = algorithmic_work(w.lengths, Hq, Hkv, d, K, W)
    b_comp = compulsory_bytes(w.lengths, Hq, Hkv, d, K, W)
    value = T / (ms_per_step * 1e-3)
    sel_tfs = f_sel / (sel_ms * 1e-3) / 1e12

    # The planned sparse layer (three of the step's kernels) against HBM: the bytes
    # that cross it per launch are rocprofv3's FETCH_SIZE / WRITE_SIZE, copy-calibrated
    # (profiles/counters.json, valid for the current sparse_attn.hip only). The
    # method's logical bytes (every (token, group) row gathered once) exceed what
    # reaches HBM: the union gathers a row once per token group and K/V stay in L2/MALL.
    prof_sp = load_profile(args.workload, "sparse_planned", "sparse_attn.hip")
    dram = prof_sp["hbm_bytes_per_launch"] if prof_sp else None
    roofline = {"bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                "achieved": round(dram / (sp_ms * 1e-3) / 1e9, 1) if dram else None,
                "frac": round(dram / (sp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if dram else None,
                "traffic": dram,
                "kernel": "sparse_attn_kernel, planned (one sparse layer)",
                "avg_launch_ms": round(sp_ms, 4),
                "logical_bytes_per_launch": b_sp,
                "logical_rate_gbs": round(b_sp / (sp_ms * 1e-3) / 1e9, 1),
                "compulsory_bytes_per_launch": b_comp,
                "reuse_factor": round(b_sp / b_comp, 1),
                "rows_gathered_per_launch": union_rows, "rows_selected_per_launch": pair_rows,
                "l2_hit_rate": prof_sp.get("l2_hit_rate") if prof_sp else None,
                "plan_ms": round(plan_ms, 4), "per_token_layer_ms": round(sp_tok_ms, 4),
                "note": "achieved/frac: HBM bytes per launch from rocprofv3 FETCH_SIZE x 2 + "
                        "WRITE_SIZE (copy-calibrated, profiles/counters.json) over the live launch "
                        "time; logical bytes count every (token, group) row once; the planned "
                        "layer gathers each row of a token group's union once "
                        "(rows_gathered / rows_selected); plan_ms once per selection"}
    prof_sel = load_profile(args.workload, "scores", "select_scores.hip")
    select_roof = {"bound": "mfma", "achieved": round(sel_tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
                   "unit": "TFLOP/s", "frac": round(sel_tfs / MFMA_BF16_PEAK_TFS, 4),
                   "algorithmic_flops": f_sel, "avg_call_ms": round(sel_ms, 4),
                   "scores_kernel_mfma_busy": prof_sel.get("mfma_busy") if prof_sel else None,
                   "note": "whole hs2_select call (key norms, scores, top-k, exact-path launches); "
                           "algorithmic flops: two QK^T passes over the causal pairs; "
                           "scores_kernel_mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES over the kernel's "
                           "SIMD-cycles (profiles/counters.json)"}
    # the step's own ceiling: the selection's flops at the bf16 peak plus each sparse
    # layer's compulsory bytes at the HBM peak
    ceiling_s = f_sel / (MFMA_BF16_PEAK_TFS * 1e12) + n_layers * b_comp / (HBM_PEAK_GBS * 1e9)

    side = {}
    if not args.no_side:
        oam_ms = timed(lambda: hs2.hs2_select_ex(case.dims, case.varlen, case.q_full, case.k, idx,
                                                 None, v=case.v, oam_beta=0.5,
                                                 workspace=case.workspace, stream=stream), reps)
        decay_ms = timed(lambda: hs2.hs2_select_ex(case.dims, case.varlen, case.q_full, case.k, idx,
                                                   None, decay_mu=0.5, workspace=case.workspace,
                                                   stream=stream), reps)
        select_roof["oam_avg_call_ms"] = round(oam_ms, 4)
        select_roof["decay_avg_call_ms"] = round(decay_ms, 4)
        select_roof["note"] += ("; oam_avg_call_ms: hs2_select_ex with the output-aware metric, "
                                "beta 0.5; decay_avg_call_ms: hs2_select_ex with the "
                                "position-decaying budget, top_k 1024 down to 512")
        # FP8 KV cache: the cache written by the quantizer, one sparse layer reading it
        ks, vs = 1.0 / 16, 1.0 / 16
        k8 = torch.empty((T, Hkv, d), dtype=torch.uint8, device="cuda")
        v8 = torch.empty_like(k8)
        quant_ms = timed(lambda: (hs2.hs2_quantize_fp8(case.k, k8, 1.0 / ks, stream=stream),
                                  hs2.hs2_quantize_fp8(case.v, v8, 1.0 / vs, stream=stream)),
                         reps)
        sp8_ms = timed(lambda: hs2.hs2_sparse_attn_planned_fp8(case.dims, case.varlen,
                                                               case.q_sparse[0], k8, v8, ks, vs,
                                                               plan, outs[0], hs2.HS2_OUT_BF16,
                                                               stream=stream), reps)
        sp8_tok_ms = timed(lambda: hs2.hs2_sparse_attn_fp8(case.dims, case.varlen,
                                                           case.q_sparse[0], k8, v8, ks, vs, idx,
                                                           outs[0], hs2.HS2_OUT_BF16,
                                                           stream=stream), reps)
        _, b_sp8, _ = algorithmic_work(w.lengths, Hq, Hkv, d, K, W, elem_bytes=1)
        q_bytes = 2 * T * Hkv * d * (2 + 1)  # K and V: bf16 read, codes written
        prof_sp8 = load_profile(args.workload, "sparse_planned_fp8", "sparse_attn.hip")
        dram8 = prof_sp8["hbm_bytes_per_launch"] if prof_sp8 else None
        side["fp8_kv"] = {
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
            "sparse_layer_ms": round(sp8_ms, 4), "per_token_layer_ms": round(sp8_tok_ms, 4),
            "sparse_achieved": round(dram8 / (sp8_ms * 1e-3) / 1e9, 1) if dram8 else None,
            "sparse_frac": round(dram8 / (sp8_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if dram8 else None,
            "sparse_logical_bytes": b_sp8,
            "quantize_ms": round(quant_ms, 4),
            "quantize_achieved": round(q_bytes / (quant_ms * 1e-3) / 1e9, 1),
            "quantize_frac": round(q_bytes / (quant_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "FP8 (E4M3) KV cache, scales 1/16: hs2_quantize_fp8 of K and V, then one "
                    "planned sparse layer over the codes (hs2_sparse_attn_planned_fp8); "
                    "sparse_achieved from the layer's counter HBM bytes"}
        # the full layer's own output, alone (full_out_kernel)
        full_out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device="cuda")
        full_ms = timed(lambda: hs2.hs2_full_attn(case.dims, case.varlen, case.q_full, case.k,
                                                  case.v, full_out, hs2.HS2_OUT_BF16,
                                                  stream=stream), reps)
        sel_full_ms = timed(lambda: hs2.hs2_select_full(case.dims, case.varlen, case.q_full, case.k,
                                                        case.v, idx, full_out, hs2.HS2_OUT_BF16,
                                                        workspace=case.workspace, stream=stream),
                            reps)
        f_out = f_sel  # one QK^T and one PV pass over the causal pairs: 2 * 2 * d * Hq * pairs
        side["full_layer_output"] = {
            "bound": "mfma", "unit": "TFLOP/s", "peak": MFMA_BF16_PEAK_TFS,
            "achieved": round(f_out / (full_ms * 1e-3) / 1e12, 1),
            "frac": round(f_out / (full_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
            "algorithmic_flops": f_out, "full_attn_ms": round(full_ms, 4),
            "select_full_ms": round(sel_full_ms, 4),
            "note": "hs2_full_attn (full_out_kernel alone: QK^T and PV over the causal pairs), "
                    "bf16 out; select_full_ms: hs2_select_full (the output sweep, then the "
                    "selection on its statistics)"}
        # a budget above the register-ranked limit: rows ranked from their candidate lists
        dims_x = hs2.make_dims(Hq, Hkv, 3000, W, w.scale)
        ws_x = torch.empty(hs2.hs2_workspace_size(dims_x, case.varlen, hs2.HS2_OP_SELECT),
                           dtype=torch.uint8, device="cuda")
        idx_x = torch.empty((T, Hkv, 3000 + W), dtype=torch.int32, device="cuda")
        big_ms = timed(lambda: hs2.hs2_select(dims_x, case.varlen, case.q_full, case.k, idx_x,
                                              None, ws_x, stream=stream), 1)
        side["large_budget"] = {"top_k": 3000, "window": W, "select_ms": round(big_ms, 3),
                                "note": "hs2_select with top_k = 3000 (above the register-ranked "
                                        "limit of 2048: up to 6016 candidates per row, ranked "
                                        "from the candidate lists by exact_kernel when a prompt "
                                        "is longer than 12032 tokens, else every ranked row "
                                        "through the dense exact path)"}
        del ws_x, idx_x
        # the exact path: every ranked row's scores written whole, then ranked
        dims_e = hs2.make_dims(Hq, Hkv, K, W, w.scale, flags=hs2.HS2_FLAG_EXACT_SELECT)
        ws_e = torch.empty(hs2.hs2_workspace_size(dims_e, case.varlen, hs2.HS2_OP_SELECT),
                           dtype=torch.uint8, device="cuda")
        idx_e = torch.empty((T, Hkv, K + W), dtype=torch.int32, device="cuda")
        exact_ms = timed(lambda: hs2.hs2_select(dims_e, case.varlen, case.q_full, case.k, idx_e,
                                                None, ws_e, stream=stream), 1)
        side["exact_path"] = {"top_k": K, "window": W, "flags": "HS2_FLAG_EXACT_SELECT",
                              "select_ms": round(exact_ms, 3),
                              "note": "hs2_select with the exact flag: every row with more "
                                      "candidates than top_k is ranked by exact_kernel over "
                                      "its whole row of scores"}
        del ws_e, idx_e

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        threads = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                             else (os.cpu_count() or 1)))
        cpu = cpu_baseline(inp, w, args.cpu_tokens, threads)

    wl = {"tiny": "B=1 L=1024 Hq=4 Hkv=1 d=128 K=256 W=32, 1 select + 1 sparse layer",
          "8k": "B=1 L=8192 Hq=32 Hkv=8 d=128 K=1024 W=128, 1 select + 1 sparse layer",
          "32k": "B=1 L=32768 Hq=32 Hkv=8 d=128 K=1024 W=128, needle keys, 1 select + 3 sparse layers",
          "128k": "B=1 L=131072 Hq=64 Hkv=8 d=128 K=1024 W=128, needle keys, 1 select + 3 sparse layers",
          "varlen": f"B=8 lognormal lengths {w.lengths} Hq=32 Hkv=8 d=128 K=1024 W=128, 1 select + 1 sparse layer"}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded bf16 N(0,1) Q/K/V (SplitMix64 + Box-Muller)"
                + (", needle keys" if w.needles else ""),
        "config": {"workload": f"{args.workload}: {wl[args.workload]}"
                               + (", 64-token block selection" if args.block else ""),
                   "global_batch": len(w.lengths),
                   "seq_len": max(w.lengths), "tokens": T, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "select": select_roof,
        **side,
        "p50_ms": round(p50, 4), "p99_ms": round(p99, 4), "jitter_flag": bool(p99 > 1.3 * p50),
        "ceiling_tokens_per_s": round(T / ceiling_s, 1),
        "ceiling_note": "the step's bound: the selection's algorithmic flops at the bf16 MFMA peak "
                        "plus each sparse layer's compulsory bytes at the HBM peak",
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(out), flush=True)


def decode_work(lengths, Hq, Hkv, d, K, W, n_sparse, elem_bytes=2):
    """Algorithmic HBM bytes of one decode step: the K cache read once and the logits
    written and read once (selection), then per sparse layer the gathered K/V rows,
    the index rows and the queries/outputs of the new tokens (K/V elements of
    elem_bytes: 2 for bf16, 1 for the FP8 cache)."""
    KW, B, T = K + W, len(lengths), sum(lengths)
    sel = T * Hkv * d * elem_bytes + 2 * T * Hq * 4 + B * Hq * d * 2 + B * Hkv * KW * 4
    n = sum(min(L, KW) for L in lengths)
    sp = Hkv * n * 2 * d * elem_bytes + B * Hkv * KW * 4 + 2 * B * Hq * d * 2
    return sel, sp


def plan_rows(plan, T, G, Hkv, KW, idx):
    """(rows the planned layer gathers, rows the (token, group) rows select): the sum of
    the plan's union counts (one word per entry, [n_grp * Hkv, NT * KW], then the counts at
    the next 256-byte boundary) and of the valid index entries."""
    import torch
    nt = 16 // G if G >= 2 else 8
    lists = (T + nt - 1) // nt * Hkv
    off = (lists * nt * KW * 4 + 255) // 256 * 256
    counts = plan[off:off + lists * 4].view(torch.int32)
    return int(counts.sum().item()), int((idx >= 0).sum().item())


def main_decode(args):
    import numpy as np
    import torch
    import synthgen
    import token_level_sparse_hs2_amd as hs2
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from hs2_testlib import to_dev_bf16

    w = synthgen.decode_workload(args.decode)
    t_in = time.perf_counter()
    inp = synthgen.make_decode_inputs(w)
    gen_s = time.perf_counter() - t_in
    B, T, Hq, Hkv, d, K, W = len(w.lengths), w.total, w.Hq, w.Hkv, w.d, w.K, w.W
    cu = inp["cu_seqlens"]
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    cache = hs2.VarlenArgs(cu_dev, [int(x) for x in cu])
    dims = hs2.make_dims(Hq, Hkv, K, W, w.scale)
    k, v, q = to_dev_bf16(inp["k"]), to_dev_bf16(inp["v"]), to_dev_bf16(inp["q_dec"])
    qs = [to_dev_bf16(x) for x in inp["q_sparse_dec"]]
    ws = torch.empty(max(1, hs2.hs2_workspace_size(dims, cache, hs2.HS2_OP_DECODE_SELECT, 0)),
                     dtype=torch.uint8, device="cuda")
    ws_sp = torch.empty(max(1, hs2.hs2_workspace_size(dims, cache, hs2.HS2_OP_DECODE_SPARSE, 0)),
                        dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, Hkv, K + W), dtype=torch.int32, device="cuda")
    outs = [torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda") for _ in qs]
    stream = torch.cuda.current_stream()

    def select():
        hs2.hs2_decode_select(dims, cache, q, k, idx, None, ws, stream=stream)

    def sparse(i):
        hs2.hs2_decode_sparse_attn(dims, cache, qs[i], k, v, idx, outs[i], hs2.HS2_OUT_BF16, ws_sp,
                                   stream=stream)

    def step():
        select()
        for i in range(len(qs)):
            sparse(i)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    steps = max(args.steps, 20)
    for _ in range(max(args.warmup, 3)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = timed(step, steps)
    wall = time.perf_counter() - t0
    sel_ms = timed(select, 20)
    sp_ms = timed(lambda: sparse(0), 20)
    # the same step captured once in a HIP graph and replayed (no per-call host work)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        hs2.hs2_decode_select(dims, cache, q, k, idx, None, ws, stream=cap)
        for i in range(len(qs)):
            hs2.hs2_decode_sparse_attn(dims, cache, qs[i], k, v, idx, outs[i], hs2.HS2_OUT_BF16,
                                       ws_sp, stream=cap)
    graph_ms = timed(graph.replay, steps)
    b_sel, b_sp = decode_work(w.lengths, Hq, Hkv, d, K, W, len(qs))
    # the same step over an FP8 (E4M3) KV cache: selection and sparse layers read codes
    ks8, vs8 = 1.0 / 16, 1.0 / 16
    k8 = torch.empty((T, Hkv, d), dtype=torch.uint8, device="cuda")
    v8 = torch.empty_like(k8)
    hs2.hs2_quantize_fp8(k, k8, 1.0 / ks8, stream=stream)
    hs2.hs2_quantize_fp8(v, v8, 1.0 / vs8, stream=stream)
    idx8 = torch.empty_like(idx)

    def step_fp8():
        hs2.hs2_decode_select_fp8(dims, cache, q, k8, ks8, idx8, None, ws, stream=stream)
        for i in range(len(qs)):
            hs2.hs2_decode_sparse_attn_fp8(dims, cache, qs[i], k8, v8, ks8, vs8, idx8, outs[i],
                                           hs2.HS2_OUT_BF16, ws_sp, stream=stream)

    step8_ms = timed(step_fp8, 20)
    b_sel8, b_sp8 = decode_work(w.lengths, Hq, Hkv, d, K, W, len(qs), elem_bytes=1)
    b_step8 = b_sel8 + len(qs) * b_sp8
    b_step = b_sel + len(qs) * b_sp
    gbs = b_step / (step_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        c0 = time.perf_counter()
        o_idx, _ = oracle.decode_select(inp["q_dec"], inp["k"], cu, Hq, Hkv, K, W, scale=w.scale,
                                        nthreads=threads)
        for x in inp["q_sparse_dec"]:
            oracle.decode_sparse_attn(x, inp["k"], inp["v"], cu, Hq, Hkv, o_idx.reshape(B, Hkv, -1),
                                      scale=w.scale, nthreads=threads, want_bf16=False)
        dt = time.perf_counter() - c0
        cpu = {"value": B / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole step ({B} sequences, every KV group, select + {len(qs)} sparse "
                         f"layers), fp64 C oracle, {dt:.1f} s wall"}

    out = {
        "metric": "decode tokens/sec (select + sparse attn over the KV cache), one new token per "
                  "sequence",
        "value": round(B / (step_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "ms_per_step": round(step_ms, 5), "wall_s": round(wall, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded bf16 N(0,1) K/V cache and queries (SplitMix64 + Box-Muller)",
        "config": {"workload": f"{args.decode}: B={B} caches of lengths {w.lengths[:8]} "
                               f"Hq={Hq} Hkv={Hkv} d={d} K={K} W={W}, 1 select + {len(qs)} sparse "
                               f"layers", "global_batch": B, "cache_tokens": T,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole decode step", "algorithmic_bytes_per_step": b_step},
        "select_ms": round(sel_ms, 5), "sparse_layer_ms": round(sp_ms, 5),
        "graph_ms_per_step": round(graph_ms, 5),
        "select_bytes": b_sel, "sparse_layer_bytes": b_sp,
        "fp8_kv": {"ms_per_step": round(step8_ms, 5),
                   "tokens_per_s": round(B / (step8_ms * 1e-3), 1),
                   "achieved": round(b_step8 / (step8_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                   "algorithmic_bytes_per_step": b_step8,
                   "note": "the same step over an E4M3 KV cache (hs2_decode_select_fp8 + "
                           "hs2_decode_sparse_attn_fp8)"},
        "cpu_baseline": cpu, "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
