#!/usr/bin/env python3
"""Top-K microbenchmark: exact radix select (qsa_topk_pages) against the
approximate, early-stopping select (qsa_topk_pages_approx) on the four score
distributions of the Vortex digest's top-K study (bimodal, normal,
lognormal, uniform), at the selection shapes of the sparse-decode
workloads:
  rows512  : 16 sequences x 8 KV heads, 512 pages per row, K = 153 (30%)
  rows8192 : 8 sequences x 8 KV heads, 8192 pages per row, K = 128
For each (shape, distribution) it reports the mean launch time of the exact
kernel and of each approximate setting (digit width, min_confident), the
speed-up, the mean number of radix passes, and recall@K of the approximate
selection against the exact one. Scores are seeded synthetic rows resident
in HBM (the selection reads them right after the scoring kernel wrote them,
so they are L2-warm here too). Times are per launch, from events around a
HIP graph replay of --iters back-to-back launches. One JSON line per
measurement, then a summary line.
"""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

SHAPES = {
    "rows512": dict(B=16, Hkv=8, L=8192, k=153),
    "rows8192": dict(B=8, Hkv=8, L=131072, k=128),
}
SETTINGS = [
    # (digit_bits, min_confident as a fraction of K)
    (8, 0.0), (11, 0.0), (13, 0.0), (11, 0.5), (11, 0.9), (13, 0.9), (11, 1.0),
]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--iters", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--shapes", default="rows512,rows8192")
    args = ap.parse_args()

    import numpy as np
    import torch
    import workloads
    from query_aware_sparse_page_amd import qsa

    if not torch.cuda.is_available():
        sys.exit("bench_topk.py needs a GPU")
    dev = "cuda:0"
    qsa.lib()

    def timed(fn):
        # The launches are captured in a HIP graph and replayed, so the time
        # is the kernels' and not the Python call overhead's.
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(args.iters):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.iters          # us per launch

    summary = []
    for shape in args.shapes.split(","):
        cfg = SHAPES[shape]
        B, Hkv, L, k = cfg["B"], cfg["Hkv"], cfg["L"], cfg["k"]
        for dist in workloads.SCORE_DISTS:
            r = workloads.score_rows(dist, [L] * B, Hkv, seed=workloads.SEED_BASE + 50).to(dev)
            kv = qsa.PagedKV(r.k_pool, None, r.page_indptr, r.page_indices, r.seq_lens)
            ex_out = qsa.topk_pages(r.scores, kv, k)
            us_exact = timed(lambda: qsa.topk_pages(r.scores, kv, k, out=ex_out))
            exact = ex_out[0].cpu().numpy()
            print(json.dumps({"shape": shape, "dist": dist, "kernel": "exact", "us": round(us_exact, 2)}),
                  flush=True)
            best = None
            for bits, frac in SETTINGS:
                mc = int(frac * k)
                ap_out = qsa.topk_pages_approx(r.scores, kv, k, r.row_rand, digit_bits=bits, min_confident=mc,
                                               with_passes=True)
                us = timed(lambda: qsa.topk_pages_approx(r.scores, kv, k, r.row_rand, digit_bits=bits,
                                                         min_confident=mc, out=ap_out))
                sel = ap_out[0].cpu().numpy()
                passes = ap_out[3].cpu().numpy()
                rec = np.mean([len(set(sel[b, h]) & set(exact[b, h])) / k for b in range(B) for h in range(Hkv)])
                row = {"shape": shape, "dist": dist, "kernel": "approx", "digit_bits": bits,
                       "min_confident": mc, "us": round(us, 2), "speedup": round(us_exact / us, 3),
                       "mean_passes": round(float(passes.mean()), 2), "recall_at_k": round(float(rec), 4)}
                print(json.dumps(row), flush=True)
                if rec >= 0.97 and (best is None or us < best["us"]):
                    best = row
            summary.append({"shape": shape, "dist": dist, "exact_us": round(us_exact, 2),
                            "best_approx_at_recall_0.97": best})
    print(json.dumps({"summary": summary}), flush=True)


if __name__ == "__main__":
    main()
