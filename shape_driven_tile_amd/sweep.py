"""Sweep every ladder rung over a list of GEMM shapes on the current GPU.

The FlyDSL pull request "Speed up the RDNA3 GEMM up to 1.85x by choosing the
tile from the shape" fits its pick_tile heuristic to a sweep of every feasible
tile over a set of shapes (Changes); this is that sweep for this library's
ladder, used to set and check the MI355X rule in launcher.cpp.

Each (shape, rung) is timed as a captured HIP graph of `--chain` dependent
launches (graph edges serialize them and no host launch cost is counted),
replayed `--repeats` times back to back; one more replay into a cleared C is
compared bit for bit with an eager launch of the same rung.

    python -m shape_driven_tile_amd.sweep [--shapes 512,1024,...] [--out file.json]
    python -m shape_driven_tile_amd.sweep --splits 2,3,4,6,8 [--shapes ...]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

DEFAULT_SQUARES = (256, 512, 768, 1024, 1280, 1536, 1792, 2048, 2560, 3072, 3584, 4096,
                   6144, 8192)


def time_rung(sdt, torch, A, B, C, tile, stagger, chain, repeats, kgroups=-1, ws=None, **cfg):
    """Median microseconds per launch of rung `tile` over `repeats` back-to-back
    graph replays, all of them, and whether a replay into a cleared C
    reproduced the eager result bit for bit.  cfg: further sdt_launch fields
    (splits, split_algo, stages, persistent); ws: a binding.Workspace."""
    def launch():
        sdt.gemm_f16_cfg(A, B, C, tile_id=tile, kgroups=kgroups, stagger=stagger, workspace=ws,
                         **cfg)
    launch()
    torch.cuda.synchronize()
    eager = C.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(chain):
                launch()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    t_end = time.perf_counter() + 0.05      # ~50 ms of replays to settle the clocks
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(repeats)]
    for e0, e1 in ev:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    per_launch = sorted(1e3 * e0.elapsed_time(e1) / chain for e0, e1 in ev)
    C.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(C.view(torch.int16), eager.view(torch.int16)))
    return per_launch[len(per_launch) // 2], per_launch, same


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", default=None,
                    help="comma list of M=N=K squares, or MxNxK entries")
    ap.add_argument("--repeats", type=int, default=7)
    ap.add_argument("--out", default=None)
    ap.add_argument("--persistent", default=None,
                    help="comma list of persistent grid sizes (0 = one workgroup per tile): "
                         "instead of the rung sweep, time the ping-pong kernel with each")
    ap.add_argument("--splits", default=None,
                    help="comma list of k-split counts: instead of the rung sweep, time every "
                         "k-split rung with each count (both reductions, one and two k-groups)")
    args = ap.parse_args(argv)

    import torch

    from shape_driven_tile_amd import binding as sdt
    from shape_driven_tile_amd import inputs

    dev = torch.device("cuda:0")
    num_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    shapes = []
    for tok in (args.shapes.split(",") if args.shapes else [str(n) for n in DEFAULT_SQUARES]):
        if "x" in tok:
            m, n, k = (int(v) for v in tok.split("x"))
        else:
            m = n = k = int(tok)
        shapes.append((m, n, k))

    # warm the clocks
    wa, wb = inputs.square_operands(4096, 2)
    WA = torch.from_numpy(wa).to(dev)
    WB = torch.from_numpy(wb).to(dev)
    WC = torch.empty((4096, 4096), dtype=torch.float16, device=dev)
    for _ in range(200):
        sdt.gemm_f16_ex(WA, WB, WC)
    torch.cuda.synchronize()

    if args.splits:
        return split_sweep(sdt, torch, inputs, dev, num_cu, shapes,
                           [int(v) for v in args.splits.split(",")], args)
    if args.persistent:
        return persistent_sweep(sdt, torch, inputs, dev, num_cu, shapes,
                                [int(v) for v in args.persistent.split(",")], args)

    results = []
    for (M, N, K) in shapes:
        # Rows padded to a multiple of 8 elements (the library's 16-byte row
        # alignment), so any M, N, K can be swept.
        kp, np_ = -(-K // 8) * 8, -(-N // 8) * 8
        A = torch.zeros((M, kp), dtype=torch.float16, device=dev)[:, :K]
        B = torch.zeros((N, kp), dtype=torch.float16, device=dev)[:, :K]
        A.copy_(torch.from_numpy(inputs.uniform_f16((M, K), 11)))
        B.copy_(torch.from_numpy(inputs.uniform_f16((N, K), 12)))
        C = torch.empty((M, np_), dtype=torch.float16, device=dev)[:, :N]
        flop = 2.0 * M * N * K
        chain = max(4, min(400, int(2e12 / max(flop, 1.0))))
        auto = sdt.pick_tile(M, N, K, num_cu)["id"]
        row = {"M": M, "N": N, "K": K, "auto_tile": auto, "rungs": {}}
        for tile in range(sdt.num_tiles()):
            med, allv, same = time_rung(sdt, torch, A, B, C, tile, -1, chain, args.repeats)
            row["rungs"][tile] = {"us": round(med, 3), "tflops": round(flop / med / 1e6, 1),
                                  "min_us": round(allv[0], 3), "max_us": round(allv[-1], 3),
                                  "replays_match_eager": same}
        if sdt.stagger_eligible(K):
            row["stagger_arms"] = {}
            for st in (0, 1):
                med, allv, same = time_rung(sdt, torch, A, B, C, auto, st, chain, args.repeats)
                row["stagger_arms"][st] = {"us": round(med, 3), "min_us": round(allv[0], 3),
                                           "max_us": round(allv[-1], 3),
                                           "replays_match_eager": same}
        if sdt.tile_info(auto)["kgroups"] == 2:
            row["kgroup_arms"] = {}
            for kg in (1, 2):
                med, allv, same = time_rung(sdt, torch, A, B, C, auto, -1, chain, args.repeats, kg)
                row["kgroup_arms"][kg] = {"us": round(med, 3), "min_us": round(allv[0], 3),
                                          "max_us": round(allv[-1], 3),
                                          "replays_match_eager": same}
        best = min(row["rungs"], key=lambda t: row["rungs"][t]["us"])
        row["best_tile"] = best
        results.append(row)
        cells = "  ".join(f"t{t}:{v['us']:8.2f}" for t, v in row["rungs"].items())
        print(f"{M}x{N}x{K}: {cells}   best t{best}  auto t{auto}"
              f"{'' if all(v['replays_match_eager'] for v in row['rungs'].values()) else '  REPLAY MISMATCH'}",
              flush=True)
        if "kgroup_arms" in row:
            a = row["kgroup_arms"]
            print(f"    t{auto} one k-group {a[1]['us']:.2f}  two {a[2]['us']:.2f}"
                  f"  auto {sdt.pick_tile(M, N, K, num_cu)['kgroups']}", flush=True)
        if "stagger_arms" in row:
            a = row["stagger_arms"]
            print(f"    t{auto} stagger off {a[0]['us']:.2f} [{a[0]['min_us']:.2f}, {a[0]['max_us']:.2f}]"
                  f"  on {a[1]['us']:.2f} [{a[1]['min_us']:.2f}, {a[1]['max_us']:.2f}]"
                  , flush=True)
    out = {"num_cu": num_cu, "device": torch.cuda.get_device_properties(dev).name,
           "ladder": [sdt.tile_info(t) for t in range(sdt.num_tiles())], "shapes": results}
    if args.out:
        with open(args.out, "w") as f:
            json.dump(out, f, indent=1)
    ok = all(v["replays_match_eager"] for r in results
             for v in (list(r["rungs"].values()) + list(r.get("stagger_arms", {}).values())
                       + list(r.get("kgroup_arms", {}).values())))
    return 0 if ok else 1


def split_sweep(sdt, torch, inputs, dev, num_cu, shapes, split_counts, args):
    """The k-split arms: on every rung built to split K, each count in
    split_counts that leaves at least two full k-tiles per split, with the
    partials reduced by a second kernel (algo 0) or by each tile's last
    workgroup (algo 1), one k-group (2-stage and deep pipelines) and two;
    beside them the rung unsplit and the automatic plans of gemm_f16 and
    gemm_f16_ws."""
    ws = sdt.Workspace(256 << 20, device=dev)
    results = []
    for (M, N, K) in shapes:
        kp, np_ = -(-K // 8) * 8, -(-N // 8) * 8
        A = torch.zeros((M, kp), dtype=torch.float16, device=dev)[:, :K]
        B = torch.zeros((N, kp), dtype=torch.float16, device=dev)[:, :K]
        A.copy_(torch.from_numpy(inputs.uniform_f16((M, K), 11)))
        B.copy_(torch.from_numpy(inputs.uniform_f16((N, K), 12)))
        C = torch.empty((M, np_), dtype=torch.float16, device=dev)[:, :N]
        flop = 2.0 * M * N * K
        chain = max(4, min(400, int(2e12 / max(flop, 1.0))))
        row = {"M": M, "N": N, "K": K, "arms": {}}
        plain = sdt.pick_tile(M, N, K, num_cu)
        wsplan = sdt.pick_tile_ws(M, N, K, num_cu, ws.nbytes)
        med, allv, same = time_rung(sdt, torch, A, B, C, -1, -1, chain, args.repeats)
        row["arms"]["gemm_f16"] = {"us": round(med, 3), "min_us": round(allv[0], 3),
                                   "max_us": round(allv[-1], 3), "replays_match_eager": same,
                                   "plan": plain}
        med, allv, same = time_rung(sdt, torch, A, B, C, -1, -1, chain, args.repeats, ws=ws)
        row["arms"]["gemm_f16_ws"] = {"us": round(med, 3), "min_us": round(allv[0], 3),
                                      "max_us": round(allv[-1], 3), "replays_match_eager": same,
                                      "plan": wsplan}
        print(f"{M}x{N}x{K}: gemm_f16 {row['arms']['gemm_f16']['us']:.2f} "
              f"(t{plain['id']} s{plain['stages']} kg{plain['kgroups']})  gemm_f16_ws "
              f"{row['arms']['gemm_f16_ws']['us']:.2f} (t{wsplan['id']} splits {wsplan['splits']}"
              f" algo {wsplan['split_algo']} s{wsplan['stages']} kg{wsplan['kgroups']})", flush=True)
        for tile in range(sdt.num_tiles()):
            info = sdt.tile_info(tile)
            if not info["ksplit"]:
                continue
            pipes = [(2, 1), (info["stages"], 1), (info["stages"], 2)]
            for sp in [1] + [v for v in split_counts if v > 1 and (K // 64) // v >= 2]:
                for (stages, kg) in pipes:
                    for algo in ((0, 1) if sp > 1 else (0,)):
                        key = f"t{tile}_s{sp}_a{algo}_st{stages}_kg{kg}"
                        try:
                            med, allv, same = time_rung(sdt, torch, A, B, C, tile, 0, chain,
                                                        args.repeats, kgroups=kg, ws=ws,
                                                        splits=sp, split_algo=algo, stages=stages)
                        except sdt.SdtError as e:
                            row["arms"][key] = {"refused": str(e)}
                            continue
                        row["arms"][key] = {"us": round(med, 3), "min_us": round(allv[0], 3),
                                            "max_us": round(allv[-1], 3),
                                            "replays_match_eager": same}
        timed = [(k, v) for k, v in row["arms"].items() if "us" in v]
        for k, v in sorted(timed, key=lambda kv: kv[1]["us"]):
            print(f"    {k:28s} {v['us']:8.2f} [{v['min_us']:.2f}, {v['max_us']:.2f}]", flush=True)
        results.append(row)
        if args.out:
            with open(args.out, "w") as f:
                json.dump({"num_cu": num_cu, "shapes": results}, f, indent=1)
    out = {"num_cu": num_cu, "device": torch.cuda.get_device_properties(dev).name,
           "shapes": results}
    if args.out:
        with open(args.out, "w") as f:
            json.dump(out, f, indent=1)
    ok = all(v.get("replays_match_eager", True) for r in results for v in r["arms"].values())
    return 0 if ok else 1


def persistent_sweep(sdt, torch, inputs, dev, num_cu, shapes, grids, args):
    """The ping-pong kernel (rung 0's deep pipeline) with each persistent grid
    size that does not exceed the tile count (0: one workgroup per tile),
    graph-timed, in alternating rounds so that clock drift spreads over the
    arms alike."""
    results = []
    for (M, N, K) in shapes:
        kp, np_ = -(-K // 8) * 8, -(-N // 8) * 8
        A = torch.zeros((M, kp), dtype=torch.float16, device=dev)[:, :K]
        B = torch.zeros((N, kp), dtype=torch.float16, device=dev)[:, :K]
        A.copy_(torch.from_numpy(inputs.uniform_f16((M, K), 11)))
        B.copy_(torch.from_numpy(inputs.uniform_f16((N, K), 12)))
        C = torch.empty((M, np_), dtype=torch.float16, device=dev)[:, :N]
        flop = 2.0 * M * N * K
        chain = max(4, min(400, int(2e12 / max(flop, 1.0))))
        tiles = -(-M // 256) * -(-N // 256)
        arms = [g for g in grids if g <= tiles]
        row = {"M": M, "N": N, "K": K, "tiles": tiles, "arms": {}}
        samples = {g: [] for g in arms}
        same = True
        for _ in range(3):
            for g in arms:
                med, allv, ok = time_rung(sdt, torch, A, B, C, 0, -1, chain, args.repeats,
                                          kgroups=1, stages=3, persistent=g)
                samples[g] += allv
                same = same and ok
        for g in arms:
            v = sorted(samples[g])
            row["arms"][g] = {"us": round(v[len(v) // 2], 3), "min_us": round(v[0], 3),
                              "max_us": round(v[-1], 3)}
        row["replays_match_eager"] = same
        print(f"{M}x{N}x{K} ({tiles} tiles): " + "  ".join(
            f"P={g}: {row['arms'][g]['us']:.2f} [{row['arms'][g]['min_us']:.2f}, "
            f"{row['arms'][g]['max_us']:.2f}]" for g in arms), flush=True)
        results.append(row)
    if args.out:
        with open(args.out, "w") as f:
            json.dump({"num_cu": num_cu, "shapes": results}, f, indent=1)
    return 0 if all(r["replays_match_eager"] for r in results) else 1


if __name__ == "__main__":
    sys.exit(main())
