"""Benchmark: full DDTree hybrid verify step on one MI355X.

Workload (one "step" = one verify round over the whole hot path):
  8 sequences, budget B = 64 (65 tree rows), drafter depth L = 15, vocab 151936,
  committed prefix 32768 tokens; build the tree from bf16 drafter logits, 64 layers
  in the pattern [GDN, GDN, GDN, attention] x 16 (attention: 24 q / 4 kv heads,
  head_dim 256; GDN: 32 heads, dk = dv = 128, fp32 state, conv width 4 over 8192
  channels, bf16 activations), greedy walk against bf16 target logits, commit of
  the accepted path.  Inputs are seeded synthetic draws resident in HBM before the
  timed region; the bonus token of each round is the next round's root and every
  commit grows the prefix, as in decoding.

Output: one JSON line (metric, value = steps/s, per-kernel breakdown, roofline of
the dominant kernel, tree-attention KV bandwidth, CPU-oracle baseline).  The round
runs W + K times eagerly with HIP events around every call (the per-kernel breakdown
and the roofline come from those K rounds), then is captured once in a HIP graph and
replayed W + K times: `value` is the K timed replays, the same work without the
launch gaps between calls (every length is read on the device, so each replay is a
new round that continues from the state the previous one left).

    python bench.py [--steps K] [--warmup W] [--prefix P] [--no-cpu] [--no-variants] [--no-graph]
    python bench.py --kernel-configs      (per-config kernel figures, one JSON line each)
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix
KERNEL_SOURCES = {  # the sources whose kernels one call runs
    "gdn_tree_step": ("gdn_tree.hip", "gdn_chunk.hip"),
    "tree_attn": "tree_attn.hip",
    "build_tree": "build_tree.hip",
    "tree_accept": "accept.hip",
    "commit": "commit.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefix", type=int, default=32768)
    ap.add_argument("--n", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-graph", action="store_true",
                    help="take value from the eager rounds (no HIP graph capture; for profiler runs)")
    ap.add_argument("--kernel-configs", action="store_true",
                    help="instead of the step line: per-config kernel figures (tree build, tree attention at "
                         "8K/32K/128K, the full step at 16K), one JSON line each")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the variants (GDN replay on commit, RoPE in attention, paged KV with the sampled "
                         "walk) timed after the main measurement and reported under 'variants'")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times and exit (calibrates HBM byte counters)")
    return ap.parse_args()


def code_hash(text):
    """Hash of a kernel source's code: comments and white space are left out, so that an
    edit of a comment keeps the counter figures taken on the same code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def src_hash(name):
    files = KERNEL_SOURCES[name]
    files = (files,) if isinstance(files, str) else files
    return code_hash("\n".join(open(os.path.join(ROOT, "tree_speculative_decoding_ddt_amd", "csrc", f)).read()
                               for f in files))


def algorithmic(cfg, prefix_now, rows_per_round):
    """Algorithmic HBM bytes (and flops) per launch of each call, for the current prefix.
    rows_per_round: rows committed per round over all sequences (sum of acc_len + 1)."""
    n, T, V, L = cfg.n, cfg.T, cfg.V, cfg.L
    kv = n * cfg.Hkv * (prefix_now + T) * cfg.D * 2 * 2                  # K and V, bf16
    attn_io = 2 * n * T * cfg.Hq * cfg.D * 2                              # q in, out
    attn_flops = 4.0 * n * T * cfg.Hq * cfg.D * (prefix_now + T)           # QK^T + PV over all keys
    state = cfg.H * cfg.dk * cfg.dk * 4
    conv = (cfg.W - 1) * cfg.C * 2
    inputs = (n * state                                                   # committed S read
              + n * T * cfg.C * 2                                         # x read
              + n * conv                                                  # committed conv state read
              + 2 * n * T * cfg.H * cfg.dk * 2                            # v read, o written
              + 2 * n * T * cfg.H * 4)                                    # beta, g
    if cfg.replay:
        gdn = inputs                                                      # no node state stored
    else:
        gdn = inputs + n * T * state + n * T * conv                       # S and conv scratch written
    build = n * L * V * 2 + n * T * 24
    accept = n * T * V * (2 + 4 if cfg.sampled else 2)                    # (+ fp32 noise when sampled)
    kv_rows = cfg.n_attn * rows_per_round * cfg.Hkv * cfg.D * 2 * 2 * 2   # k, v rows read + written
    if cfg.replay:
        # replay: committed S and conv rows read + written, the path rows' x, v, beta, g read
        path = rows_per_round * (cfg.C * 2 + cfg.H * cfg.dk * 2 + cfg.H * 8)
        commit = kv_rows + cfg.n_gdn * (2 * n * state + 2 * n * conv + path)
    else:
        commit = kv_rows + cfg.n_gdn * 2 * n * (state + conv)             # deepest row's S, conv: read + written
    return {"tree_attn": (kv + attn_io, attn_flops), "gdn_tree_step": (gdn, 0.0),
            "build_tree": (build, 0.0), "tree_accept": (accept, 0.0), "commit": (int(commit), 0.0)}


def cpu_baseline(step, a):
    """The CPU oracle on sequence 0 of one round of the workload, all of it (tree build,
    the 16 attention and 48 GDN layers, the walk, the commit), on the very inputs the GPU
    reads at the start of that round (copied from the device before it; the copies and
    the fp64 conversions are not timed).  The GPU then runs the same round and its
    sequence-0 tree and walk are compared with the oracle's.  A step is n sequences, so
    the oracle's steps/s is 1 / (n x its time for one sequence)."""
    import numpy as np
    import torch

    from oracle import accept as oacc
    from oracle import attention as oattn
    from oracle import commit as ocommit
    from oracle import gdn as ogdn
    from oracle import tree as otree

    cfg, s = step.cfg, 0
    torch.cuda.synchronize(step.dev)
    f64 = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
    P = int(step.prefix_len[s])
    root = int(step.root_token[s])
    z = f64(step.draft_logits[s])
    y = f64(step.target_logits[s])
    # snapshot in the storage dtype (host copies, converted to fp64 one layer at a time)
    attn_in = [{k: lay[k][s].cpu() for k in ("q", "k_tree", "v_tree")} |
               {"k_cache": lay["k_cache"][s, :, :P].cpu(), "v_cache": lay["v_cache"][s, :, :P].cpu()}
               for lay in step.attn]
    gdn_in = [{k: lay[k][s].cpu() for k in ("x", "v", "beta", "g", "S", "conv_state")} | {"conv_w": lay["conv_w"].cpu()}
              for lay in step.gdn]
    # the GPU's own round on those inputs
    step()
    torch.cuda.synchronize(step.dev)
    gpu_tok, gpu_par = step.tree["tok"][s].cpu().numpy(), step.tree["parent"][s].cpu().numpy()
    gpu_rows = step.acc["acc_rows"][s].cpu().numpy()

    from threadpoolctl import threadpool_info
    blas = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
    t = {}
    t0 = time.perf_counter()
    tree = otree.build_tree(z, cfg.B, root)
    t["build"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    rows, acc, _ = oacc.tree_accept(y, tree["tok"], tree["parent"], cfg.L)
    t["walk"] = time.perf_counter() - t0
    path = [int(r) for r in rows[: acc + 1]]
    t["attn"] = t["gdn"] = t["commit"] = 0.0
    for lay in attn_in:
        x = {k: v.float().numpy().astype(np.float64) for k, v in lay.items()}
        t0 = time.perf_counter()
        oattn.tree_attention(x["q"], x["k_cache"], x["v_cache"], P, x["k_tree"], x["v_tree"], tree["anc"])
        t["attn"] += time.perf_counter() - t0
        cap = np.zeros((cfg.Hkv, P + acc + 1, cfg.D))
        kv = [dict(k_tree=x["k_tree"], v_tree=x["v_tree"], k_cache=np.concatenate([x["k_cache"], cap[:, P:]], 1),
                   v_cache=np.concatenate([x["v_cache"], cap[:, P:]], 1))]
        t0 = time.perf_counter()
        ocommit.commit(rows, acc, P, kv, [], P + acc + 1)
        t["commit"] += time.perf_counter() - t0
        del x, kv
    for lay in gdn_in:
        x = {k: v.float().numpy().astype(np.float64) for k, v in lay.items()}
        t0 = time.perf_counter()
        o, S_scr, c_scr = ogdn.gdn_tree_step(x["x"], x["conv_w"], x["conv_state"], x["v"], x["beta"], x["g"], x["S"],
                                             tree["parent"], cfg.H, cfg.dk)
        t["gdn"] += time.perf_counter() - t0
        gd = [dict(S_scratch=S_scr, S=x["S"], conv_scratch=c_scr, conv_state=x["conv_state"])]
        t0 = time.perf_counter()
        ocommit.commit(rows, acc, P, [], gd, P + acc + 1)
        t["commit"] += time.perf_counter() - t0
        del x, gd, S_scr
    per_seq = sum(t.values())
    agrees = bool(np.array_equal(gpu_tok, tree["tok"]) and np.array_equal(gpu_par, tree["parent"])
                  and np.array_equal(gpu_rows, rows))
    cores = len(os.sched_getaffinity(0))
    return {"value": 1.0 / (cfg.n * per_seq), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": ("sequence 0 of %d, whole round on the same inputs as the GPU round (copied from the device): "
                       "tree build %.2fs, %d attention layers at prefix %d %.2fs, %d GDN layers %.2fs, walk %.2fs, "
                       "commit %.2fs = %.1fs per sequence, 64 layers timed; step = %d sequences = %.1fs; numpy "
                       "fp64, BLAS threads %s, %d host cores"
                       % (cfg.n, t["build"], cfg.n_attn, P, t["attn"], cfg.n_gdn, t["gdn"], t["walk"], t["commit"],
                          per_seq, cfg.n, cfg.n * per_seq, blas, cores)),
            "blas_threads": blas[0] if blas else None, "cpu_model": cpu_model(),
            "agrees_with_gpu_round": agrees, "accepted_seq0": int(acc)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        return None


def kernel_configs(a):
    """Per-config kernel figures (tree build, tree attention at 8K/32K/128K, the full step at
    its 16K prefix): median of 50 calls after 10 warm-up calls, each timed call preceded by a
    512 MB write so that no input is served from the 256 MB last-level cache.  Prints one JSON
    line per measurement, fractions against the nominal HBM peak and against this GPU's own
    device-copy rate; for n = 1 the CPU oracle's time on the same shapes is given beside it
    (one sequence, float64 NumPy on every host core and, except at 131072, on one BLAS
    thread; skipped with --no-cpu)."""
    import numpy as np
    import torch

    from tree_speculative_decoding_ddt_amd import ddt, synth
    from tree_speculative_decoding_ddt_amd.step import HybridConfig, HybridVerifyStep

    dev = torch.device("cuda:0")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(a.seed)
    L, V, Hq, Hkv, D = 15, 151936, 24, 4, 256

    def cold(fn, reps=50, warm=10):
        for _ in range(warm):
            fn()
        ev = []
        for _ in range(reps):
            flush.fill_(1)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            ev.append((s, e))
        torch.cuda.synchronize(dev)
        return float(np.median([s.elapsed_time(e) for s, e in ev])) * 1e-3  # seconds

    def drafter(n):
        z = 3.0 * torch.randn(n, L, V, generator=gen, device=dev)
        hit = torch.rand(n, L, generator=gen, device=dev) < 0.6
        where = torch.randint(0, V, (n, L), generator=gen, device=dev)
        zz = z.view(-1, V)
        rows = torch.nonzero(hit.view(-1)).flatten()
        zz[rows, where.view(-1)[rows]] = z.amax(dim=-1).view(-1)[rows] + 8.0
        return z.bfloat16()

    def emit(rec):
        print(json.dumps(rec), flush=True)

    # the host and this GPU's own copy rate (a STREAM-style 1 GiB device-to-device copy,
    # bytes read + written), beside the nominal HBM peak
    emit({"config": "host", "cpu_model": cpu_model() or "?", "cpu_threads": len(os.sched_getaffinity(0))})
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(3)
    for _ in range(3):
        dst.copy_(src)
    cs, ce = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cs.record()
    for _ in range(10):
        dst.copy_(src)
    ce.record()
    torch.cuda.synchronize(dev)
    copy_gbps = 2 * src.numel() * 10 / (cs.elapsed_time(ce) * 1e-3) / 1e9
    # write-only stream (a device fill of the same 1 GiB): the rate a call that mostly
    # writes, like the GDN tree step with stored node states, compares against
    cs.record()
    for _ in range(10):
        dst.fill_(7)
    ce.record()
    torch.cuda.synchronize(dev)
    fill_gbps = dst.numel() * 10 / (cs.elapsed_time(ce) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    emit({"config": "device copy", "bytes_per_copy": 2 << 30, "GBps": round(copy_gbps, 1),
          "frac_of_nominal": round(copy_gbps / HBM_PEAK_GBPS, 4)})
    emit({"config": "device fill", "bytes_per_fill": 1 << 30, "GBps": round(fill_gbps, 1),
          "frac_of_nominal": round(fill_gbps / HBM_PEAK_GBPS, 4)})

    def cpu_baseline_seconds(kind, threads=None, **k):
        """The CPU oracle on one sequence of the config (the same workload shapes); threads
        limits the BLAS pool (None: every host core)."""
        if a.no_cpu:
            return None
        if threads is not None:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=threads):
                return cpu_baseline_seconds(kind, None, **k)
        from oracle import attention as oattn
        from oracle import tree as otree
        rng = np.random.default_rng(1)
        z = synth.quantize(synth.draft_logits(rng, 1, L, V, 3.0, plant_p=0.6), "bf16")[1][0]
        if kind == "build":
            t0 = time.perf_counter()
            otree.build_tree(z, k["B"], 0)
            return time.perf_counter() - t0
        P = k["P"]
        tree = otree.build_tree(z, 64, 0)
        anc = tree["anc"] if k["tree"] == "random" else k["anc"]
        x = synth.attention_inputs(rng, 1, 65, Hq, Hkv, D, P)
        x = {kk: synth.quantize(v, "bf16")[1][0] for kk, v in x.items()}
        t0 = time.perf_counter()
        oattn.tree_attention(x["q"], x["k_cache"], x["v_cache"], P, x["k_tree"], x["v_tree"], anc)
        return time.perf_counter() - t0

    # [1] tree build: n in {1, 16}, B in {32, 64}
    for n in (1, 16):
        z = drafter(n)
        root = torch.zeros(n, dtype=torch.int32, device=dev)
        for B in (32, 64):
            ws = torch.empty(ddt.build_tree_workspace(n, L, V, B), dtype=torch.uint8, device=dev)
            out = ddt.build_tree(z, B, root, ws=ws)
            t = cold(lambda: ddt.build_tree(z, B, root, ws=ws, out=out))
            nb = n * L * V * 2 + n * (B + 1) * 24
            oc = cpu_baseline_seconds("build", B=B) if n == 1 else None
            o1 = cpu_baseline_seconds("build", threads=1, B=B) if n == 1 else None
            emit({"config": "tree build", "n": n, "B": B, "L": L, "V": V, "us": round(t * 1e6, 1),
                  "GBps": round(nb / t / 1e9, 1), "hbm_frac": round(nb / t / 1e9 / HBM_PEAK_GBPS, 4),
                  "copy_frac": round(nb / t / 1e9 / copy_gbps, 4),
                  "cpu_oracle_s_per_seq": None if oc is None else round(oc, 3),
                  "cpu_oracle_s_per_seq_1thread": None if o1 is None else round(o1, 3)})
    # [2] tree attention (n in {1, 8}, P in {8192, 32768}) and [3] long context (n 1, P 131072, lopsided tree)
    cases = [(1, 8192, "random"), (8, 8192, "random"), (1, 32768, "random"), (8, 32768, "random"),
             (1, 131072, "lopsided")]
    for n, P, kind in cases:
        T = 65
        if kind == "random":
            tree = ddt.build_tree(drafter(n), 64, torch.zeros(n, dtype=torch.int32, device=dev))
            anc = tree["anc"]
        else:
            parent, _ = synth.lopsided_parents()
            m = [0] * T
            for i in range(1, T):
                m[i] = m[int(parent[i])] | (1 << (i - 1))
            anc = torch.tensor(np.array(m, dtype=np.uint64).view(np.int64), device=dev).view(1, T).repeat(n, 1)
        anc_np = None if kind == "random" else np.array(m, dtype=np.uint64)
        rn = lambda *sh: torch.randn(*sh, generator=gen, device=dev).bfloat16()
        q, kc, vc, kt, vt = rn(n, T, Hq, D), rn(n, Hkv, P, D), rn(n, Hkv, P, D), rn(n, Hkv, T, D), rn(n, Hkv, T, D)
        pl = torch.full((n,), P, dtype=torch.int32, device=dev)
        ws = torch.empty(max(ddt.tree_attn_workspace(n, T - 1, Hq, Hkv, D, P, torch.bfloat16), 16),
                         dtype=torch.uint8, device=dev)
        o = torch.empty_like(q)
        t = cold(lambda: ddt.tree_attn(q, kc, vc, pl, kt, vt, anc, ws=ws, out=o))
        kv = n * Hkv * (P + T) * D * 2 * 2
        fl = 4.0 * n * T * Hq * D * (P + T)
        del q, kc, vc, kt, vt, ws, o
        torch.cuda.empty_cache()
        oc = cpu_baseline_seconds("attn", P=P, tree=kind, anc=anc_np) if n == 1 else None
        o1 = cpu_baseline_seconds("attn", threads=1, P=P, tree=kind, anc=anc_np) if n == 1 and P < 131072 else None
        emit({"config": "tree attention" if P < 131072 else "long-context attention", "n": n, "P": P,
              "tree": kind, "us": round(t * 1e6, 1), "kv_GBps": round(kv / t / 1e9, 1),
              "kv_hbm_frac": round(kv / t / 1e9 / HBM_PEAK_GBPS, 4), "kv_copy_frac": round(kv / t / 1e9 / copy_gbps, 4),
              "TFLOPps": round(fl / t / 1e12, 1), "mfma_frac": round(fl / t / 1e12 / BF16_PEAK_TFLOPS, 4),
              "cpu_oracle_s_per_seq": None if oc is None else round(oc, 3),
              "cpu_oracle_s_per_seq_1thread": None if o1 is None else round(o1, 3)})
        torch.cuda.empty_cache()
    # [4] the full hybrid step at its own prefix, 16384
    cfg = HybridConfig(n=8, prefix=16384, extra_cap=(a.steps + a.warmup + 4) * 16 + 64)
    step = HybridVerifyStep(cfg, dev)
    step.fill_random(seed=a.seed)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize(dev)
    dt = (time.perf_counter() - t0) / a.steps
    emit({"config": "full hybrid verify step", "n": 8, "P": 16384, "steps_per_s": round(1.0 / dt, 3),
          "ms_per_step": round(dt * 1e3, 3)})


def load_traffic(name):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(name)
    if not rec or rec.get("source_sha") != src_hash(name):
        return None  # counters were taken on another version of the kernel
    return rec.get("bytes_per_launch")


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py runs on one GPU only: the verify step is measured on a single MI355X "
              "(requested --gpus %d)" % a.gpus, file=sys.stderr)
        return 2
    import torch

    if a.kernel_configs:
        kernel_configs(a)
        return 0

    if a.copy_probe:
        x = torch.empty(a.copy_probe << 20, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print("copied %d MiB x3" % a.copy_probe, file=sys.stderr)
        return 0

    from tree_speculative_decoding_ddt_amd import ddt
    from tree_speculative_decoding_ddt_amd.step import HybridConfig, HybridVerifyStep

    ddt.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # every round commits at most L + 1 = 16 rows: room for the main rounds, the CPU
    # leg's round and the two variants timed on this step object
    rounds = 3 * (2 * (a.warmup + a.steps) + 2) + 4
    cfg = HybridConfig(n=a.n, prefix=a.prefix, extra_cap=rounds * 16 + 64)
    step = HybridVerifyStep(cfg, dev)
    step.fill_random(seed=a.seed)
    print("bench: inputs ready (%.1f GB on device)" % (torch.cuda.memory_allocated(dev) / 1e9),
          file=sys.stderr, flush=True)

    names = ("build_tree", "tree_attn", "gdn_tree_step", "tree_accept", "commit")

    def measure(step, label):
        """W untimed + K timed eager rounds with HIP events around every call, then the
        round captured once in a HIP graph and replayed W + K times (the K replays give
        steps/s).  Returns the per-kernel table, the rates and the prefixes seen."""
        cfg = step.cfg
        ev = {k: [] for k in names}
        rows = torch.zeros((), dtype=torch.int64, device=dev)

        def timed(name, fn):
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record()
            fn()
            e_.record()
            ev[name].append((s_, e_))

        def attn_call(lay):
            if step.block_table is not None:
                return lambda: ddt.tree_attn_paged(lay["q"], lay["k_cache"], lay["v_cache"], step.block_table,
                                                   step.prefix_len, lay["k_tree"], lay["v_tree"], step.tree["anc"],
                                                   ws=step.ws_attn, out=lay["out"])
            if cfg.rope:
                return lambda: ddt.tree_attn_rope(lay["q"], lay["k_new"], lay["v_new"], step.tree["depth"],
                                                  cfg.rope[0], cfg.rope[1], lay["k_cache"], lay["v_cache"],
                                                  step.prefix_len, step.tree["anc"], ws=step.ws_attn,
                                                  out={"o": lay["out"], "k_tree": lay["k_tree"],
                                                       "v_tree": lay["v_tree"]})
            return lambda: ddt.tree_attn(lay["q"], lay["k_cache"], lay["v_cache"], step.prefix_len, lay["k_tree"],
                                         lay["v_tree"], step.tree["anc"], ws=step.ws_attn, out=lay["out"])

        def run_round():
            timed("build_tree", step.build)
            ia = ig = 0
            for kind in step.pattern:
                if kind == "attn":
                    lay = step.attn[ia]
                    ia += 1
                    timed("tree_attn", attn_call(lay))
                else:
                    g = step.gdn[ig]
                    ig += 1
                    timed("gdn_tree_step", lambda: ddt.gdn_tree_step(
                        g["x"], g["conv_w"], g["conv_state"], g["v"], g["beta"], g["g"], g["S"],
                        step.tree["parent"], cfg.L, ws=step.ws_gdn, out=g["out"], store_states=not cfg.replay))
            timed("tree_accept", step.accept)
            timed("commit", step.commit)
            rows.add_((step.acc["acc_len"].clamp(min=-1) + 1).sum())   # rows this round committed

        for _ in range(a.warmup):
            step()
        torch.cuda.synchronize(dev)
        p0 = int(step.prefix_len.float().mean().item())
        t0 = time.perf_counter()
        for _ in range(a.steps):
            run_round()
        torch.cuda.synchronize(dev)
        dt = time.perf_counter() - t0
        p1 = int(step.prefix_len.float().mean().item())
        rows_per_round = float(rows.item()) / a.steps

        # The same round captured once in a HIP graph and replayed (every length is read on
        # the device, so a replay continues from the state the previous round left): the
        # launch gaps of the eager rounds drop out, the work is identical.
        dtg, p2 = None, p1
        if not a.no_graph:
            try:
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    step()
            except RuntimeError as exc:  # capture refused: report the eager rounds instead
                print("bench: %s: HIP graph capture failed (%s); eager rounds only" % (label, exc),
                      file=sys.stderr, flush=True)
                graph = None
                torch.cuda.synchronize(dev)
            if graph is not None:
                for _ in range(a.warmup):
                    graph.replay()
                torch.cuda.synchronize(dev)
                tg = time.perf_counter()
                for _ in range(a.steps):
                    graph.replay()
                torch.cuda.synchronize(dev)
                dtg = time.perf_counter() - tg
                p2 = int(step.prefix_len.float().mean().item())
                del graph

        alg = algorithmic(cfg, (p0 + p1) // 2, rows_per_round)
        kernels = {}
        for k in names:
            ms = [s_.elapsed_time(e_) for s_, e_ in ev[k]]
            per = sum(ms) / len(ms)
            rec = {"ms_per_launch": round(per, 4), "launches_per_step": len(ms) // a.steps,
                   "ms_per_step": round(sum(ms) / a.steps, 4)}
            b, fl = alg[k]
            rec["algorithmic_bytes"] = b
            rec["GBps"] = round(b / (per * 1e-3) / 1e9, 1)
            rec["hbm_frac"] = round(rec["GBps"] / HBM_PEAK_GBPS, 4)
            if fl:
                rec["TFLOPps"] = round(fl / (per * 1e-3) / 1e12, 1)
                rec["mfma_frac"] = round(rec["TFLOPps"] / BF16_PEAK_TFLOPS, 4)
            kernels[k] = rec
        kernels["commit"]["rows_committed_per_round"] = round(rows_per_round, 2)
        dom = max(("gdn_tree_step", "tree_attn", "build_tree", "tree_accept"),
                  key=lambda k: kernels[k]["ms_per_step"])
        kd = kernels[dom]
        if dom == "tree_attn":
            roof = {"bound": "mfma", "achieved": kd["TFLOPps"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": kd["mfma_frac"]}
        else:
            roof = {"bound": "hbm", "achieved": kd["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": kd["hbm_frac"]}
        roof["kernel"] = dom
        ka = kernels["tree_attn"]
        kv_bytes = cfg.n * cfg.Hkv * ((p0 + p1) // 2 + cfg.T) * cfg.D * 4
        attn = {"kv_bytes_per_launch": kv_bytes,
                "kv_GBps": round(kv_bytes / (ka["ms_per_launch"] * 1e-3) / 1e9, 1),
                "kv_frac_of_hbm_peak": round(kv_bytes / (ka["ms_per_launch"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "TFLOPps": ka.get("TFLOPps"), "mfma_frac": ka.get("mfma_frac")}
        return {"kernels": kernels, "roofline": roof, "tree_attn": attn, "dt_eager": dt, "dt_graph": dtg,
                "prefix": (p0, p1, p2), "mean_accepted": float(step.acc["acc_len"].float().mean().item())}

    main = measure(step, "main")
    main["roofline"]["traffic"] = load_traffic(main["roofline"]["kernel"])

    cpu = None
    if not a.no_cpu:
        print("bench: timing the CPU oracle on one whole sequence of a round (same inputs)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(step, a)

    # Variants of the same step (the next rows of the path), each measured like the main
    # step: the GDN tree step storing no node state with the commit replaying the accepted
    # path; that plus RoPE at prefix + depth inside the attention call (pre-rotation q and
    # tree K/V in; rotate-half over all 256 channels, theta 10000); and, on a fresh step
    # object, the committed KV in pages of 16 positions scattered over a pool with the walk
    # over sampled target tokens (temperature 1, noise drawn once).
    variant = None
    if not a.no_variants:
        variant = {}

        def record(vname, m):
            variant[vname] = {
                "steps_per_s": round(a.steps / (m["dt_graph"] or m["dt_eager"]), 3),
                "ms_per_step": round((m["dt_graph"] or m["dt_eager"]) / a.steps * 1e3, 3),
                "eager_steps_per_s": round(a.steps / m["dt_eager"], 3),
                "kernels": m["kernels"], "roofline": m["roofline"], "mean_accepted": round(m["mean_accepted"], 3)}

        for vname, mode in (("gdn_replay_on_commit", dict(replay=True)),
                            ("gdn_replay_and_rope_attention", dict(replay=True, rope=(cfg.D, 10000.0)))):
            step.set_mode(**mode)
            record(vname, measure(step, vname))
        step = None
        torch.cuda.empty_cache()
        vcfg = HybridConfig(n=a.n, prefix=a.prefix, extra_cap=rounds * 16 + 64, replay=True, page_size=16,
                            sampled=True)
        step = HybridVerifyStep(vcfg, dev)
        step.fill_random(seed=a.seed)
        record("paged16_gdn_replay_sampled_walk", measure(step, "paged"))

    dtg = main["dt_graph"]
    value = a.steps / (dtg or main["dt_eager"])
    p0, p1, p2 = main["prefix"]
    line = {
        "metric": "tree-verify steps/sec at B=64, 32K prefix; tree-attn KV GB/s vs HBM peak",
        "value": round(value, 3), "unit": "steps/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round((dtg or main["dt_eager"]) / a.steps * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded device RNG draws)",
        "config": {"workload": "full hybrid verify step: 8 seqs, B=64, L=15, vocab 151936, prefix %d, "
                               "16 attn (24/4 heads, D 256) + 48 GDN (32 heads, dk=dv=128, C 8192, W 4) layers"
                               % a.prefix,
                   "global_batch": cfg.n, "seq_len": a.prefix, "parallelism": "single GPU"},
        "roofline": main["roofline"], "tree_attn": main["tree_attn"], "kernels": main["kernels"],
        "timing": ("value and kernels: HIP events per call over K eager rounds" if dtg is None else
                   "value: K replays of one round captured in a HIP graph; kernels: HIP events per call "
                   "over K eager rounds run before it (the same work, launched one call at a time)"),
        "eager": {"steps_per_s": round(a.steps / main["dt_eager"], 3),
                  "ms_per_step": round(main["dt_eager"] / a.steps * 1e3, 3), "prefix_during_timing": [p0, p1]},
        "mean_accepted": round(main["mean_accepted"], 3),
        "prefix_during_timing": [p1, p2] if dtg is not None else [p0, p1],
        "cpu_baseline": cpu, "variants": variant,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
