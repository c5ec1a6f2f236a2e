"""Benchmark of the Engram lookup hot path on one MI355X.

One step = the whole path over one batch: engram_hash (48 addresses per
token) then engram_gather_reduce (48 FP8 rows -> two fp32 vectors of 256 per
token).  Workload: 1 sequence of 131,072 Zipf(1.1) ids over a 129,280-id
vocabulary, 48 sub-tables x 2^24 rows x 256 B FP8 E4M3 (192 GiB) plus fp32
row scales, resident in HBM and filled on the device from a seeded
generator.  Inputs are resident before the timed region starts.

Prints one JSON line.  Extra figures ride in that line: the roofline of the
gather kernel (algorithmic bytes over its HIP-event time, and the bytes the
request-size counters saw leave L2), two control timings of the gather
(uniform ids, caches flushed), the same step as one fused launch and under
HIP-graph replay, memory-ceiling probes, and the CPU oracle timed on whole
workloads with one process and with the host's cores.
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
BYTES_PER_TOKEN = {  # algorithmic bytes of engram_gather_reduce per token
    "rows": 48 * 256, "scales": 48 * 4, "addresses": 48 * 4, "output": 2 * 256 * 4}
GATHER_BYTES_PER_TOKEN = sum(BYTES_PER_TOKEN.values())  # 14,720
HASH_BYTES_PER_TOKEN = 4 + 48 * 4  # id in, addresses out
MAX_CPU_WORKERS = 16  # a GPU's share of the host's cores
WORKLOAD_TEXT = {
    1: "tiny: 1 x 512 uniform ids in [0, 1024); 48 sub-tables x 4096 rows x 256 B FP8 E4M3 + fp32 row scales",
    2: ("decode: 64 sequences x 1 new token against a 3-token history, Zipf(1.1) ids over 129280; 48 sub-tables x "
        "2^20 rows x 256 B FP8 E4M3 (12 GiB) + fp32 row scales"),
    3: ("prefill: 1 x 32768 Zipf(1.1) ids over 129280; 48 sub-tables x 2^22 rows x 256 B FP8 E4M3 (48 GiB) + fp32 "
        "row scales"),
    4: ("full-size prefill: 1 x 131072 Zipf(1.1) ids over 129280; 48 sub-tables x 2^24 rows x 256 B FP8 E4M3 "
        "(192 GiB) + fp32 row scales, resident in HBM"),
    5: ("batched prefill with shared prefixes: 64 x (4096 shared + 4096 own) Zipf(1.1) ids over 129280; 48 "
        "sub-tables x 2^24 rows x 256 B FP8 E4M3 (192 GiB) + fp32 row scales"),
}
CSRC = os.path.join(ROOT, "hashed_gram_memory_amd", "csrc")
# Counter summaries of the timed gather kernel, per workload, each valid only for the exact code it was taken on:
# the file and the sources that kernel is compiled from.
PMC_RECORDS = {
    (4, "direct"): (os.path.join(ROOT, "profiles", "gather_reduce_full_131072_pmc.json"),
                    [os.path.join(CSRC, f) for f in ("gather_reduce.hip", "row_sum.h", "engram_internal.h")]),
    (5, "direct"): (os.path.join(ROOT, "profiles", "gather_batched_524288_pmc.json"),
                    [os.path.join(CSRC, f) for f in ("gather_batched.hip", "batch_order.h", "row_sum.h",
                                                     "engram_internal.h")]),
    (5, "dedup"): (os.path.join(ROOT, "profiles", "lookup_dedup_524288_pmc.json"),
                   [os.path.join(CSRC, f) for f in ("lookup.hip", "batch_order.h", "row_sum.h", "engram_internal.h")]),
}


def source_sha256(srcs) -> str:
    """sha256 of a kernel's code: its sources with // comments, blank lines and indentation removed, so that
    editing a comment does not detach the stored counters from the kernel they were taken on."""
    h = hashlib.sha256()
    for f in srcs:
        for line in open(f, encoding="utf-8"):
            code = line.split("//", 1)[0].strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def gather_source_sha256() -> str:
    """The code hash of the flat gather (workload 4's timed kernel)."""
    return source_sha256(PMC_RECORDS[(4, "direct")][1])


def _log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _pmc_record(key, n_tok: int, id_batches: int):
    """The committed counter summary of the timed kernel of (workload, step kind), if it matches the current kernel
    and run."""
    if key not in PMC_RECORDS:
        return None
    path, srcs = PMC_RECORDS[key]
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if (rec.get("kernel_source_sha256") != source_sha256(srcs) or rec.get("n_tok") != n_tok
            or rec.get("id_batches") != id_batches):
        return None
    return rec


def _traffic(key, n_tok: int, id_batches: int):
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE scaled by the copy calibration, when recorded."""
    rec = _pmc_record(key, n_tok, id_batches)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def _traffic_exact(key, n_tok: int, id_batches: int):
    """Bytes per launch leaving L2 from the request-size counters (128- and 64-byte reads) and WRITE_SIZE, under the
    same kernel and run checks."""
    rec = _pmc_record(key, n_tok, id_batches)
    return None if rec is None else rec.get("request_sizes", {}).get("bytes_exact")


def _oracle_worker(pieces, rows: int, seed: int, dense: bool, barrier, queue) -> None:
    """One CPU worker (a spawned process that never touches the GPU): the oracle over its pieces of the workload.

    Untimed preparation: the host tables (dense for small row counts; otherwise a lazily committed full-size
    mapping with only the rows its tokens read filled in).  Timed, after every worker is ready: windows, hash
    and gather-reduce of each piece."""
    import oracle
    import workloads

    mult = oracle.multipliers()
    rows48 = [rows] * 48
    host = None
    try:
        if dense:
            tabs, scs = workloads.dense_tables(seed, rows)
        else:
            host = workloads.SparseHostTables(seed, rows)
            for ids, hist in pieces:
                host.materialise(oracle.hash_addresses(oracle.windows(ids, hist), mult, rows48))
            tabs, scs = host.tables, host.scales
        barrier.wait()
        t0 = time.perf_counter()
        n = 0
        for ids, hist in pieces:
            a = oracle.hash_addresses(oracle.windows(ids, hist), mult, rows48)
            oracle.gather_reduce(tabs, scs, a)
            n += ids.size
        t1 = time.perf_counter()
        queue.put((t0, t1, n))
    except Exception as e:  # report instead of leaving the parent waiting
        queue.put(("error", repr(e), 0))
        barrier.abort()
    finally:
        if host is not None:
            host.close()


def _split_tokens(ids, hist, workers: int):
    """Token pieces for ``workers`` processes: whole sequences when there are enough of them, else contiguous
    chunks of each sequence, each carrying the 3 ids before it as its history (pad 0 at the sequence start)."""
    n_seq, seq_len = ids.shape
    if n_seq >= workers:
        b = np.linspace(0, n_seq, workers + 1).astype(int)
        return [[(ids[lo:hi], None if hist is None else hist[lo:hi])] for lo, hi in zip(b[:-1], b[1:]) if hi > lo]
    per = [[] for _ in range(workers)]
    for s in range(n_seq):
        pad = hist[s] if hist is not None else np.zeros(3, np.int32)
        ext = np.concatenate([pad, ids[s]]).astype(np.int32)  # ext[3 + p] is position p
        b = np.linspace(0, seq_len, workers + 1).astype(int)
        for w, (lo, hi) in enumerate(zip(b[:-1], b[1:])):
            if hi > lo:
                per[w].append((np.ascontiguousarray(ids[s:s + 1, lo:hi]), np.ascontiguousarray(ext[lo:lo + 3][None])))
    return [p for p in per if p]


def _time_oracle(ids, hist, rows: int, seed: int, workers: int) -> dict:
    import multiprocessing as mp

    ctx = mp.get_context("spawn")  # fresh interpreters: nothing of this process's GPU state is inherited
    parts = _split_tokens(ids, hist, workers)
    barrier, queue = ctx.Barrier(len(parts)), ctx.Queue()
    dense = rows <= 4096
    procs = [ctx.Process(target=_oracle_worker, args=(p, rows, seed, dense, barrier, queue)) for p in parts]
    for p in procs:
        p.start()
    res = [queue.get(timeout=600) for _ in procs]
    for p in procs:
        p.join(timeout=60)
    errors = [r for r in res if r[0] == "error"]
    if errors:
        raise RuntimeError(f"oracle worker failed: {errors[0][1]}")
    wall = max(r[1] for r in res) - min(r[0] for r in res)
    n = sum(r[2] for r in res)
    return {"tokens": n, "seconds": wall, "tokens_per_s": n / wall, "processes": len(parts)}


def cpu_baseline(keys, workers: int, tokens4: int) -> dict:
    """The CPU oracle (numpy, float64) on whole workloads, timed with 1 process and with ``workers`` processes that
    split the tokens.  Workload 4 is limited to its first ``tokens4`` tokens."""
    import workloads

    per = {}
    for key in keys:
        w = workloads.WORKLOADS[key]
        ids, hist = workloads.make_ids(w)
        if key == 4:
            ids = np.ascontiguousarray(ids[:, :tokens4])
        _log(f"cpu baseline: oracle on the {w.name} workload ({ids.size} tokens), 1 and {workers} processes")
        one = _time_oracle(ids, hist, w.rows, w.table_seed, 1)
        many = _time_oracle(ids, hist, w.rows, w.table_seed, workers)
        per[str(key)] = {"tokens": int(ids.size), "rows_per_subtable": w.rows, "cores_1": one, "cores_all": many}
    head = per.get("4") or per[str(keys[-1])]
    return {
        "value": head["cores_all"]["tokens_per_s"],
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "cores_1": head["cores_1"]["tokens_per_s"],
        "cores_all": head["cores_all"]["tokens_per_s"],
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "per_workload": per,
        "sample": (f"workload {'4' if '4' in per else keys[-1]}, {head['tokens']} tokens: oracle windows + hash + "
                   f"gather-reduce (numpy, float64) against host tables (full size; only the rows read are "
                   f"resident), tokens split over {workers} spawned processes (value) and in 1 process (cores_1); "
                   f"workloads {', '.join(per)} in per_workload, whole inputs"
                   + (f" (workload 4: first {tokens4} tokens)" if '4' in per else "")),
    }


def _median_ms(torch, fn, stream, reps: int) -> float:
    fn()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b))
    return float(np.median(times))


def measure_ceiling(hg, torch, plan, tables, addr, out, stream):
    """What the memory system delivers on this device: streaming read and copy, and the gather without scales."""
    flat = tables.view(-1)
    read_bytes = min(8 << 30, flat.numel())
    sink = torch.zeros(1, dtype=torch.int32, device=tables.device)
    t_read = _median_ms(torch, lambda: hg.probe_read(flat[:read_bytes], sink, stream=stream), stream, 5)
    copy_bytes = 2 << 30
    dst = torch.empty(copy_bytes, dtype=torch.uint8, device=tables.device)
    t_copy = _median_ms(torch, lambda: hg.probe_copy(flat[:copy_bytes], dst, stream=stream), stream, 5)
    del dst
    n_tok = addr.shape[0]
    t_rows = _median_ms(torch, lambda: hg.probe_rows(plan, addr, out, stream=stream), stream, 10)
    rows_bytes = n_tok * (48 * 256 + 48 * 4 + 2 * 256 * 4)
    rand = {}
    random_bytes = 2 << 30
    for chunk in (256, 512, 1024):
        t = _median_ms(torch, lambda: hg.probe_random(flat, chunk, random_bytes, sink, stream=stream), stream, 5)
        rand[f"random_{chunk}B_read_GBps"] = random_bytes / (t / 1e3) / 1e9
    # the same random-row gather-sum with the row scales in four places: what DRAM charges per row
    layouts = {}
    for name in hg.PROBE_RECORD_LAYOUTS:
        t = _median_ms(torch, lambda: hg.probe_records(flat, name, out, stream=stream), stream, 5)
        layouts[name] = t * 1e3
    return {
        "stream_read_GBps": read_bytes / (t_read / 1e3) / 1e9,
        "stream_copy_GBps": 2 * copy_bytes / (t_copy / 1e3) / 1e9,
        **rand,
        "random_rows_us": layouts,
        "gather_rows_only_us": t_rows * 1e3,
        "gather_rows_only_GBps": rows_bytes / (t_rows / 1e3) / 1e9,
    }


def measure_controls(hg, torch, workloads, plan, w, batches, addr, out, stream, seq_len: int, gather_bytes: int,
                     launches: int = 20, flush_mib: int = 1024) -> dict:
    """Two control timings of engram_gather_reduce (HIP events around each launch, mean over the launches).

    uniform_ids: 4 batches of ids uniform over the vocabulary, hashed ahead, gathered in turn: no Zipf row reuse.
    flushed: the workload's own batches, with a 1 GiB read between launches, so every launch starts with L2
    and the MALL holding none of the rows it reads."""
    dev = addr.device
    uni = []
    for b in range(4):
        ids = np.ascontiguousarray(workloads.uniform_ids(w.n_seq, w.seq_len, w.token_seed + 9000 + b)[:, :seq_len])
        a = torch.empty_like(addr)
        hg.hash(plan, torch.from_numpy(ids).to(dev), None, out=a, stream=stream)
        uni.append(a)
    for a in uni:  # warm-up
        hg.gather_reduce(plan, a, out=out, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        hg.gather_reduce(plan, uni[i % 4], out=out, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    t_uni = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    del uni
    flush = torch.ones(flush_mib << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros((), dtype=torch.uint8, device=dev)
    for i, (e0, e1) in enumerate(ev):
        b = batches[i % len(batches)]
        hg.hash(plan, b[1], b[2], out=addr, stream=stream)
        sink.copy_(flush.max())
        e0.record(stream)
        hg.gather_reduce(plan, addr, out=out, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    t_flush = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    del flush

    def rec(t_ms, what):
        gbps = gather_bytes / (t_ms / 1e3) / 1e9
        return {"gather_us": t_ms * 1e3, "achieved_GBps": gbps, "frac": gbps / HBM_PEAK_GBPS, "ids": what}

    return {"launches": launches,
            "uniform_ids": rec(t_uni, "4 batches uniform over 129280, hashed ahead, gathered in turn"),
            "flushed": rec(t_flush, f"the workload's batches with a {flush_mib} MiB read before every launch")}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000,
                    help="timed steps (5000 on the default workload: about 2 s of GPU work, long enough for a "
                         "utilisation sampler to see it)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-sample", type=int, default=131072,
                    help="tokens of the full workload (1 x 131,072 tokens, 2^24-row tables) the CPU oracle baseline takes "
                         "(0: skip the baseline)")
    ap.add_argument("--cpu-workloads", default="1,2,3,4",
                    help="workload keys (1 tiny, 2 decode, 3 prefill, 4 full) the CPU oracle baseline times, with 1 process "
                         "and with all cores")
    ap.add_argument("--pipeline", action="store_true",
                    help="hash (and dedup) the next batch on other streams while the current one is gathered, instead "
                         "of running each step in order on one stream (measured: helps only the dedup step, ~2%%)")
    ap.add_argument("--no-controls", action="store_true",
                    help="skip the uniform-id and cache-flushed control timings of the gather")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="synthetic workload: 1 tiny (512 tokens), 2 decode (64 x 1), 3 prefill (32,768), 4 full (131,072 tokens over 48 x 2^24-row tables, the default), 5 batched (64 x 8,192 sharing a 4,096-token prefix)")
    ap.add_argument("--dedup", action="store_true",
                    help="batched workloads: engram_dedup + engram_lookup_dedup (one hash and gather per group)")
    ap.add_argument("--dedup-two-call", action="store_true",
                    help="with --dedup: engram_hash + engram_dedup + engram_gather_reduce in dedup mode instead")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the memory-ceiling probes")
    ap.add_argument("--scale-format", default="f32_row", choices=["f32_row", "e8m0_block32"],
                    help="row scales: one fp32 per row, or 8 E8M0 bytes per row (one per 32 elements)")
    ap.add_argument("--vocab-map", action="store_true",
                    help="normalise window ids through a seeded 129,280 -> 99,092 vocabulary map before hashing")
    ap.add_argument("--prime-rows", action="store_true",
                    help="per-sub-table prime row counts (the 48 largest primes below the workload's row count)")
    ap.add_argument("--uniform-ids", action="store_true",
                    help="control run: ids uniform over the vocabulary instead of Zipf (no row reuse)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="read this many MiB of scratch before every timed step (evicts L2 and MALL without leaving "
                         "dirty lines; outside the per-kernel event pairs)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="use only the first N positions of every sequence (tokens per call = sequences x N), against "
                         "the workload's full-size tables; 0: the whole workload")
    ap.add_argument("--id-batches", type=int, default=4,
                    help="rotate among this many seeded id batches of the same shape; the first is the workload's own "
                         "ids.  Rotation keeps a step from reading rows the previous step left in the caches (1: "
                         "replay the same batch)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the lookup needs no collective and the library runs on a "
              "single MI355X; multi-GPU sharding is described in the design notes, not run.", file=sys.stderr)
        return 2

    import torch

    import hashed_gram_memory_amd as hg
    import workloads

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seq_len = w.seq_len if args.tokens <= 0 else min(args.tokens, w.seq_len)
    n_tok = w.n_seq * seq_len

    _log(f"allocating 48 x {w.rows} x 256 B tables")
    tables = torch.empty((48, w.rows, 256), dtype=torch.uint8, device=dev)
    mx = args.scale_format == "e8m0_block32"
    if mx:
        scales = torch.empty((48, w.rows, 8), dtype=torch.uint8, device=dev)
    else:
        scales = torch.empty((48, w.rows), dtype=torch.float32, device=dev)
    vocab = workloads.VOCAB if w.ids_kind != "uniform1024" else 1024
    d_map = torch.from_numpy(workloads.vocab_map(7).view(np.int32)).to(dev) if args.vocab_map else None
    if args.prime_rows:
        rows = workloads.prime_rows(48, below=w.rows)
        tab_list = [tables[s, :rows[s]] for s in range(48)]
        sc_list = [scales[s, :rows[s]] for s in range(48)]
    else:
        tab_list, sc_list = list(tables.unbind(0)), list(scales.unbind(0))
    hg.synth_fill(tab_list, sc_list, w.table_seed, scale_format=args.scale_format)
    torch.cuda.synchronize()
    plan = hg.Plan(tab_list, sc_list, vocab_size=vocab, scale_format=args.scale_format, vocab_map=d_map)

    batches = []
    for b in range(args.id_batches):
        if args.uniform_ids:
            ids, hist = workloads.uniform_ids(w.n_seq, w.seq_len, w.token_seed + 100 * b), None
            if w.history:
                hist = workloads.uniform_ids(w.n_seq, 3, w.token_seed + 100 * b + 1)
        else:
            ids, hist = workloads.make_ids(w, None if b == 0 else w.token_seed + 100 * b)
        ids = np.ascontiguousarray(ids[:, :seq_len])
        batches.append((ids, torch.from_numpy(ids).to(dev), None if hist is None else torch.from_numpy(hist).to(dev)))
    addr = torch.empty((n_tok, 48), dtype=torch.uint32, device=dev)
    out = torch.empty((n_tok, 2, 256), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    groups = ws = None

    def new_groups():
        return hg.Groups(torch.empty(n_tok, dtype=torch.int32, device=dev),
                         torch.empty(n_tok + 1, dtype=torch.int32, device=dev),
                         torch.empty(1, dtype=torch.int32, device=dev))

    # two buffers of addresses (and groups): batch i's lookup inputs live in buffer i % 2
    addr_bufs = [addr, torch.empty_like(addr)]
    group_bufs = [None, None]
    if args.dedup:
        group_bufs = [new_groups(), new_groups()]
        groups = group_bufs[0]
        ws = torch.empty(hg.dedup_workspace_bytes(plan, n_tok), dtype=torch.uint8, device=dev)
    s_hash = torch.cuda.Stream()  # default priority
    s_dedup = torch.cuda.Stream() if args.dedup else None

    # a batch of sequences is gathered in the batch order (engram_gather_reduce_batched): same results, and
    # sequences that share a prefix read it from L2
    batched = not args.dedup and w.n_seq > 1
    # dedup step: the fused lookup over the groups (no address buffer, no hash launch), or hash + dedup-mode gather
    fused_dedup = args.dedup and not args.dedup_two_call

    def gather_into(k, stream=None, b=None):
        if batched:
            hg.gather_reduce_batched(plan, addr_bufs[k], w.n_seq, out=out, stream=stream)
        elif fused_dedup:
            b = batches[0] if b is None else b
            hg.lookup(plan, b[1], b[2], out=out, groups=group_bufs[k], stream=stream)
        else:
            hg.gather_reduce(plan, addr_bufs[k], out=out, groups=group_bufs[k], stream=stream)

    def gather(stream=None):
        gather_into(0, stream)

    flush = torch.ones(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib > 0 else None
    flush_sink = torch.zeros((), dtype=torch.uint8, device=dev)

    def run_steps(n: int, pipelined: bool, ev=None, stages: bool = False) -> None:
        """n steps.  Step i hashes (and groups) batch i into buffer i % 2, then gathers that buffer.  Pipelined, the
        hash and dedup of batch i + 1 run on side streams while batch i is gathered -- they depend on the ids
        alone -- and wait only for the gather that last read their buffer; serial, everything runs in order on one
        stream.  ev[i] = 6 events around step i's hash, dedup and gather; only the gather's pair is recorded unless
        ``stages`` (each recorded pair adds a few us of queue work to the step)."""
        stage_ev = ev if stages else None
        freed = [torch.cuda.Event(), torch.cuda.Event()]  # the gather that last read buffer k has finished

        def produce(i):
            k, b = i % 2, batches[i % len(batches)]
            hs = s_hash if pipelined else stream
            if pipelined:
                hs.wait_event(freed[k])
            done = []
            if not fused_dedup:
                if stage_ev:
                    stage_ev[i][0].record(hs)
                hg.hash(plan, b[1], b[2], out=addr_bufs[k], stream=hs)
                if stage_ev:
                    stage_ev[i][1].record(hs)
                if pipelined:
                    done.append(torch.cuda.Event())
                    done[-1].record(hs)
            if args.dedup:
                ds = s_dedup if pipelined else stream
                if pipelined:
                    ds.wait_event(freed[k])
                if stage_ev:
                    stage_ev[i][2].record(ds)
                hg.dedup(plan, b[1], b[2], workspace=ws, groups=group_bufs[k], stream=ds)
                if stage_ev:
                    stage_ev[i][3].record(ds)
                if pipelined:
                    done.append(torch.cuda.Event())
                    done[-1].record(ds)
            return done

        def consume(i, done):
            k, b = i % 2, batches[i % len(batches)]
            for e in done:
                stream.wait_event(e)
            if flush is not None:
                flush_sink.copy_(flush.max())
            if ev:
                ev[i][4].record(stream)
            gather_into(k, stream, b)
            if ev:
                ev[i][5].record(stream)
            if pipelined:
                freed[k].record(stream)

        if pipelined:
            done = produce(0)
            for i in range(n):
                consume(i, done)
                if i + 1 < n:
                    done = produce(i + 1)
        else:
            for i in range(n):
                consume(i, produce(i))

    pipelined = args.pipeline
    _log(f"warmup {args.warmup}")
    run_steps(args.warmup, pipelined)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    _log(f"timing {args.steps} steps ({'pipelined' if pipelined else 'serial'})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps, pipelined, ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-stage times (hash, dedup, gather) from a separate, shorter run with an event pair around every stage
    n_stage = min(args.steps, 200)
    ev_stage = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_stage)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    run_steps(n_stage, pipelined, ev_stage, stages=True)
    torch.cuda.synchronize()
    stage_us = (time.perf_counter() - t2) / n_stage * 1e6

    serial = None
    if pipelined:
        # the same steps one after the other on one stream, for comparison with the pipelined ones
        n_serial = min(args.steps, 200)
        run_steps(min(args.warmup, 5), False)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        run_steps(n_serial, False)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t1) / n_serial
        serial = {"steps": n_serial, "us_per_step": dt * 1e6, "tokens_per_s": n_tok / dt}

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    controls = None
    if args.workload == 4 and not (args.no_controls or args.dedup or args.uniform_ids or args.flush_mib):
        controls = measure_controls(hg, torch, workloads, plan, w, batches, addr, out, stream, seq_len,
                                    (GATHER_BYTES_PER_TOKEN - 48 * 4 + 48 * (8 if mx else 4)) * n_tok)
    ceiling = None if args.no_ceiling or args.dedup else measure_ceiling(hg, torch, plan, tables, addr, out, stream)
    graph = None
    if not args.dedup:
        # the same step captured once into a HIP graph and replayed: the cost without host launch overhead
        b0 = batches[0]
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            hg.hash(plan, b0[1], b0[2], out=addr)
            gather()
            hg.lookup(plan, b0[1], b0[2], out=out)
        stream.wait_stream(side)
        # 20 steps per graph: one replay shows the device-side time of back-to-back steps
        per_graph = 20
        g_two, g_fused = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_two):
            for j in range(per_graph):
                b = batches[j % len(batches)]
                hg.hash(plan, b[1], b[2], out=addr)
                gather()
        with torch.cuda.graph(g_fused):
            for j in range(per_graph):
                b = batches[j % len(batches)]
                hg.lookup(plan, b[1], b[2], out=out)
        reps = 5
        t_two = _median_ms(torch, g_two.replay, stream, reps) / per_graph
        t_fused = _median_ms(torch, g_fused.replay, stream, reps) / per_graph
        graph = {"steps_per_graph": per_graph, "two_call_us_per_step": t_two * 1e3, "fused_us_per_step": t_fused * 1e3,
                 "two_call_tokens_per_s": n_tok / (t_two / 1e3), "fused_tokens_per_s": n_tok / (t_fused / 1e3)}
        del g_two, g_fused
    fused = None
    if not args.dedup:
        # the same step as one fused launch (engram_lookup): addresses never leave the wave
        turn = [0]

        def fused_step():
            b = batches[turn[0] % len(batches)]
            turn[0] += 1
            hg.lookup(plan, b[1], b[2], out=out, stream=stream)

        t_fused = _median_ms(torch, fused_step, stream, max(5, min(args.steps, 50)))
        # one id read per token (the window's other ids are cache hits), rows, scales, output
        fused_bytes = n_tok * (4 + 48 * 256 + 48 * (8 if mx else 4) + 2 * 256 * 4)
        fused = {"us_per_step": t_fused * 1e3, "tokens_per_s": n_tok / (t_fused / 1e3),
                 "bytes_per_launch": fused_bytes, "frac": fused_bytes / (t_fused / 1e3) / 1e9 / HBM_PEAK_GBPS}

    # the gate-input calls on the first batch's addresses (one batch replayed): per-module sums with one
    # weight per row, and the 48 dequantised rows un-reduced (fp32 [n_tok, 48, 256], 48 KiB per token); and the
    # opt-in input check over the same ids and addresses
    scale_bytes = 48 * (8 if mx else 4)  # per token
    gate = None
    if not args.dedup and n_tok <= 131072:
        b0 = batches[0]
        hg.hash(plan, b0[1], b0[2], out=addr, stream=stream)
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.token_seed + 7)
        weights = torch.rand((n_tok, 48), generator=gen, device=dev)
        rows_out = torch.empty((n_tok, 48, 256), dtype=torch.float32, device=dev)
        t_w = _median_ms(torch, lambda: hg.gather_weighted(plan, addr, weights, out=out, stream=stream), stream, 10)
        t_r = _median_ms(torch, lambda: hg.gather_rows(plan, addr, out=rows_out, stream=stream), stream, 5)
        del rows_out, weights
        w_bytes = n_tok * (48 * 256 + scale_bytes + 48 * 4 + 48 * 4 + 2 * 256 * 4)
        r_bytes = n_tok * (48 * 256 + scale_bytes + 48 * 4 + 48 * 256 * 4)
        # the opt-in range check over the same batch's ids and addresses (engram_check_inputs)
        counts = torch.empty(3, dtype=torch.int32, device=dev)
        t_c = _median_ms(torch, lambda: hg.check_inputs(plan, b0[1], b0[2], addr=addr, counts=counts, stream=stream),
                         stream, 10)
        c_bytes = n_tok * (4 + 48 * 4) + (0 if b0[2] is None else b0[2].numel() * 4)
        gate = {
            "ids": "first batch, replayed",
            "check_inputs_us": t_c * 1e3,
            "check_inputs_bytes_per_launch": c_bytes,
            "check_inputs_frac": c_bytes / (t_c / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "gather_weighted_us": t_w * 1e3,
            "gather_weighted_bytes_per_launch": w_bytes,
            "gather_weighted_frac": w_bytes / (t_w / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "gather_rows_us": t_r * 1e3,
            "gather_rows_bytes_per_launch": r_bytes,
            "gather_rows_frac": r_bytes / (t_r / 1e3) / 1e9 / HBM_PEAK_GBPS,
        }

    # distinct (sub-table, row) pairs of the first batch: the bytes a perfect cache would still fetch
    b0 = batches[0]
    hg.hash(plan, b0[1], b0[2], out=addr, stream=stream)
    keys = addr.view(torch.int32).cpu().numpy().view(np.uint32).astype(np.uint64)
    keys |= np.arange(48, dtype=np.uint64)[None, :] << np.uint64(32)
    distinct = int(np.unique(keys).size)

    hash_ms = None if fused_dedup else float(np.mean([e[0].elapsed_time(e[1]) for e in ev_stage]))
    dedup_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev_stage])) if args.dedup else None
    gather_ms = float(np.mean([e[4].elapsed_time(e[5]) for e in ev]))
    ms_per_step = wall / args.steps * 1e3
    tok_s = n_tok / (ms_per_step / 1e3)
    n_unique = int(groups.n_unique.item()) if args.dedup else None
    if args.dedup:
        # one lookup per group (rows, scales, its offsets pair, and either its 48 addresses or, fused, its 4 window
        # ids) + one perm read and one 2 KiB output store per token
        per_group = 48 * 256 + scale_bytes + 8 + (4 * 4 if fused_dedup else 48 * 4)
        gather_bytes = n_unique * per_group + n_tok * (4 + 2 * 256 * 4)
    else:
        gather_bytes = (GATHER_BYTES_PER_TOKEN - 48 * 4 + scale_bytes) * n_tok
    achieved = gather_bytes / (gather_ms / 1e3) / 1e9
    plain = not (mx or args.vocab_map or args.prime_rows or args.uniform_ids or args.flush_mib
                 or (args.dedup and not fused_dedup))
    pmc_key = (args.workload, "dedup" if fused_dedup else "direct")
    traffic_fetch = _traffic(pmc_key, n_tok, args.id_batches) if plain else None
    traffic = _traffic_exact(pmc_key, n_tok, args.id_batches) if plain else None

    base = None
    if args.cpu_sample > 0 and args.workload == 4:
        workers = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
        keys = [int(k) for k in args.cpu_workloads.split(",") if k.strip()]
        base = cpu_baseline(keys, workers, min(args.cpu_sample, n_tok))

    rec = {
        "metric": "Engram lookup tokens/sec and achieved gather HBM GB/s (% of peak), 1 MI355X",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": (WORKLOAD_TEXT[args.workload]),
            "n_tok": n_tok,
            "tokens_per_sequence": seq_len,
            "rows_per_subtable": w.rows,
            "scale_format": args.scale_format,
            "vocab_map": "seeded 129280 -> 99092" if args.vocab_map else None,
            "prime_rows": bool(args.prime_rows),
            "ids": "uniform over 129280 (control)" if args.uniform_ids else "Zipf(1.1) over 129280",
            "flush_mib_per_step": args.flush_mib,
            "id_batches": args.id_batches,
            "step": ("engram_dedup + engram_lookup_dedup" if fused_dedup
                     else "engram_hash + engram_dedup + engram_gather_reduce (dedup mode)" if args.dedup
                     else "engram_hash + engram_gather_reduce_batched" if batched
                     else "engram_hash + engram_gather_reduce")
                    + (("; batch i+1's dedup on another stream while batch i is looked up" if fused_dedup
                        else "; batch i+1's hash (and dedup) on other streams while batch i is gathered") if pipelined
                       else "; all in order on one stream"),
            "n_unique": n_unique,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("gather_batched_kernel" if batched else "lookup_kernel (dedup mode)" if fused_dedup
                       else "gather_reduce_kernel"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "traffic_detail": None if traffic is None else {
            "bytes_by_request_size": traffic,
            "ratio_to_algorithmic": traffic / gather_bytes,
            "GBps": traffic / (gather_ms / 1e3) / 1e9,
            "fetch_size_estimate_bytes": traffic_fetch,
            "note": "roofline.traffic: bytes leaving L2 per launch from the request-size counters (128-byte row "
                    "reads, 64-byte scale reads, 64-byte writes); the FETCH_SIZE x copy-calibration estimate counts "
                    "each 64-byte scale request as 128 bytes",
        },
        "controls": controls,
        "serial_step": serial,
        "per_step_us": {"eager": ms_per_step * 1e3,
                        "graph_two_call": None if graph is None else graph["two_call_us_per_step"],
                        "graph_fused": None if graph is None else graph["fused_us_per_step"]},
        "gather_ms": gather_ms,
        "hash_ms": hash_ms,
        "dedup_ms": dedup_ms,
        "stage_timing": {"steps": n_stage, "us_per_step": stage_us,
                         "gather_ms": float(np.mean([e[4].elapsed_time(e[5]) for e in ev_stage])),
                         "note": "hash_ms and dedup_ms come from this separate run, with an event pair around every "
                                 "stage; the timed steps record only the gather's pair"
                                 + ("; pipelined, the stages on the side streams overlap the previous gather and their "
                                    "times include waiting for the compute units it holds" if pipelined else "")},
        "us_per_step": ms_per_step * 1e3,
        "hash_gbps": None if hash_ms is None else HASH_BYTES_PER_TOKEN * n_tok / (hash_ms / 1e3) / 1e9,
        "gather_bytes_per_launch": gather_bytes,
        "unique_rows": {
            "distinct_rows": distinct,
            "row_reads": 48 * n_tok,
            "bytes": distinct * (256 + scale_bytes // 48) + n_tok * 2 * 256 * 4,
        },
        "fused_lookup": fused,
        "gate_inputs": gate,
        "graph_replay": graph,
        "ceiling": ceiling,
        "cpu_baseline": base,
        "pages_context": {
            "rows_per_token": 48,
            "table_bytes_per_token": 12672,
            "decode": "10 tokens/s needs ~120 KB/s of table reads",
            "note": "figures the pages give for the whole model on other hardware, not an Engram kernel result",
        },
    }
    if ceiling:
        rec["ceiling"]["gather_vs_read_ceiling"] = achieved / ceiling["stream_read_GBps"]
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
