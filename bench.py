#!/usr/bin/env python3
"""Decode-step benchmark of the paged-KV hot path on one MI355X.

One *step* is one pass of the whole path for one batch of sequences:
  1. host block manager: reserve every sequence's next slot (copy-on-write
     pairs included) and emit the padded block tables and context lengths;
  2. copy slots, pairs, tables and lengths to the device (pinned, async, on
     the compute stream);
  3. pa_cache_write: copy-on-write block copies, then the new K/V rows;
  4. pa_decode: attention of every query head over its paged context
     (single pass, or split context plus the log-sum-exp merge).

Inputs (pool contents, new K/V rows, queries) are synthetic, seeded and
resident in HBM before timing starts.  The pool is fragmented first (every
block taken once and given back in a seeded random order), so each
sequence's blocks are scattered across it.

Printed: one JSON line.  ``value`` is the whole-step KV-read throughput
(algorithmic K+V bytes the decode reads / wall time per step); ``roofline``
is the decode call alone (HIP events on its stream) against the 8 TB/s HBM
peak; ``cpu_baseline`` is the fp64 CPU oracle timed on a bounded sample of
the same step on this host; ``cache_write_us`` is the upload + cache write
(+ copy-on-write) launch timed on its own in further steps.  The default
run (the 7B layer) adds ``workloads``: one compact record for each other
workload of the benchmark set (GQA, 70B with automatic and 512-token
partitions, shared prefix at block 8/16/32, tiny), the INT8 pools and the
GQA prefill chunk over an f16 and an INT8 pool.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import random
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD specification
METRIC = "decode attention KV-read GB/s and % of HBM peak; seq·ctx tokens/sec per layer"

WORKLOADS = {
    # name: (num_seqs, Hq, Hkv, D, bs, dtype, lengths-spec, std, pool)
    "llama7b_mha": dict(S=32, Hq=32, Hkv=32, D=128, bs=16, dtype="f16", ctx=4096, std=1.0,
                        pool=9000,
                        desc="LLaMA-2-7B-shaped layer: 32 seqs x ctx 4096, 32 heads (MHA) x 128, "
                             "fp16 KV, block 16, 9000-block pool"),
    "gqa7b": dict(S=64, Hq=32, Hkv=8, D=128, bs=16, dtype="f16", ctx=(128, 8192), std=1.0,
                  pool=None,
                  desc="GQA 7B-shaped layer: 64 seqs, ctx ~ U[128, 8192], 32 q / 8 KV heads x "
                       "128, fp16, block 16"),
    "llama70b": dict(S=16, Hq=64, Hkv=8, D=128, bs=16, dtype="f16", ctx=32768, std=0.5,
                     pool=None,
                     desc="LLaMA-2-70B-shaped layer: 16 seqs x ctx 32768, 64 q / 8 KV heads x "
                          "128, fp16, block 16, values N(0, 0.5^2)"),
    "shared_prefix": dict(S=64, Hq=32, Hkv=8, D=128, bs=16, dtype="f16", ctx=None, std=1.0,
                          pool=None,
                          desc="shared-prefix decode: 64 seqs = one 512-token ref-counted prefix "
                               "+ private suffix U[1, 2048], 32 q / 8 KV heads x 128, fp16; one "
                               "fork + copy-on-write per step"),
    "tiny": dict(S=4, Hq=8, Hkv=8, D=64, bs=16, dtype="f32", ctx=[100, 37, 16, 1], std=1.0,
                 pool=64, desc="tiny: 4 seqs, MHA 8 x 64, fp32, block 16, lengths 100/37/16/1"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class StepEvent:
    """A HIP timing event recorded on the current stream, created through
    the HIP runtime the process already uses (torch's, found by its soname)
    with hipEventDisableSystemFence: a record is then a queue marker without
    the system-scope cache write-back and invalidate of a default event,
    which cost the step several microseconds per marker on this stack; a
    timestamp and a completion wait need none of it.  Same methods as the
    torch event it replaces (record, synchronize, elapsed_time)."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        import torch
        if StepEvent._hip is None:
            torch.cuda.init()
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            StepEvent._hip = hip
        self._ev = ctypes.c_void_p()
        self._ctypes = ctypes
        if StepEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._ev),
                                                  self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self._stream = torch.cuda.current_stream().cuda_stream

    def record(self):
        if StepEvent._hip.hipEventRecord(self._ev, self._stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        if StepEvent._hip.hipEventSynchronize(self._ev) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_time(self, end):
        ms = self._ctypes.c_float()
        if StepEvent._hip.hipEventElapsedTime(self._ctypes.byref(ms), self._ev, end._ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def release(self):
        """Destroy the event now (not left to interpreter shutdown)."""
        if StepEvent._hip is not None and self._ev:
            StepEvent._hip.hipEventDestroy(self._ev)
            self._ev = self._ctypes.c_void_p()

    @staticmethod
    def release_all(pairs):
        for a, b in pairs:
            a.release()
            b.release()


# Sources each kernel's code and launch depend on (csrc/): a committed
# counter profile stays valid while these files hash to its fingerprint.
_DECODE_COMMON = ["decode_epilogue.h", "decode_schedule.h", "device_common.h", "kernels.h",
                  "merge.hip", "pa_api.cpp"]
KERNEL_SOURCES = {
    "decode_valu": ["decode_valu.hip"] + _DECODE_COMMON,
    "decode_mfma": ["decode_mfma.hip"] + _DECODE_COMMON,
    "decode_valu_i8": ["decode_valu_i8.hip"] + _DECODE_COMMON,
    "decode_mfma_i8": ["decode_mfma_i8.hip", "i8_codes.h"] + _DECODE_COMMON,
    "prefill_mfma": ["prefill_mfma.hip", "prefill_common.h", "device_common.h", "kernels.h",
                     "pa_api.cpp"],
    "prefill_mfma_i8": ["prefill_mfma_i8.hip", "prefill_common.h", "i8_codes.h",
                        "device_common.h", "kernels.h", "pa_api.cpp"],
}


def source_fingerprint(files):
    """sha256 (first 16 hex) over the named csrc/ files, concatenated in
    name order: the key under which measured counter figures stay valid."""
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_cache_153_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic_ratio(kernel, profile_key):
    """(HBM bytes / algorithmic bytes, profile file) for one dispatch of
    ``kernel``, from the committed rocprofv3 counter summary
    ``profiles/<kernel>_<key>.md`` (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated), or (None, None) when there is none or the kernel's
    sources changed since it was taken.  The bench scales the ratio by its
    own algorithmic bytes per launch, so the figure matches the line's step
    count and lengths."""
    for path in [os.path.join(ROOT, "profiles", f"{kernel}_{profile_key}.md")]:
        if not os.path.exists(path):
            continue
        fields = {}
        for line in open(path):
            if " = " in line:
                k, v = line.split(" = ", 1)
                fields[k.strip()] = v.strip()
        files = fields.get("kernel_source_files", "").split()
        if "traffic_ratio" not in fields or not files:
            continue
        if fields.get("kernel_source_fingerprint") == source_fingerprint(files):
            return float(fields["traffic_ratio"]), os.path.basename(path)
    return None, None


def cpu_model():
    """The host CPU's model name (first ``model name`` of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class Step:
    """Holds the block manager, device buffers and the per-step logic."""

    def __init__(self, name, bs, seed, steps_total, kernel, partition, device, context=0,
                 window=0, kv_dtype="f16", kv_loads="auto", prefix_cache=False,
                 upload="fused"):
        import torch
        import paged_kv_cache_153_amd as pa
        import synth
        self.torch, self.pa = torch, pa
        w = dict(WORKLOADS[name])
        if bs and bs != w["bs"]:
            w["bs"] = bs
            w["pool"] = None  # fixed pool sizes are in blocks of the default size
        self.w, self.name, self.kernel, self.partition = w, name, kernel, partition
        self.window = window
        self.int8 = kv_dtype == "i8"
        if self.int8 and w["dtype"] != "f16":
            raise SystemExit("--kv-dtype i8 needs a float16 workload")
        # a pool whose prefix blocks every sequence shares is read with cached
        # loads (the block manager knows it shares); streaming loads otherwise
        self.cached_kv = name == "shared_prefix" if kv_loads == "auto" else kv_loads == "cached"
        S, Hq, Hkv, D, bs = w["S"], w["Hq"], w["Hkv"], w["D"], w["bs"]
        self.S, self.Hq, self.Hkv, self.D, self.bs = S, Hq, Hkv, D, bs
        tdt = synth.DTYPES[w["dtype"]]
        self.elem = 1 if self.int8 else torch.tensor([], dtype=tdt).element_size()
        # HBM bytes one (token, KV head) costs the decode: K and V rows, plus
        # their two float32 scales in an INT8 pool
        self.row_bytes = 2 * D * self.elem + (2 * 4 if self.int8 else 0)
        g_cpu = torch.Generator().manual_seed(seed)

        # ---- context lengths at the first decoded step ----
        if name == "shared_prefix":
            self.prefix = 512
            suffix = torch.randint(1, 2049, (S - 1,), generator=g_cpu).tolist()
            lens0 = [self.prefix + n for n in suffix]           # sequences 0..S-2
        elif context:
            lens0 = [context] * S
        elif isinstance(w["ctx"], tuple):
            lens0 = synth.gqa_lengths(S, w["ctx"][0], w["ctx"][1], seed)
        elif isinstance(w["ctx"], list):
            lens0 = list(w["ctx"])
        else:
            lens0 = [w["ctx"]] * S
        grow = steps_total
        need = sum(-(-(n + grow) // bs) for n in lens0) + (S * 2 if name == "shared_prefix" else 0)
        nb = w["pool"] or math.ceil(1.1 * need)
        nb = max(nb, need)
        self.num_blocks = nb
        self.mb = max(-(-(n + grow) // bs) for n in lens0) + 1

        # ---- host block manager over a fragmented pool ----
        bm = pa.BlockManager(nb, bs)
        tmp = 1 << 40
        for i in range(nb):
            bm.allocate(tmp + i, 1)
        for i in torch.randperm(nb, generator=g_cpu).tolist():
            bm.free(tmp + i)
        self.bm = bm
        self.prefix_info = None
        if name == "shared_prefix" and prefix_cache:
            # requests admitted through the prefix cache: the first one's
            # system-prompt blocks are registered, the others find them by
            # block-hash lookup (token ids are synthetic)
            bm.enable_prefix_cache()
            gen = torch.Generator().manual_seed(seed + 3)
            sys_ids = torch.randint(0, 32000, (self.prefix,), generator=gen).tolist()
            prompts = [sys_ids + torch.randint(0, 32000, (n - self.prefix,), generator=gen).tolist()
                       for n in lens0]
            t0 = time.perf_counter()
            for s_, toks in enumerate(prompts):
                bm.allocate_prompt(s_, toks)
                bm.register(s_)
            admit = time.perf_counter() - t0
            st_ = bm.prefix_stats()
            self.prefix_info = {"admitted_prompts": len(prompts),
                                "admit_us_per_prompt": round(admit / len(prompts) * 1e6, 2),
                                "cached_blocks": st_[0], "hit_blocks": st_[3],
                                "missed_full_blocks": st_[4]}
            self.fork_child = S - 1
            self.parent_rng = random.Random(seed + 1)   # the parent forked each step
        elif name == "shared_prefix":
            self.prefix_seq = 1 << 41
            bm.allocate(self.prefix_seq, self.prefix)
            pblocks, _ = bm.block_table(self.prefix_seq)
            for s in range(S - 1):
                bm.share(s, pblocks, self.prefix)
            # private suffix tokens, one batched append per token position
            remaining = [n - self.prefix for n in lens0]
            while any(r > 0 for r in remaining):
                live = [s for s in range(S - 1) if remaining[s] > 0]
                bm.append_slots(live)
                for s in live:
                    remaining[s] -= 1
            # every sequence was decoded once already: last token is appended per step
            self.fork_child = S - 1
            self.parent_rng = random.Random(seed + 1)   # the parent forked each step
        else:
            for s, n in enumerate(lens0):
                bm.allocate(s, n - 1)        # the step appends token n
        self.seqs = torch.arange(S, dtype=torch.int64)
        if name == "shared_prefix":
            self.seqs = torch.cat([torch.tensor([S - 1]), torch.arange(S - 1)]).to(torch.int64)

        # ---- device data (resident before timing) ----
        dev = device
        g = torch.Generator(device=dev).manual_seed(seed + 2)
        log(f"[bench] {name}: pool {nb} blocks x {2 * Hkv * bs * D * self.elem} B = "
            f"{nb * 2 * Hkv * bs * D * self.elem / 2**30:.2f} GiB, generating on {dev}")
        if self.int8:
            self.pool = synth.int8_codes((nb, 2, Hkv, bs, D), g, dev,
                                         chunk_rows=max(1, (1 << 26) // (2 * Hkv * bs * D)))
            self.kv_scales = (torch.rand((nb, Hkv, 2, bs), generator=g, device=dev) * 0.02
                              + 0.01) * w["std"]
        else:
            self.pool = synth.normal((nb, 2, Hkv, bs, D), tdt, g, dev, w["std"],
                                     chunk_rows=max(1, (1 << 26) // (2 * Hkv * bs * D)))
            self.kv_scales = None
        self.q = synth.normal((S, Hq, D), tdt, g, dev, w["std"])
        self.new_k = synth.normal((S, Hkv, D), tdt, g, dev, w["std"])
        self.new_v = synth.normal((S, Hkv, D), tdt, g, dev, w["std"])
        self.scale = 1.0 / math.sqrt(D)
        self.out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
        ws = pa.decode_workspace_size(S, Hq, Hkv, D, bs, self.mb, self.mb * bs, partition,
                                      pa.I8 if self.int8 else
                                      pa.F32 if w["dtype"] == "f32" else pa.F16, kernel,
                                      sliding_window=window, cached_kv=self.cached_kv)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        # one packed host->device transfer per step: slots | pairs | lens | tables
        self.upload = upload
        self.n_i32 = 2 * S + 2 * S + S + S * self.mb
        self.d_pack = torch.empty(self.n_i32, dtype=torch.int32, device=dev)
        self.d_slots, self.d_pairs, self.d_lens, self.d_tables = self._views(self.d_pack)
        self.bufs = []
        for _ in range(2):
            h = torch.empty(self.n_i32, dtype=torch.int32).pin_memory()
            slots, pairs, lens, tables = self._views(h)
            stream = torch.cuda.current_stream(dev).cuda_stream
            dtype_code = pa.I8 if self.int8 else pa.F32 if w["dtype"] == "f32" else pa.F16
            fused = ((self.d_pack.data_ptr(), h.data_ptr(), self.n_i32 * 4,
                      self.new_k.data_ptr(), self.new_v.data_ptr(), self.pool.data_ptr(),
                      self.kv_scales.data_ptr() if self.int8 else None, slots.data_ptr(), S),
                     pairs.data_ptr(),
                     (nb, Hkv, D, bs, dtype_code, stream))
            self.bufs.append(dict(pack=h, slots=slots, pairs=pairs, lens=lens, tables=tables,
                                  event=torch.cuda.Event(),
                                  stage_args=(self.d_pack.data_ptr(), h.data_ptr(),
                                              self.n_i32 * 4, stream),
                                  fused_args=fused))
        # pa_decode's arguments but the per-step length bound, prepared once
        # (the binding's checks would add host time to every step)
        self.decode_pre = (self.out.data_ptr(), self.q.data_ptr(), self.pool.data_ptr(),
                           self.kv_scales.data_ptr() if self.int8 else None,
                           self.d_tables.data_ptr(), self.d_lens.data_ptr(), S, Hq, Hkv, D, bs,
                           self.mb)
        self.decode_post = (nb, float(self.scale), int(window), int(partition),
                            pa.KERNELS[kernel] | (pa.KV_CACHED if self.cached_kv else 0),
                            self.ws.data_ptr(), self.ws.numel(), None,
                            pa.I8 if self.int8 else pa.F32 if w["dtype"] == "f32" else pa.F16,
                            torch.cuda.current_stream(dev).cuda_stream)
        self.k = 0
        self.host_s = []         # host bookkeeping time per step (block manager, tables)
        self.kv_bytes = []       # algorithmic decode bytes per step
        self.ctx_tokens = []
        self.ncow = []

    def _views(self, flat):
        S, mb = self.S, self.mb
        slots = flat[0:2 * S].view(self.torch.int64)
        pairs = flat[2 * S:4 * S].view(S, 2)
        lens = flat[4 * S:5 * S]
        tables = flat[5 * S:5 * S + S * mb].view(S, mb)
        return slots, pairs, lens, tables

    def host_step(self, buf):
        """Block-manager part of a step: fork/COW bookkeeping, slots, tables."""
        pa = self.pa
        if self.name == "shared_prefix":
            child = self.fork_child
            try:
                self.bm.free(child)
            except pa.PAError:
                pass
            while True:
                parent = self.parent_rng.randrange(self.S - 1)
                if self.bm.num_tokens(parent) % self.bs:
                    break
            self.bm.fork(parent, child)
        ncow = self.bm.append_slots_into(self.seqs, buf["slots"], buf["pairs"])
        self.bm.block_tables_into(self.seqs, buf["tables"], buf["lens"])
        tokens = self.key_tokens(buf["lens"])
        self.ctx_tokens.append(tokens)
        self.kv_bytes.append(tokens * self.Hkv * self.row_bytes)
        self.ncow.append(ncow)
        return ncow

    def key_tokens(self, lens):
        """Tokens the decode attends to: the whole context, or at most the
        last ``window`` tokens of each sequence."""
        import numpy as np
        ln = lens.numpy()
        if self.window > 0:
            return int(np.minimum(ln, self.window).sum())
        return int(ln.sum())

    def run(self, timed_events=None, write_events=None):
        """One decode step.  ``timed_events`` (a pair) brackets the decode
        call; ``write_events`` (a pair) brackets the upload + cache write
        (copy-on-write launch included)."""
        torch, pa = self.torch, self.pa
        buf = self.bufs[self.k % 2]
        fence = buf.pop("fence", None) or buf["event"]
        fence.synchronize()                 # its previous upload has left pinned memory
        t_host = time.perf_counter()
        ncow = self.host_step(buf)
        maxlen = int(buf["lens"].numpy().max())
        self.host_s.append(time.perf_counter() - t_host)
        if write_events is not None:
            write_events[0].record()
        # the C calls take arguments prepared once per buffer (the binding's
        # checks would add host time to every step)
        if self.upload == "fused":   # upload + K/V scatter in one launch
            a = buf["fused_args"]
            rc = pa.lib().pa_stage_and_write(*a[0], a[1] if ncow else None, ncow, *a[2])
            if rc != 0:
                raise pa.PAError(rc, pa.lib().pa_last_error().decode())
            # the pinned buffer may be refilled once this upload has run: in a
            # timed step an event recorded after it anyway marks that (one
            # queue marker fewer per step), otherwise a marker of its own
            if timed_events is not None:
                buf["fence"] = timed_events[1]
            elif write_events is not None:
                buf["fence"] = write_events[1]
            else:
                buf["event"].record()
        else:
            if self.upload == "kernel":
                rc = pa.lib().pa_stage_from_host(*buf["stage_args"])
                if rc != 0:
                    raise pa.PAError(rc, pa.lib().pa_last_error().decode())
            else:
                self.d_pack.copy_(buf["pack"], non_blocking=True)
            buf["event"].record()
            pa.cache_write(self.new_k, self.new_v, self.pool, self.d_slots,
                           cow_pairs=self.d_pairs[:ncow] if ncow else None,
                           kv_scales=self.kv_scales)
        if write_events is not None:
            write_events[1].record()
        if timed_events is not None:
            timed_events[0].record()
        rc = pa.lib().pa_decode(*self.decode_pre, maxlen, *self.decode_post)
        if rc != 0:
            raise pa.PAError(rc, pa.lib().pa_last_error().decode())
        if timed_events is not None:
            timed_events[1].record()
        self.k += 1
        return buf

    def oracle_decode(self, q, pool, bt, lens):
        """The fp64 oracle on host copies from ``host_inputs``."""
        import oracle
        if self.int8:
            return oracle.decode_i8_ref(q, pool[0], pool[1], bt, lens, self.scale,
                                        window=self.window)
        return oracle.decode_ref(q, pool, bt, lens, self.scale, window=self.window)

    def host_inputs(self, positions):
        """Host copies of the last step's inputs for some table rows: only those
        rows' blocks (renumbered 0..), so the oracle reads the very same bits."""
        import numpy as np
        buf = self.bufs[(self.k - 1) % 2]
        tables, lens = buf["tables"], buf["lens"]
        blocks, rows, lns, off = [], [], [], 0
        for pos in positions:
            n = int(lens[pos])
            nblk = -(-n // self.bs)
            ids = tables[pos, :nblk].long().to(self.pool.device)
            if self.int8:
                blocks.append((self.pool[ids].cpu().numpy(), self.kv_scales[ids].cpu().numpy()))
            else:
                blocks.append(self.pool[ids].cpu().numpy())
            rows.append(np.arange(off, off + nblk))
            off += nblk
            lns.append(n)
        if self.int8:
            pool = (np.concatenate([b[0] for b in blocks]), np.concatenate([b[1] for b in blocks]))
        else:
            pool = np.concatenate(blocks)
        bt = np.full((len(rows), max(1, max(len(r) for r in rows))), -1, dtype=np.int64)
        for i, r in enumerate(rows):
            bt[i, :len(r)] = r
        pos_t = self.torch.tensor(list(positions), device=self.q.device)
        q = self.q[pos_t].cpu().numpy()
        return q, pool, bt, np.array(lns), pos_t


def cpu_baseline(st, budget_s=20.0, cap_wall_s=8.0):
    """Time the fp64 oracle on the host cores: the last step's sequences
    (copied to host memory first, outside the timed region) decoded in turn
    by a pool of worker threads (BLAS limited to one thread each; NumPy
    releases the GIL inside its array operations), until about ``budget_s``
    of CPU time (workers x wall time) or ``cap_wall_s`` of wall time."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import numpy as np
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    picks = list(range(min(st.S, workers)))
    inputs = [st.host_inputs([p]) for p in picks]
    keys = [int(np.minimum(x[3], st.window).sum()) if st.window > 0 else int(x[3].sum())
            for x in inputs]
    runs, nbytes, toks = 0, 0, 0
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        t0 = time.perf_counter()
        while True:
            futs = [ex.submit(st.oracle_decode, *x[:4]) for x in inputs]
            for f in futs:
                f.result()
            runs += len(inputs)
            toks += sum(keys)
            nbytes += sum(keys) * st.Hkv * st.row_bytes
            wall = time.perf_counter() - t0
            if wall * workers >= budget_s or wall >= cap_wall_s:
                break
    return dict(value=round(nbytes / wall / 1e9, 4), unit="GB/s", cores=workers, kind="oracle",
                sample=f"fp64 NumPy oracle on {workers} worker threads (BLAS 1 thread each): "
                       f"{runs} sequence decodes of {len(inputs)} of the last timed step's "
                       f"{st.S} sequences ({toks} key tokens, {nbytes} KV bytes) in "
                       f"{wall:.2f} s wall; {toks / wall:.4g} seq*ctx tokens/s")


def prefill_cpu_baseline(q, x, S, T, n, budget_s=20.0, cap_wall_s=8.0, rows=16, window=0):
    """Time the fp64 oracle (prefill_ref) on the host cores: groups of
    ``rows`` consecutive query rows of the step's first sequences, each group
    the last ``rows`` tokens of a context ending at its last row (host copies
    of the sequences' blocks and queries are made first, outside the timed
    region), computed by a pool of worker threads (BLAS limited to one thread
    each) until about ``budget_s`` of CPU time or ``cap_wall_s`` of wall
    time.  TFLOP/s of useful flops (4 * D * Hq per query row and key)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import numpy as np
    import oracle
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    bs, Hq, D = x.block_size, x.num_q_heads, x.head_dim
    nseq = min(S, 4)
    host = []
    for s_ in range(nseq):
        ids = x.block_tables[s_, :-(-n // bs)].long()
        host.append((x.kv_cache[ids].cpu().numpy(), q[s_ * T:(s_ + 1) * T].cpu().numpy()))
    groups = [(s_, i0) for i0 in range(0, T - rows + 1, rows) for s_ in range(nseq)]
    rng = np.random.default_rng(0)
    rng.shuffle(groups)

    def one(item):
        s_, i0 = item
        blocks, qs = host[s_]
        ctx = n - T + i0 + rows                 # the group is the last `rows` tokens
        return oracle.prefill_ref(qs[i0:i0 + rows], blocks, np.arange(blocks.shape[0])[None],
                                  np.array([ctx]), np.array([0, rows]), x.scale, window=window)

    done, flops = 0, 0.0
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        t0 = time.perf_counter()
        while True:
            batch = [groups[(done + k) % len(groups)] for k in range(workers)]
            for f in [ex.submit(one, it) for it in batch]:
                f.result()
            for s_, i0 in batch:
                keys = sum(min(n - T + i + 1, window) if window > 0 else n - T + i + 1
                           for i in range(i0, i0 + rows))
                flops += 4.0 * D * Hq * keys
            done += len(batch)
            wall = time.perf_counter() - t0
            if wall * workers >= budget_s or wall >= cap_wall_s:
                break
    return dict(value=round(flops / wall / 1e12, 6), unit="TFLOP/s", cores=workers,
                kind="oracle",
                sample=f"fp64 NumPy prefill oracle on {workers} worker threads (BLAS 1 thread "
                       f"each): {done} groups of {rows} query rows from the first {nseq} "
                       f"sequences' chunks ({done * rows} query rows, {flops:.4g} useful flops) "
                       f"in {wall:.2f} s wall")


def stream_ceiling(dev, tile_bytes=4096, nbytes=4 << 30, reps=5):
    """Measured HBM read ceiling on this GPU (libpa_probe.so): a linear
    grid-stride read and reads of 4 KiB (and, when the decode's K/V tiles
    are 2 KiB, 2 KiB) tiles in random order — the access pattern of paged K/V
    tiles.  GB/s, best over launch shapes and over plain / non-temporal
    loads."""
    import ctypes
    import torch
    probe = ctypes.CDLL(os.path.join(ROOT, "bench_probe", "libpa_probe.so"))
    probe.pa_probe_read_linear.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.pa_probe_read_tiles_sized.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.ones(nbytes // 2, dtype=torch.float16, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream

    def timed(fn):
        if fn() != 0:
            raise RuntimeError("probe launch failed")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9

    lin = max(timed(lambda: probe.pa_probe_read_linear(buf.data_ptr(), nbytes, w, nt,
                                                       sink.data_ptr(), st))
              for w in (1024, 2048, 4096) for nt in (0, 1))
    res = {"linear_read_GBps": round(lin, 1)}
    for tb in sorted({4096, tile_bytes}):
        ntiles = nbytes // tb
        order = torch.randperm(ntiles, generator=torch.Generator().manual_seed(5))
        order = order.to(torch.int32).to(dev)
        til = max(timed(lambda: probe.pa_probe_read_tiles_sized(
            buf.data_ptr(), ntiles, order.data_ptr(), ntiles, per, tb, nt, sink.data_ptr(), st))
            for per in (16, 64) for nt in (0, 1))
        res[f"random_{tb // 1024}KiB_tile_read_GBps"] = round(til, 1)
        del order
    del buf
    torch.cuda.empty_cache()
    return res


def calibrate_copy(dev, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) and as a streaming reference."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / 1e3 / reps
    return {"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
            "dispatches": reps + 1, "copy_GBps_read_plus_write": round(2 * nbytes / sec / 1e9, 1)}


def parity_sample(st, samples=3):
    """Max-abs error of the last step's output vs the oracle on a few sequences."""
    import numpy as np
    picks = sorted({0, st.S - 1, st.S // 2})[:samples]
    q, pool, bt, lens, pos = st.host_inputs(picks)
    want = st.oracle_decode(q, pool, bt, lens)
    got = st.out[pos].cpu().numpy().astype(np.float64)
    return float(np.abs(got - want).max())


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak, AMD specification


def prefill_bench(args, dev, workload=None, steps=None, warmup=None, check_parity=True,
                  cpu=True, kv_dtype=None):
    """Chunked-prefill attention: each step writes a chunk of new K/V rows per
    sequence (pa_cache_write) and runs causal multi-token attention over the
    paged cache (pa_prefill).  Flops counted: 4 * D per (query, head, key
    attended), the q.K and P.V products.  Returns the result line."""
    import torch
    import numpy as np
    import paged_kv_cache_153_amd as pa
    import synth
    workload = workload or args.workload
    steps = steps or args.steps
    warmup = args.warmup if warmup is None else warmup
    w = WORKLOADS[workload]
    S, Hq, Hkv, D = args.seqs or 8, w["Hq"], w["Hkv"], w["D"]
    bs = args.block_size or w["bs"]
    n, T = args.context or (8192 if workload == "llama70b" else 4096), args.chunk
    if w["dtype"] != "f16" or T > n:
        raise SystemExit("prefill needs a float16 workload and chunk <= context")
    x = synth.make_decode_inputs([n] * S, Hq, Hkv, D, bs, dtype="f16", seed=args.seed,
                                 device=dev, std=w["std"])
    int8 = (kv_dtype or args.kv_dtype) == "i8"
    if int8:
        x = synth.int8_pool(x)
    g = synth._gen(args.seed + 7, dev)
    q = synth.normal((S * T, Hq, D), torch.float16, g, dev, w["std"])
    new_k = synth.normal((S * T, Hkv, D), torch.float16, g, dev, w["std"])
    new_v = synth.normal((S * T, Hkv, D), torch.float16, g, dev, w["std"])
    bt = x.block_tables.cpu().numpy()
    pos = np.arange(n - T, n)
    slots = torch.tensor(np.concatenate([bt[s_, pos // bs] * bs + pos % bs for s_ in range(S)]),
                         dtype=torch.int64, device=dev)
    qstart = torch.arange(0, S * T + 1, T, dtype=torch.int32, device=dev)
    out = torch.empty((S * T, Hq, D), dtype=torch.float32, device=dev)
    win = args.window
    # keys attended per query at position p: p + 1, or at most the window
    keys = S * sum(min(p + 1, win) if win > 0 else p + 1 for p in range(n - T, n))
    flops = 4.0 * D * Hq * keys

    def step(ev=None):
        pa.cache_write(new_k, new_v, x.kv_cache, slots, kv_scales=x.kv_scales)
        if ev:
            ev[0].record()
        pa.prefill(q, x.kv_cache, x.block_tables, x.context_lens, qstart, scale=x.scale,
                   max_query_len=T, out=out, sliding_window=win, kv_scales=x.kv_scales)
        if ev:
            ev[1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(StepEvent(), StepEvent()) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    att_s = sum(a.elapsed_time(b) for a, b in ev) / steps / 1e3
    StepEvent.release_all(ev)
    tflops = flops / att_s / 1e12
    parity = None
    if check_parity:
        import oracle
        rng = np.random.default_rng(0)
        errs = []
        for s_ in (0, S - 1):
            ids = x.block_tables[s_, :-(-n // bs)].long()
            blocks = x.kv_cache[ids].cpu().numpy()
            scl = x.kv_scales[ids].cpu().numpy() if int8 else None
            for i in (0, T - 1, int(rng.integers(T))):
                row = s_ * T + i
                args_ = (q[row:row + 1].cpu().numpy(), blocks)
                rest = (np.arange(blocks.shape[0])[None], np.array([n - T + i + 1]),
                        np.array([0, 1]), x.scale)
                want = (oracle.prefill_i8_ref(*args_, scl, *rest, window=win) if int8 else
                        oracle.prefill_ref(*args_, *rest, window=win))
                errs.append(float(np.abs(out[row].cpu().numpy() - want[0]).max()))
        parity = max(errs)
    log(f"[bench] prefill step {wall / steps * 1e6:.1f} us, attention {att_s * 1e6:.1f} us, "
        f"{tflops:.1f} TFLOP/s")
    # HBM bytes the kernel must move at least: every K/V row of the
    # contexts once, the queries, the outputs
    rows_read = min(n, T + win - 1) if win > 0 else n     # keys some query of a chunk sees
    row_bytes = 2 * D + 8 if int8 else 2 * D * 2           # K + V of one (token, KV head)
    unique = S * rows_read * Hkv * row_bytes + S * T * Hq * D * (2 + 4)
    kname = "prefill_mfma_i8" if int8 else "prefill_mfma"
    ratio, prof = measured_traffic_ratio(kname, f"prefill_{workload}" + ("_i8" if int8 else ""))
    res = {
        "metric": "chunked-prefill attention TFLOP/s (q.K and P.V, useful flops)",
        "value": round(flops * steps / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8" if int8 else "f16",
        "data": "synthetic (seeded N(0, std^2) K/V/Q; no weights)",
        "config": {"workload": f"{w['desc']}: {S} seqs, chunk {T} at context {n} (past {n - T})"
                               + (f", sliding window {win}" if win > 0 else ""),
                   "sliding_window": win or None,
                   "kv_cache": "int8 codes + f32 row scales" if int8 else "f16",
                   "num_seqs": S, "chunk": T, "context": n, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "step": "pa_cache_write (chunk rows) + pa_prefill"},
        "attention_us": round(att_s * 1e6, 2),
        "query_tokens_per_s": round(S * T / att_s, 1),
        "parity_max_abs_err": parity,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     # HBM bytes per pa_prefill dispatch: the committed counter
                     # profile's ratio to the unique bytes, times this line's
                     "traffic": round(ratio * unique) if ratio else None},
        "traffic_profile": prof,
        "cpu_baseline": (prefill_cpu_baseline(q, x, S, T, n, window=win)
                         if cpu and not int8 else None),
    }
    del x, q, new_k, new_v, out
    torch.cuda.empty_cache()
    return res


# The other workloads the default run also measures (one compact record
# each, after the headline): the remaining configurations of the method's
# benchmark set, the INT8 pools and a chunked prefill.
EXTRA_DECODE = [
    # (key, workload, overrides)
    ("tiny", "tiny", {}),
    ("gqa7b", "gqa7b", {}),
    ("llama70b", "llama70b", {}),
    ("llama70b_p512", "llama70b", {"partition": 512}),
    ("shared_prefix_bs8", "shared_prefix", {"block_size": 8}),
    ("shared_prefix", "shared_prefix", {}),           # block 16, the workload's own
    ("shared_prefix_bs32", "shared_prefix", {"block_size": 32}),
    ("llama7b_mha_i8", "llama7b_mha", {"kv_dtype": "i8"}),
    ("gqa7b_i8", "gqa7b", {"kv_dtype": "i8"}),
    ("llama70b_i8", "llama70b", {"kv_dtype": "i8"}),
]
EXTRA_PREFILL = [
    # (key, workload, pool)
    ("prefill_gqa7b", "gqa7b", "f16"),
    ("prefill_gqa7b_i8", "gqa7b", "i8"),
]


def measure_decode(args, dev, name, block_size=None, partition=0, kv_dtype="f16", window=0,
                   context=0, kernel="auto", kv_loads="auto", prefix_cache=False,
                   upload="fused", steps=None, warmup=None, parity=True, write_steps=None):
    """Warm-up steps, then ``steps`` timed steps (decode call bracketed by
    HIP events), then ``write_steps`` steps with the upload + cache write
    bracketed instead.  Returns (Step, metrics)."""
    import torch
    steps = steps or args.steps
    warmup = args.warmup if warmup is None else warmup
    write_steps = min(steps, 20) if write_steps is None else write_steps
    st = Step(name, block_size, args.seed, warmup + steps + write_steps, kernel, partition, dev,
              context=context, window=window, kv_dtype=kv_dtype, kv_loads=kv_loads,
              prefix_cache=prefix_cache, upload=upload)
    log(f"[bench] {name}: warmup {warmup} steps")
    for _ in range(warmup):
        st.run()
    torch.cuda.synchronize()
    st.kv_bytes.clear()
    st.ctx_tokens.clear()
    st.ncow.clear()
    st.host_s.clear()
    ev = [(StepEvent(), StepEvent()) for _ in range(steps)]
    log(f"[bench] {name}: timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st.run(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    StepEvent.release_all(ev)
    for b in st.bufs:            # the released events no longer fence the buffers
        b.pop("fence", None)
    m = {"steps": steps, "warmup": warmup, "wall": wall,
         "kv_bytes": sum(st.kv_bytes), "tokens": sum(st.ctx_tokens),
         "ncow": sum(st.ncow), "host_us": sum(st.host_s) / steps * 1e6}
    m["dec_avg_s"] = sum(dec_ms) / len(dec_ms) / 1e3
    m["dec_med_s"] = sorted(dec_ms)[len(dec_ms) // 2] / 1e3
    m["achieved"] = m["kv_bytes"] / steps / m["dec_avg_s"] / 1e9
    m["value"] = m["kv_bytes"] / wall / 1e9
    m["parity"] = parity_sample(st) if parity else None
    if write_steps:
        wev = [(StepEvent(), StepEvent()) for _ in range(write_steps)]
        for i in range(write_steps):
            st.run(write_events=wev[i])
        torch.cuda.synchronize()
        w_ms = [a.elapsed_time(b) for a, b in wev]
        StepEvent.release_all(wev)
        for b in st.bufs:
            b.pop("fence", None)
        m["write_us"] = sum(w_ms) / len(w_ms) * 1e3
    else:
        m["write_us"] = None
    log(f"[bench] {name}: step {wall / steps * 1e6:.1f} us, decode {m['dec_avg_s'] * 1e6:.1f} us, "
        f"{m['achieved']:.1f} GB/s decode, {m['value']:.1f} GB/s whole step")
    return st, m


def decode_kernel_name(st, kernel):
    """Family of the decode kernel a Step's launches use (as the library's
    automatic choice picks it: matrix cores for f16 / INT8 with G >= 4)."""
    g = st.Hq // st.Hkv
    if kernel == "auto":
        kernel = "mfma" if st.w["dtype"] != "f32" and g >= 4 else "valu"
    return f"decode_{kernel}" + ("_i8" if st.int8 else "")


def extra_line(args, dev, key, name, kw):
    """One compact record for a further workload at the default launch."""
    import torch
    st, m = measure_decode(args, dev, name, steps=args.steps, warmup=args.warmup,
                           parity=not args.no_parity, **kw)
    ratio, prof = measured_traffic_ratio(decode_kernel_name(st, "auto"), key)
    per_launch = m["kv_bytes"] / m["steps"]
    rec = {
        "workload": st.w["desc"] + (f" (block {st.bs})" if kw.get("block_size") else "")
        + (", INT8 pool" if st.int8 else "")
        + (f", {kw['partition']}-token partitions" if kw.get("partition") else ""),
        "kernel": decode_kernel_name(st, "auto"),
        "partition": kw.get("partition", 0),
        "decode_us": round(m["dec_avg_s"] * 1e6, 2),
        "decode_GBps": round(m["achieved"], 1),
        "hbm_frac": round(m["achieved"] / HBM_PEAK_GBPS, 4),
        "decode_seq_ctx_tokens_per_s": round(m["tokens"] / m["steps"] / m["dec_avg_s"], 1),
        "whole_step_GBps": round(m["value"], 1),
        "ms_per_step": round(m["wall"] / m["steps"] * 1e3, 4),
        "cache_write_us": round(m["write_us"], 2) if m["write_us"] else None,
        "host_bookkeeping_us": round(m["host_us"], 2),
        "cow_pairs_per_step": round(m["ncow"] / m["steps"], 3),
        "parity_max_abs_err": m["parity"],
        "traffic": round(ratio * per_launch) if ratio else None,
        "traffic_profile": prof,
    }
    del st
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_mha", choices=sorted(WORKLOADS))
    ap.add_argument("--block-size", type=int, default=None,
                    help="override the workload's block size (8, 16 or 32)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition", type=int, default=0, help="0 auto, -1 single pass, or tokens")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--context", type=int, default=0,
                    help="override: every sequence at this context length (not shared_prefix)")
    ap.add_argument("--kv-dtype", default="f16", choices=["f16", "i8"],
                    help="i8: INT8 pool with one float32 scale per (token, head) row")
    ap.add_argument("--kv-loads", default="auto", choices=["auto", "cached", "streaming"],
                    help="K/V load policy (auto: cached for shared_prefix, else streaming)")
    ap.add_argument("--prefix-cache", action="store_true",
                    help="shared_prefix: admit the requests through the block manager's prefix "
                         "cache (block-hash lookup) instead of sharing the prefix by hand")
    ap.add_argument("--upload", default="fused", choices=["fused", "kernel", "dma"],
                    help="per-step host->device upload of tables/lengths/slots: in the same "
                         "launch as the K/V scatter (pa_stage_and_write), a kernel of its own "
                         "(pa_stage_from_host) or a DMA copy")
    ap.add_argument("--mode", default="decode", choices=["decode", "prefill"],
                    help="prefill: chunked-prefill attention (pa_prefill) instead of decode")
    ap.add_argument("--chunk", type=int, default=512, help="prefill: new tokens per sequence")
    ap.add_argument("--seqs", type=int, default=0, help="prefill: sequences (default 8)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: attend to the last W tokens (0 = whole context)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured HBM read ceiling (libpa_probe.so)")
    ap.add_argument("--extras", default="auto", choices=["auto", "all", "none"],
                    help="also measure the other workloads (GQA, 70B with automatic and "
                         "512-token partitions, shared prefix at block 8/16/32, tiny, INT8 "
                         "pools, a GQA prefill chunk) in one compact record each; auto = only "
                         "when the headline is the default 7B launch")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", flush=True)
        sys.exit(2)

    import torch
    import paged_kv_cache_153_amd as pa
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    pa.lib()
    dev = torch.device("cuda:0")
    if args.mode == "prefill":
        print(json.dumps(prefill_bench(args, dev, check_parity=not args.no_parity,
                                       cpu=not args.no_cpu_baseline)), flush=True)
        return
    if args.calibrate_copy:
        print(json.dumps(calibrate_copy(dev)), flush=True)
        return
    st, m = measure_decode(args, dev, args.workload, block_size=args.block_size,
                           partition=args.partition, kv_dtype=args.kv_dtype, window=args.window,
                           context=args.context, kernel=args.kernel, kv_loads=args.kv_loads,
                           prefix_cache=args.prefix_cache, upload=args.upload,
                           parity=not args.no_parity)
    steps = args.steps
    step_s = m["wall"] / steps
    dec_avg_s = m["dec_avg_s"]
    achieved = m["achieved"]
    # bytes of one K (or V) tile of one KV head: the unit the decode reads
    tile_bytes = 2048 if st.bs * st.D * st.elem <= 2048 else 4096
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(st)
        cpu["cpu_model"] = cpu_model()
    key = (args.workload + ("_i8" if st.int8 else "")
           + (f"_w{args.window}" if args.window else "")
           + (f"_bs{args.block_size}" if args.block_size else "")
           + (f"_p{args.partition}" if args.partition else ""))
    kernel_name = decode_kernel_name(st, args.kernel)
    ratio, prof = measured_traffic_ratio(kernel_name, key)
    w = st.w
    res = {
        "metric": METRIC,
        "value": round(m["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if st.int8 else w["dtype"],
        "data": "synthetic (seeded N(0, std^2) K/V/Q; fragmented pool; no weights)",
        "config": {
            "workload": w["desc"] + (f" (block {st.bs})" if args.block_size else ""),
            "num_seqs": st.S, "num_q_heads": st.Hq, "num_kv_heads": st.Hkv, "head_dim": st.D,
            "block_size": st.bs, "pool_blocks": st.num_blocks,
            "mean_key_tokens": round(m["tokens"] / steps / st.S, 1),
            "kernel": args.kernel, "partition": args.partition, "seed": args.seed,
            "context_override": args.context or None,
            "sliding_window": args.window or None,
            "kv_cache": "int8 codes + f32 row scales" if st.int8 else w["dtype"],
            "kv_loads": "cached" if st.cached_kv else "streaming (non-temporal)",
            "upload": {"fused": "pa_stage_and_write (upload + scatter, one launch)",
                       "kernel": "pa_stage_from_host kernel",
                       "dma": "DMA copy (torch copy_)"}[st.upload],
            "step": "block-manager append + tables H2D + pa_cache_write (+COW) + pa_decode",
        },
        "hbm_frac_whole_step": round(m["value"] / HBM_PEAK_GBPS, 4),
        "seq_ctx_tokens_per_s": round(m["tokens"] / m["wall"], 1),
        "decode_kernel": kernel_name,
        "decode_us": round(dec_avg_s * 1e6, 2),
        "decode_us_median": round(m["dec_med_s"] * 1e6, 2),
        "decode_seq_ctx_tokens_per_s": round(m["tokens"] / steps / dec_avg_s, 1),
        "cache_write_us": round(m["write_us"], 2) if m["write_us"] else None,
        "host_bookkeeping_us": round(m["host_us"], 2),
        "cow_pairs_per_step": round(m["ncow"] / steps, 3),
        "prefix_cache": st.prefix_info,
        "parity_max_abs_err": m["parity"],
    }
    res["roofline"] = {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        # HBM bytes per decode launch: the committed counter profile's
        # ratio to the algorithmic bytes, times this line's algorithmic bytes
        "traffic": round(ratio * m["kv_bytes"] / steps) if ratio else None,
    }
    res["traffic_profile"] = prof
    res["cpu_baseline"] = cpu
    del st
    torch.cuda.empty_cache()
    ceiling = None if args.no_ceiling else stream_ceiling(dev, tile_bytes)
    res["measured_read_ceiling"] = ceiling
    res["decode_frac_of_tile_ceiling"] = (
        round(achieved / ceiling[f"random_{tile_bytes // 1024}KiB_tile_read_GBps"], 4)
        if ceiling else None)
    default_launch = (args.workload, args.block_size, args.partition, args.kv_dtype, args.window,
                      args.context, args.kernel, args.kv_loads, args.prefix_cache,
                      args.upload) == ("llama7b_mha", None, 0, "f16", 0, 0, "auto", "auto",
                                       False, "fused")
    if args.extras == "all" or (args.extras == "auto" and default_launch):
        extra = {}
        for k, name, kw in EXTRA_DECODE:
            extra[k] = extra_line(args, dev, k, name, kw)
        for k, name, pool in EXTRA_PREFILL:
            r = prefill_bench(args, dev, workload=name, steps=args.steps, warmup=args.warmup,
                              check_parity=not args.no_parity, cpu=False, kv_dtype=pool)
            extra[k] = {
                "workload": r["config"]["workload"],
                "kernel": "prefill_mfma_i8" if pool == "i8" else "prefill_mfma",
                "attention_us": r["attention_us"], "tflops": r["roofline"]["achieved"],
                "mfma_frac": r["roofline"]["frac"], "parity_max_abs_err": r["parity_max_abs_err"],
                "traffic": r["roofline"]["traffic"], "traffic_profile": r["traffic_profile"]}
        res["workloads"] = extra
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
