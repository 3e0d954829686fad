"""The training loop that bench.py times, as a reusable object (the parity tests run the
same object, so the launch configuration they check is the one the benchmark measures).

Every batch is grouped (tt_bag_plan, or tt_bag_plan_dedup for the backward over distinct
indices), then runs the planned forward and the planned backward.  Pipelined (default):
the grouping of batch i+AHEAD is enqueued on a second stream right after the forward of
batch i and runs beside the backward; the host waits for a batch's grouping before it
enqueues the batch's forward.  Two batches ahead, a grouping has a whole step more to
finish than the host needs to reach it, so the host does not wait on it; with a cache and
fewer than three batches it is one batch ahead.  A grouping must not
overwrite a
workspace before the last step that used it has finished.  An event recorded on the main
stream costs several microseconds of that stream's time, so it is recorded only after every
DONE_EVERY-th step, AHEAD + DONE_EVERY workspaces rotate, and a grouping waits for the
latest step with an event, which is at or after the last user of its workspace.  With a
cache, the lookup of a batch runs on the grouping stream just before its grouping and
writes that batch's slot buffer; the lookup of batch i + AHEAD, enqueued during step i,
overwrites the buffer step i + AHEAD - len(batches) read, which must be a step the grouping
waits for (<= i - 1: hence three batches for two ahead), so there an event follows every
step.  Argument marshalling only: every step runs in libttbag.

Captured (graph=True, the plain path): each step -- forward of batch i on the capture
stream, then the grouping of batch i + AHEAD forked onto the second stream beside the
backward of batch i, joined back at the end -- is captured once per (batch, workspace)
combination into a HIP graph (torch.cuda.CUDAGraph), all of them when the loop is built,
and a step is one replay.  Replays run in order on one stream and every graph joins its
grouping, so workspace reuse needs no events; the kernels tag their grid-wide flags with
the workspace's own call counts, so a replayed launch does not see the flags of the last.
"""
from __future__ import annotations

import math
import time
from typing import List

import torch

from . import abi

DONE_EVERY = 4  # steps per main-stream "done" event in the pipelined loop (without a cache)


class TrainLoop:
    """step() enqueues one training step of the next batch (batches are cycled) and
    returns its index.  batches: dicts with device tensors "indices", "offsets",
    "grad_out", "per_sample_weights" (or None).  update: "sgd" (fused SGD, lr), "adagrad"
    (fused Adagrad with eps 1e-10; aux / aux_rows hold the running sums) or "grad"
    (gradients written to aux / aux_rows).  cache: an abi.Cache with its rows and one
    slot buffer per batch.  out receives the pooled forward of the step.  A d-core
    descriptor (abi.TTDescD) runs the d-core calls (no cache, no distinct-index backward,
    sgd or grad)."""

    def __init__(self, desc, cores: List[torch.Tensor], batches, num_bags: int, lr: float,
                 out: torch.Tensor, status: torch.Tensor, update: str = "sgd", aux=None,
                 aux_rows=None, cache=None, rows=None, slots=None, dedup: bool = False,
                 pipeline: bool = True, graph: bool = False):
        if dedup and (cache is not None or update == "adagrad"):
            raise ValueError("the backward over distinct indices takes no cache and updates "
                             "by sgd or grad")
        self.dcore = isinstance(desc, abi.TTDescD)
        if self.dcore and (cache is not None or dedup or update == "adagrad"):
            raise ValueError("d-core tables take no cache and no distinct-index backward, "
                             "and update by sgd or grad")
        if update not in ("sgd", "adagrad", "grad"):
            raise ValueError("update must be sgd, adagrad or grad")
        if cache is not None and pipeline and len(batches) < 2:
            # the lookup of batch i+1 writes the slot buffer of batch (i+1) % len(batches),
            # which the forward of step i may still read when that is the same buffer
            raise ValueError("the pipelined loop with a cache needs at least two batches")
        self.desc, self.g, self.batches, self.B, self.lr = desc, cores, batches, num_bags, lr
        self.out, self.status, self.update = out, status, update
        self.aux, self.aux_rows = aux, aux_rows
        self.cache, self.rows, self.slots = cache, rows, slots
        self.dedup, self.pipeline = dedup, pipeline
        max_nnz = max(b["indices"].numel() for b in batches)
        csize = cache.cache_size if cache is not None else 0
        if self.dcore:
            make_ws = lambda: abi.workspace_d(desc, max_nnz, num_bags)  # noqa: E731
        elif dedup:
            make_ws = lambda: abi.workspace_dedup(desc, max_nnz, num_bags)  # noqa: E731
        else:
            make_ws = lambda: abi.workspace(desc, max_nnz, num_bags, csize)  # noqa: E731
        # done events after steps k with k % every == every - 1.  The grouping of batch j is
        # enqueued during step j - ahead and waits for the latest such k <= j - ahead - 1,
        # which is >= j - ahead - every; batch j's workspace j % (ahead + every) was last
        # used by step j - ahead - every, so that event covers it.
        self.every = 1 if cache is not None else DONE_EVERY
        self.ahead = 2 if (pipeline and (cache is None or len(batches) >= 3)) else 1
        self.wss = [make_ws() for _ in range(self.ahead + self.every if pipeline else 1)]
        self.main = torch.cuda.current_stream()
        self.side = torch.cuda.Stream() if pipeline else self.main  # default priority
        self.ev_plan = [torch.cuda.Event() for _ in range(self.ahead + 1)]
        self.ev_done = {-1: torch.cuda.Event()}  # step -> event after its backward
        self.ev_done[-1].record(self.main)
        self.next = 0
        self.cvs = {}
        self.infos = {}
        # three-core calls (the plain path and the backward over distinct indices) are checked
        # and marshalled once per (batch, workspace) and then replayed (abi.prepare_*): the
        # host work per step is the C calls
        self.fast = not self.dcore
        self.prepared = {}
        self.wait_s = 0.0  # host time spent waiting for groupings
        self.graph = graph
        if graph and not (pipeline and self.fast and cache is None and not dedup):
            raise ValueError("a captured loop takes the plain pipelined path: three cores, "
                             "no cache, no distinct-index backward")
        if graph:
            # steps are captured on a stream of their own (default priority) and replayed
            # on the main stream; the calls are prepared for the capture streams
            self.cap = torch.cuda.Stream()
            self.graphs = []
        if pipeline:
            for j in range(self.ahead):
                self.cvs[j] = self._plan(j)
        if graph:
            torch.cuda.synchronize()
            nb, nw = len(batches), len(self.wss)
            period = nb * nw // math.gcd(nb, nw)  # (batch, workspace) combinations in turn
            self.graphs = [self._capture(k) for k in range(period)]

    def _calls(self, i: int, stream):
        """The prepared forward and backward of batch i (workspace i), on `stream`."""
        bi, wi = i % len(self.batches), i % len(self.wss)
        key = ("fwd", bi, wi, id(stream))
        if key not in self.prepared:
            b, ws = self.batches[bi], self.wss[wi]
            w = b["per_sample_weights"]
            eps = 1e-10 if self.update == "adagrad" else 0.0
            self.prepared[key] = abi.prepare_forward(
                self.desc, self.g, b["indices"], b["offsets"], self.B, w, out=self.out, ws=ws,
                dev_status=self.status, stream=stream)
            self.prepared[("bwd", bi, wi, id(stream))] = abi.prepare_backward(
                self.desc, self.g, b["indices"], b["offsets"], self.B, b["grad_out"],
                update=self.update, lr=self.lr, eps=eps, aux=self.aux, aux_rows=self.aux_rows,
                per_sample_weights=w, ws=ws, dev_status=self.status, stream=stream)
        return self.prepared[key], self.prepared[("bwd", bi, wi, id(stream))]

    def _capture(self, k: int):
        """Graph of step k (and of every step k + period): the forward of batch k, the
        grouping of batch k + ahead beside the backward of batch k, joined."""
        j = k + self.ahead
        bj, wj = self.batches[j % len(self.batches)], self.wss[j % len(self.wss)]
        plan = abi.prepare_plan(self.desc, bj["indices"], bj["offsets"], self.B,
                                bj["per_sample_weights"], ws=wj, dev_status=self.status,
                                stream=self.side)
        fwd, bwd = self._calls(k, self.cap)
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=self.cap):
            fwd()
            fork.record(self.cap)
            self.side.wait_event(fork)
            plan()
            join.record(self.side)
            bwd()
            self.cap.wait_event(join)
        return gr

    def _plan(self, i: int):
        b = self.batches[i % len(self.batches)]
        ws = self.wss[i % len(self.wss)]
        cv = None
        if self.pipeline:
            k = self.done_step(i)
            self.side.wait_event(self.ev_done[k])
            for old in [k0 for k0 in self.ev_done if k0 < k]:
                del self.ev_done[old]
        if self.cache is not None:
            s = self.slots[i % len(self.batches)]
            self.cache.lookup(b["indices"], slot_out=s, count_freq=True, dev_status=self.status,
                              stream=self.side)
            cv = (s, self.rows)
        if self.dcore:
            abi.tt_bag_plan_d(self.desc, b["indices"], b["offsets"], self.B,
                              b["per_sample_weights"], ws=ws, dev_status=self.status,
                              stream=self.side)
        elif self.dedup:  # the virtual batch's bounds come back (the count stays on the device)
            key = ("pland", i % len(self.batches), i % len(self.wss))
            call = self.prepared.get(key)
            if call is None:
                call = self.prepared[key] = abi.prepare_plan_dedup(
                    self.desc, b["indices"], b["offsets"], self.B, b["per_sample_weights"],
                    ws=ws, dev_status=self.status, stream=self.side)
            call[0]()
            self.infos[i] = call[1]
        else:
            key = ("plan", i % len(self.batches), i % len(self.wss))
            call = self.prepared.get(key)
            if call is None:
                call = self.prepared[key] = abi.prepare_plan(
                    self.desc, b["indices"], b["offsets"], self.B, b["per_sample_weights"],
                    cache=cv, ws=ws, dev_status=self.status, stream=self.side)
            call()
        if self.pipeline:
            self.ev_plan[i % (self.ahead + 1)].record(self.side)
        return cv

    def _fast_step(self, i, b, ws, cv):
        """Planned forward, the grouping `ahead` batches on, planned backward: prepared calls."""
        bi, wi = i % len(self.batches), i % len(self.wss)
        fwd = self.prepared.get(("fwd", bi, wi))
        if fwd is None:
            w = b["per_sample_weights"]
            fwd = self.prepared[("fwd", bi, wi)] = abi.prepare_forward(
                self.desc, self.g, b["indices"], b["offsets"], self.B, w, cache=cv,
                out=self.out, ws=ws, dev_status=self.status, stream=self.main)
            eps = 1e-10 if self.update == "adagrad" else 0.0
            if self.dedup:
                self.prepared[("bwd", bi, wi)] = abi.prepare_backward_dedup(
                    self.desc, self.g, b["indices"], b["offsets"], self.B, b["grad_out"],
                    self.infos[i], update=self.update, lr=self.lr, aux=self.aux,
                    per_sample_weights=w, ws=ws, dev_status=self.status, stream=self.main)
            else:
                self.prepared[("bwd", bi, wi)] = abi.prepare_backward(
                    self.desc, self.g, b["indices"], b["offsets"], self.B, b["grad_out"],
                    update=self.update, lr=self.lr, eps=eps, aux=self.aux,
                    aux_rows=self.aux_rows, per_sample_weights=w, cache=cv, ws=ws,
                    dev_status=self.status, stream=self.main)
        if self.dedup:
            self.infos.pop(i)  # (the prepared backward holds the bounds)
        fwd()
        if self.pipeline:
            self.cvs[i + self.ahead] = self._plan(i + self.ahead)
        self.prepared[("bwd", bi, wi)]()
        if self.pipeline and i % self.every == self.every - 1:
            ev = torch.cuda.Event()
            ev.record(self.main)
            self.ev_done[i] = ev

    def done_step(self, i: int) -> int:
        """The step whose done event the grouping of batch i waits for: the latest step
        k <= i - ahead - 1 with an event (-1 = before the first step).  Batch i's workspace
        was last used by step i - ahead - every, and k >= i - ahead - every."""
        e = self.every
        k = ((i - self.ahead) // e) * e - 1
        return max(k, -1)

    def step(self) -> int:
        i = self.next
        self.next += 1
        if self.graph:
            self.graphs[i % len(self.graphs)].replay()
            return i
        b = self.batches[i % len(self.batches)]
        ws = self.wss[i % len(self.wss)]
        if self.pipeline:
            # the host waits for this batch's grouping (it ran beside the previous
            # backward and is normally long done) instead of the device: a cross-stream
            # wait on the device costs about 5 us per step even when the event is done
            t = time.perf_counter()
            self.ev_plan[i % (self.ahead + 1)].synchronize()
            self.wait_s += time.perf_counter() - t
            cv = self.cvs.pop(i)
        else:
            cv = self._plan(i)
        w = b["per_sample_weights"]
        if self.fast:
            self._fast_step(i, b, ws, cv)
            return i
        if self.dcore:
            abi.tt_bag_forward_d(self.desc, self.g, b["indices"], b["offsets"], self.B, w,
                                 out=self.out, ws=ws, dev_status=self.status, planned=True)
        else:
            abi.tt_bag_forward(self.desc, self.g, b["indices"], b["offsets"], self.B, w,
                               cache=cv, out=self.out, ws=ws, dev_status=self.status,
                               planned=True)
        if self.pipeline:
            # the grouping `ahead` batches on starts now, beside this batch's backward
            self.cvs[i + self.ahead] = self._plan(i + self.ahead)
        if self.dcore:
            if self.update == "sgd":
                abi.tt_bag_backward_sgd_d(self.desc, self.g, b["indices"], b["offsets"], self.B,
                                          b["grad_out"], self.lr, w, ws=ws,
                                          dev_status=self.status, planned=True)
            else:
                abi.tt_bag_backward_grad_d(self.desc, self.g, b["indices"], b["offsets"],
                                           self.B, b["grad_out"], grad_cores=self.aux,
                                           per_sample_weights=w, ws=ws,
                                           dev_status=self.status, planned=True)
        elif self.dedup:
            info = self.infos.pop(i)
            if self.update == "sgd":
                abi.tt_bag_backward_sgd_dedup(self.desc, self.g, b["indices"], b["offsets"],
                                              self.B, b["grad_out"], self.lr, info,
                                              per_sample_weights=w, ws=ws,
                                              dev_status=self.status)
            else:
                abi.tt_bag_backward_grad_dedup(self.desc, self.g, b["indices"], b["offsets"],
                                               self.B, b["grad_out"], info, grad_cores=self.aux,
                                               per_sample_weights=w, ws=ws,
                                               dev_status=self.status)
        elif self.update == "sgd":
            abi.tt_bag_backward_sgd(self.desc, self.g, b["indices"], b["offsets"], self.B,
                                    b["grad_out"], self.lr, w, cache=cv, ws=ws,
                                    dev_status=self.status, planned=True)
        elif self.update == "adagrad":
            abi.tt_bag_backward_adagrad(self.desc, self.g, b["indices"], b["offsets"], self.B,
                                        b["grad_out"], self.lr, 1e-10, self.aux,
                                        state_rows=self.aux_rows, per_sample_weights=w,
                                        cache=cv, ws=ws, dev_status=self.status, planned=True)
        else:
            abi.tt_bag_backward_grad(self.desc, self.g, b["indices"], b["offsets"], self.B,
                                     b["grad_out"], grad_cores=self.aux, grad_rows=self.aux_rows,
                                     per_sample_weights=w, cache=cv, ws=ws,
                                     dev_status=self.status, planned=True)
        if self.pipeline:
            if i % self.every == self.every - 1:
                ev = torch.cuda.Event()
                ev.record(self.main)
                self.ev_done[i] = ev
        return i
