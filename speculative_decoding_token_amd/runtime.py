"""Host loop over the C ABI: workspace set-up and the draft / verify / accept / trim cycle.

The loop follows "Speculative Decoding on Apple Silicon: 119% Faster...", section "How
speculative decoding works" (draft several tokens, verify them in one target pass, keep
the agreeing prefix plus the target's own token) and reads the emitted tokens back once
per cycle, which is the only device-to-host transfer of a cycle.  All computation runs in
libspec.so; this module allocates device buffers with torch and passes their addresses.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import torch

from . import binding as B


@dataclasses.dataclass
class Cycle:
    drafts: List[List[int]]      # [batch][k]
    n: List[int]
    tokens: List[List[int]]      # [batch][n+1]
    near_tie: List[int]
    logits: Optional[torch.Tensor] = None      # [batch, k+1, V] when kept
    p: Optional[list] = None                   # host lists when kept
    q: Optional[list] = None
    verify_ms: Optional[float] = None          # Engine.run(time_verify=True)


class Engine:
    """One context: a target, an optional drafter (a draft model, the target's MTP layer or
    n-gram lookup), a sampler and a workspace."""

    def __init__(self, target_shape, target_w: Dict, draft_shape=None, draft_w: Optional[Dict] = None,
                 temperature: float = 0.0, top_k: int = 20, top_p: float = 0.95, seed: int = 0,
                 max_batch: int = 1, max_ctx: int = 256, max_k: int = 8, stream=None,
                 drafter: Optional[str] = None, ngram: Sequence[int] = (3, 16)):
        """drafter: None (a draft model when draft_shape is given, else none), "model",
        "mtp" (target_w["mtp"] holds the layer) or "ngram" (ngram = (n_min, max_match))."""
        self._keep: list = []
        cfg = B.spec_config()
        cfg.target = B.model_desc(target_shape, target_w, self._keep)
        if drafter is None:
            drafter = "model" if draft_shape is not None else "none"
        self.drafter = drafter
        if drafter == "model":
            cfg.draft_kind = B.DRAFT_MODEL
            cfg.draft = B.model_desc(draft_shape, draft_w, self._keep)
        elif drafter == "mtp":
            cfg.draft_kind = B.DRAFT_MTP
            cfg.mtp = B.mtp_desc(target_w["mtp"])
        elif drafter == "ngram":
            cfg.draft_kind = B.DRAFT_NGRAM
        elif drafter == "none":
            cfg.draft_kind = B.DRAFT_NONE
        else:
            raise ValueError(f"drafter {drafter!r}")
        cfg.ngram = B.spec_ngram_cfg(int(ngram[0]), int(ngram[1]))
        cfg.sampler = B.sampler(temperature, top_k, top_p)
        cfg.seed = seed
        cfg.max_batch, cfg.max_ctx, cfg.max_k = max_batch, max_ctx, max_k
        self.cfg = cfg
        self.weights = (target_w, draft_w)        # keep the borrowed weights alive
        self.target_shape, self.draft_shape = target_shape, draft_shape
        # a stream of its own (default priority) so that draft/verify can be graph-replayed
        self.stream = stream if stream is not None else torch.cuda.Stream()
        nbytes = B.spec_workspace_size(cfg)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        base = self.workspace.data_ptr()
        aligned = (base + 255) // 256 * 256
        self.stream.wait_stream(torch.cuda.current_stream())
        self.ctx = B.spec_init(cfg, aligned, nbytes, self.stream)
        self.greedy = temperature <= 0.0
        self.cap = 1 if self.greedy else top_k
        self.vocab = target_shape.vocab
        self.max_batch, self.max_k = max_batch, max_k

    def close(self):
        if self.ctx:
            B.spec_destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- starts
    def _enter(self):
        """Order the engine stream after work already queued on the caller's stream."""
        self.stream.wait_stream(torch.cuda.current_stream())
        return torch.cuda.stream(self.stream)

    def _hold(self, *tensors):
        """The library reads these caller tensors on the engine stream, after the call returns:
        keep their memory from being reused by the caching allocator (which tracks only the
        stream that allocated it) until that work has run."""
        for t in tensors:
            if t is not None and t.is_cuda:
                t.record_stream(self.stream)

    def prefill(self, tokens: torch.Tensor):
        """tokens: int32 [batch, P] on the device."""
        with self._enter():
            b, P = tokens.shape
            B.spec_prefill(self.ctx, tokens, b, P)
            self._hold(tokens)

    def load_prefix(self, which: int, seq: int, k: torch.Tensor, v: torch.Tensor, length: int):
        with self._enter():
            B.spec_load_kv(self.ctx, which, seq, k, v, length)
            self._hold(k, v)

    def set_last(self, last_tok: torch.Tensor, prev_tok: Optional[torch.Tensor] = None,
                 hidden: Optional[torch.Tensor] = None):
        """hidden: float32 [batch, d] target hidden state at L-1 (the MTP drafter)."""
        with self._enter():
            B.spec_set_last(self.ctx, last_tok, prev_tok, hidden, last_tok.shape[0])
            self._hold(last_tok, prev_tok, hidden)

    def load_history(self, seq: int, tokens: torch.Tensor):
        """Token history (int32, device) of sequence seq at positions 0..len-1."""
        with self._enter():
            B.spec_load_history(self.ctx, seq, tokens, int(tokens.numel()))
            self._hold(tokens)

    # ---- one cycle
    def buffers(self, batch: int, k: int):
        """Views of this batch's cycle buffers, sized once for max_k.  The accepted counts,
        near-tie flags, emitted tokens and drafts share one int32 device array (each region
        256-byte aligned), so a cycle's results come back in one copy."""
        if getattr(self, "_buf_batch", None) != batch:
            dev, mk = "cuda", max(self.max_k, 1)
            sizes = dict(n=batch, tie=(batch + 3) // 4, out=batch * (mk + 1), draft=batch * mk)
            self._off, o = {}, 0
            for name, sz in sizes.items():
                self._off[name] = o
                o += (sz + 63) // 64 * 64
            self._dev = torch.zeros((o,), dtype=torch.int32, device=dev)
            self._host = [torch.zeros((o,), dtype=torch.int32, pin_memory=True) for _ in range(2)]
            d, off = self._dev, self._off
            self._flat = dict(
                draft=d[off["draft"]: off["draft"] + batch * mk],
                q=B.Probs(batch * mk, self.cap),
                p=B.Probs(batch * (mk + 1), self.cap),
                n=d[off["n"]: off["n"] + batch],
                out=d[off["out"]: off["out"] + batch * (mk + 1)],
                tie=d[off["tie"]: off["tie"] + sizes["tie"]].view(torch.uint8)[:batch],
            )
            self._buf_batch = batch
            self._logits = {}
        f = self._flat
        kk = max(k, 1)
        return dict(draft=f["draft"][: batch * kk].view(batch, kk), q=f["q"], p=f["p"], n=f["n"],
                    out=f["out"][: batch * (k + 1)].view(batch, k + 1), tie=f["tie"])

    def _results(self, h: torch.Tensor, batch: int, k: int, kk: int) -> Cycle:
        """A cycle's results from a host copy h of the packed array: k tokens verified per
        sequence, drafts stored at row stride kk."""
        off = self._off
        n = h[off["n"]: off["n"] + batch].tolist()
        tie = h[off["tie"]:].view(torch.uint8)[:batch].tolist()
        out = h[off["out"]: off["out"] + batch * (k + 1)].view(batch, k + 1).tolist()
        dr = h[off["draft"]: off["draft"] + batch * kk].view(batch, kk).tolist()
        return Cycle(drafts=[row[:k] for row in dr], n=n, tokens=[out[b][: n[b] + 1] for b in range(batch)],
                     near_tie=tie)

    def cycle(self, batch: int, k: int, rnd: int, drafts: Optional[torch.Tensor] = None,
              keep: bool = False, sync: bool = True, events: Optional[dict] = None) -> Optional[Cycle]:
        """draft_step (unless ``drafts`` are given) -> verify_step -> accept -> kv_trim.
        ``events``: a dict that receives (start, end) CUDA events of each call, recorded on
        the engine stream."""
        with self._enter():
            c = self._cycle(batch, k, rnd, drafts, keep, sync, events)
            return c if sync else None

    def _mark(self, events, name, i):
        if events is not None:
            if name not in events:
                events[name] = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            events[name][i].record(self.stream)

    def _cycle(self, batch, k, rnd, drafts, keep, sync, events=None):
        buf = self.buffers(batch, k)
        kk0 = max(k, 1)
        if k > 0:
            if drafts is None:
                self._mark(events, "draft", 0)
                found = B.draft_step(self.ctx, batch, k, rnd, buf["draft"], buf["q"])
                self._mark(events, "draft", 1)
                if self.drafter == "ngram" and batch == 1 and found < k:
                    # verify only what the lookup found (one sequence: the row stride is moot)
                    k = found
                    buf = dict(buf, out=buf["out"].view(-1)[: batch * (k + 1)].view(batch, k + 1))
            else:
                if not self.greedy:
                    raise ValueError("explicit drafts are supported with the greedy sampler")
                d32 = drafts.to(torch.int32)
                buf["draft"].copy_(d32)
                self._hold(d32, drafts)
        logits = None
        if keep:
            logits = self._logits.get(k)
            if logits is None:
                logits = self._logits[k] = torch.empty((batch, k + 1, self.vocab), dtype=torch.float32,
                                                       device="cuda")
        self._mark(events, "verify", 0)
        B.verify_step(self.ctx, buf["draft"] if k > 0 else None, batch, k, logits, buf["p"])
        self._mark(events, "verify", 1)
        self._mark(events, "accept", 0)
        B.accept(self.ctx, buf["draft"] if k > 0 else None, buf["q"] if k > 0 else None, buf["p"],
                 batch, k, rnd, buf["n"], buf["out"], buf["tie"])
        B.kv_trim(self.ctx, buf["n"], batch)
        self._mark(events, "accept", 1)
        if not sync:
            return k, kk0
        h = self._host[0]
        h.copy_(self._dev, non_blocking=True)
        self.stream.synchronize()
        c = self._results(h, batch, k, kk0)
        if keep:
            c.logits = logits.clone()
            c.p = buf["p"].to_lists(batch * (k + 1))
            c.q = buf["q"].to_lists(batch * k) if k > 0 else []
        return c

    def run(self, batch: int, k: int, rnd0: int, n_cycles: int, time_verify: bool = False) -> List[Cycle]:
        """n_cycles cycles at a fixed k with the next cycle queued before the host reads the
        current one: each cycle's packed results are copied to one of two pinned host arrays
        behind its kernels, and the host parses cycle r while the device runs cycle r + 1.
        Lengths and last tokens live on the device, so nothing of cycle r is needed to queue
        cycle r + 1 (the n-gram drafter reads its match count back and is excluded).
        ``time_verify`` stores each cycle's verify_step time (ms, events on the engine
        stream) in Cycle.verify_ms.  Tokens are the same as n_cycles calls of ``cycle``."""
        if self.drafter == "ngram" and k > 0:
            raise ValueError("the n-gram drafter reads its match count back every cycle; use cycle()")
        cycles: List[Cycle] = []
        evs = [{}, {}] if time_verify else [None, None]
        pending = None
        with self._enter():
            for r in range(n_cycles):
                slot = r % 2
                kv, kk = self._cycle(batch, k, rnd0 + r, None, False, False, evs[slot])
                self._host[slot].copy_(self._dev, non_blocking=True)
                done = torch.cuda.Event()
                done.record(self.stream)
                if pending is not None:
                    cycles.append(self._collect(*pending))
                pending = (slot, done, batch, kv, kk, evs[slot])
            if pending is not None:
                cycles.append(self._collect(*pending))
        return cycles

    def _collect(self, slot, done, batch, k, kk, ev):
        done.synchronize()
        c = self._results(self._host[slot], batch, k, kk)
        if ev is not None:
            c.verify_ms = ev["verify"][0].elapsed_time(ev["verify"][1])
        return c

    def generate(self, n_new: int, k: int, batch: int = 1, rnd0: int = 0, keep: bool = False,
                 teacher: Optional[Sequence[int]] = None, gate: Optional["B.Gate"] = None):
        """Run cycles until every sequence emitted n_new tokens (batch 1 for ``teacher`` and
        ``gate``).  ``gate`` (the n-gram acceptance gate B.Gate, or the adaptive draft length
        B.Depth) picks each cycle's k and is told its outcome.
        Returns (tokens [batch][n_new], cycles)."""
        out = [[] for _ in range(batch)]
        cycles = []
        rnd = rnd0
        while min(len(o) for o in out) < n_new:
            drafts = None
            if gate is not None:
                k = gate.choose()
            if teacher is not None and k > 0:
                done = len(out[0])
                t = list(teacher[done: done + k])
                t += [0] * (k - len(t))
                drafts = torch.tensor([t], dtype=torch.int32, device="cuda")
            c = self.cycle(batch, k, rnd, drafts=drafts, keep=keep)
            if gate is not None:
                gate.update(c.n[0], len(c.drafts[0]))
            for b in range(batch):
                out[b].extend(c.tokens[b])
            cycles.append(c)
            rnd += 1
        return [o[:n_new] for o in out], cycles

    def profile(self, enable: bool):
        B.spec_profile(self.ctx, enable)

    def profile_read(self):
        return B.spec_profile_read(self.ctx)

    def profile_repeat(self, slot_name: str, reps: int):
        B.spec_profile_repeat(self.ctx, slot_name, reps)

    def set_draft_controls(self, p_min: float = 0.0, min_draft: int = 0):
        """Draft probability and min draft of the next cycles (see spec_draft_controls); the k
        of each cycle is the most drafts."""
        B.spec_draft_controls(self.ctx, p_min, min_draft)

    def set_schedule(self, schedule: str):
        """'step', 'stream' (the default) or 'forward' (see spec_set_schedule)."""
        B.spec_set_schedule(self.ctx, schedule)

    def use_graphs(self, enable: bool):
        B.spec_use_graphs(self.ctx, enable)

    def use_gemv(self, enable: bool):
        """The draft model's one- and two-row projections on the vector ALUs (True, the
        default) or on the MFMA weight-streaming kernels (False)."""
        B.spec_use_gemv(self.ctx, enable)

    def stats(self):
        return B.spec_get_stats(self.ctx)

    def read_buffer(self, which: int, buffer: int, shape, dtype=torch.float32) -> torch.Tensor:
        """A device copy of the start of one of the context's activation buffers (see
        spec_debug_read), viewed as ``shape`` of ``dtype``."""
        out = torch.empty(shape, dtype=dtype, device="cuda")
        with self._enter():
            B.spec_debug_read(self.ctx, which, buffer, out, out.numel() * out.element_size())
        self.stream.synchronize()
        return out

    def draft_logits(self, batch: int, k: int) -> torch.Tensor:
        """[k, batch, vocab] float32: the draft model's logits row that draft j + 1 of each
        sequence was drawn from in the last draft_step over ``batch`` sequences and ``k`` drafts
        (see SPEC_BUF_LOGITS)."""
        rows = self.read_buffer(1, B.BUF_LOGITS, ((k + 1) * batch, self.draft_shape.vocab))
        first = rows[: 2 * batch].view(batch, 2, -1)[:, 1]
        return torch.stack([first] + [rows[j * batch:(j + 1) * batch] for j in range(2, k + 1)])

    def lengths(self, batch: int):
        return B.spec_get_lengths(self.ctx, batch)
