"""Reference model of the host step composer, as a plain Python simulation.

TEST INFRASTRUCTURE (see the package docstring). It states the scheduling
policy step by step so that the native composer's integer output (slot ids,
block tables, row order, admissions, retirements) can be compared with it
bit for bit.

Policy (Go under the hood, section 20.3.2, Forma's scheduler and batch):
  * Admission with reservation: a request is admitted only when a slot is
    free AND the pool can hold its prompt AND its answer, so every admitted
    request can finish; all of its blocks are taken at admission
    (ceil((prompt + max_new) / block_size) blocks).
  * Step composition: prefill chunks of sequences that have no first token
    yet go first (FCFS by arrival), each up to chunk_size rows and cut to
    the remaining row budget; then one row per decoding sequence while rows
    remain, the sequences that have waited longest for a row first (ties in
    ascending slot order). A sequence that does not fit waits and goes first
    in the next step; nothing is evicted.
  * Free-slot-only admission (the figure's third case): admit whenever a
    slot is free and take blocks only when a row first writes into a new
    block; a row whose block cannot be had waits. When no row can run the
    schedule is stalled: slots full, pool empty, no sequence can grow.
  * Request-level batching (the figure's first case): a new group is
    admitted only when the batch is empty; blocks are reserved as above.
Pacing of prefill against decode (the step's composition), three readings:
  * PREFILL_FIRST (Forma, Go under the hood 20.3.2): as above.
  * ALBATROSS (RWKV-Runner Albatross article, worker main loop steps 4-5 and
    the pacing parameters after them): no more than max_prefill sequences
    may be in prefill at once -- admission stops there (default
    max(floor(0.125 * slots), 1)); a step takes the decode rows first; then
    every prompt shorter than min_forward_seq_len (default 10) advances by
    one token (single-token prefill beside the decode rows); then, only on a
    "sequence-prefill" step, the longer prompts advance by a chunk each. A
    step is a sequence-prefill step when the countdown is 0 or the step has
    no decode rows; a sequence-prefill step that ran a chunk beside decode
    rows sets the countdown to decode_prefill_ratio (default 5), and every
    other step with decode rows lowers it by one -- so about five decode
    steps pass between chunks of a long prompt.
  * SEPARATE (the Kestrel engine prefills under the engine mutex, apart from
    the batched forward: "0.8MB 跑通 Qwen" 14-1 section 2): while any
    admitted sequence still has prompt left, the step carries only prefill
    chunks (arrival order); otherwise only decode rows.
Allocators: slots go lowest free id first; blocks come from a FIFO free
list seeded with a given order; freed blocks are appended in table order.
Positions, ctx_len and step ids: a sequence's ctx_len counts positions
already cached; a decode row feeds the last generated token at position
ctx_len; step id = number of tokens generated so far.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

RESERVE, FREE_SLOT, REQUEST_LEVEL = 0, 1, 2
PREFILL_FIRST, ALBATROSS, SEPARATE = 0, 1, 2
FINISH_EOS, FINISH_LENGTH, FINISH_ABORT = 1, 2, 3


@dataclass
class Req:
    request_id: int
    prompt: list
    max_new: int
    slot: int = -1
    blocks: list = field(default_factory=list)
    ctx: int = 0            # positions cached
    prefilled: int = 0      # prompt tokens cached
    generated: list = field(default_factory=list)
    admitted_step: int = -1
    last_row_step: int = -1  # last step that gave this sequence a row


@dataclass
class Plan:
    slots: list
    block_tables: list      # per sequence, its block ids (unpadded)
    ctx_lens: list
    n_new: list
    tokens: list
    want_token: list
    step_ids: list
    request_ids: list
    stalled: bool = False

    @property
    def n_rows(self):
        return sum(self.n_new)


def ceil_div(a, b):
    return -(-a // b)


class ComposerRef:
    def __init__(self, max_slots, block_size, num_blocks, max_rows, chunk_size,
                 eos_id, policy=RESERVE, block_order=None, max_blocks_per_seq=None,
                 pacing=PREFILL_FIRST, max_prefill=0, decode_prefill_ratio=0,
                 min_forward_seq_len=0):
        self.pacing = pacing
        self.max_prefill = max_prefill or max(int(max_slots * 0.125), 1)
        self.decode_prefill_ratio = decode_prefill_ratio or 5
        self.min_forward_seq_len = min_forward_seq_len or 10
        self.countdown = 0
        self.max_slots, self.bs, self.num_blocks = max_slots, block_size, num_blocks
        self.max_rows, self.chunk, self.eos, self.policy = max_rows, chunk_size, eos_id, policy
        self.max_blocks_per_seq = max_blocks_per_seq or num_blocks
        self.free_blocks = deque(block_order if block_order is not None else range(num_blocks))
        self.free_slots = set(range(max_slots))
        self.queue: deque = deque()
        self.active: dict = {}      # slot -> Req
        self.order = []             # admitted sequences in arrival order
        self.finished = []          # (request_id, reason, generated)
        self.step = 0
        self.last_plan = None

    # -------------------------------------------------------------- intake
    def submit(self, request_id, prompt, max_new):
        if len(prompt) < 1 or max_new < 1:
            raise ValueError("empty prompt or max_new < 1")
        need = ceil_div(len(prompt) + max_new, self.bs)
        if need > self.max_blocks_per_seq or need > self.num_blocks:
            raise ValueError("request can never fit")
        self.queue.append(Req(request_id, list(prompt), max_new))

    def abort(self, request_id):
        for slot, r in list(self.active.items()):
            if r.request_id == request_id:
                self._retire(r, FINISH_ABORT)
                return True
        for r in list(self.queue):
            if r.request_id == request_id:
                self.queue.remove(r)
                self.finished.append((request_id, FINISH_ABORT, []))
                return True
        return False

    # --------------------------------------------------------------- plan
    def _admit(self):
        if self.policy == REQUEST_LEVEL and self.active:
            return
        while self.queue and self.free_slots:
            if self.pacing == ALBATROSS and \
                    sum(1 for x in self.order if x.prefilled < len(x.prompt)) >= self.max_prefill:
                break
            r = self.queue[0]
            if self.policy in (RESERVE, REQUEST_LEVEL):
                need = ceil_div(len(r.prompt) + r.max_new, self.bs)
                if len(self.free_blocks) < need:
                    break
                r.blocks = [self.free_blocks.popleft() for _ in range(need)]
            self.queue.popleft()
            r.slot = min(self.free_slots)
            self.free_slots.remove(r.slot)
            r.admitted_step = self.step
            self.active[r.slot] = r
            self.order.append(r)

    def _grow(self, r, n_pos):
        """Free-slot-only policy: make sure r holds blocks for n_pos positions."""
        need = ceil_div(n_pos, self.bs) - len(r.blocks)
        if need <= 0:
            return True
        if len(self.free_blocks) < need:
            return False
        r.blocks += [self.free_blocks.popleft() for _ in range(need)]
        return True

    def plan(self) -> Plan:
        self._admit()
        p = Plan([], [], [], [], [], [], [], [])
        self._budget = self.max_rows
        if self.pacing == ALBATROSS:
            n_dec = self._decode_rows(p)
            for r in self.order:      # short prompts: one token per step
                if len(r.prompt) < self.min_forward_seq_len:
                    self._chunk(p, r, 1)
            if self.countdown == 0 or n_dec == 0:
                ran = False
                for r in self.order:  # long prompts: a chunk on this step
                    if len(r.prompt) >= self.min_forward_seq_len:
                        ran = self._chunk(p, r, self.chunk) or ran
                if ran and n_dec > 0:
                    self.countdown = self.decode_prefill_ratio
            else:
                self.countdown -= 1
        elif self.pacing == SEPARATE:
            for r in self.order:
                self._chunk(p, r, self.chunk)
            if not p.n_new:
                self._decode_rows(p)
        else:
            # prefill chunks first, FCFS by arrival; then the decode rows
            for r in self.order:
                self._chunk(p, r, self.chunk)
            self._decode_rows(p)
        p.stalled = (not p.n_new) and bool(self.active)
        self.last_plan = p
        return p

    def _chunk(self, p, r, limit):
        """A prefill chunk of r: up to `limit` prompt tokens, cut to the row
        budget; free-slot admission takes its blocks first."""
        left = len(r.prompt) - r.prefilled
        n = min(limit, left, self._budget)
        if r.slot < 0 or n <= 0:
            return False
        if self.policy == FREE_SLOT and not self._grow(r, r.ctx + n):
            return False
        self._emit(p, r, r.prompt[r.prefilled:r.prefilled + n], r.prefilled + n == len(r.prompt))
        self._budget -= n
        return True

    def _decode_rows(self, p):
        """One row per decoding sequence while rows remain, the sequences
        that waited longest first (ties by slot). Returns the rows taken."""
        taken = 0
        dec = [r for r in self.active.values() if r.prefilled >= len(r.prompt)]
        for r in sorted(dec, key=lambda r: (r.last_row_step, r.slot)):
            if self._budget <= 0:
                break
            if self.policy == FREE_SLOT and not self._grow(r, r.ctx + 1):
                continue
            self._emit(p, r, [r.generated[-1]], True)
            self._budget -= 1
            taken += 1
        return taken

    def _emit(self, p, r, toks, want):
        r.last_row_step = self.step
        p.slots.append(r.slot)
        p.block_tables.append(list(r.blocks))
        p.ctx_lens.append(r.ctx)
        p.n_new.append(len(toks))
        p.tokens += toks
        p.want_token.append(1 if want else 0)
        p.step_ids.append(len(r.generated))
        p.request_ids.append(r.request_id)

    # ------------------------------------------------------------- commit
    def commit(self, tokens_out):
        p = self.last_plan
        o = 0
        retire = []
        for i, slot in enumerate(p.slots):
            r = self.active[slot]
            r.ctx += p.n_new[i]
            if r.prefilled < len(r.prompt):
                r.prefilled += p.n_new[i]
            if p.want_token[i]:
                t = int(tokens_out[o])
                o += 1
                r.generated.append(t)
                if t == self.eos:
                    retire.append((r, FINISH_EOS))
                elif len(r.generated) >= r.max_new:
                    retire.append((r, FINISH_LENGTH))
        for r, why in retire:
            self._retire(r, why)
        self.step += 1
        self.last_plan = None

    def _retire(self, r, why):
        del self.active[r.slot]
        self.free_slots.add(r.slot)
        self.free_blocks.extend(r.blocks)
        r.blocks = []
        self.order.remove(r)
        self.finished.append((r.request_id, why, list(r.generated)))
        r.slot = -1
