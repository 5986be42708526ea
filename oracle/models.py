"""Bit-level models of the barrier-free protocols (LL, Sentinel, LL128 atomic,
double buffering with implicit credits).

TEST INFRASTRUCTURE ONLY (see the package docstring).  These are written from
the prose of "Every Microsecond Matters: Achieving Near Speed-of-Light Latency
in GPU Collectives" (agihunt.info summary), the four protocol paragraphs:

* LL: an 8-byte flag and 8 bytes of data leave in one 16-byte write, so seeing
  the flag means the data is there.  Half the bandwidth, twice the staging.
* Sentinel: the receive buffer is prefilled with a value data should not take
  (the page's example is -NaN); a change of value means arrival; the buffer
  must be reset after use and data must never equal the sentinel.
* Bidirectional + double buffering: a chunk received from the peer is the
  permission to send the next one, and two alternating buffers remove the
  barrier between iterations.
* Two-shot LL128 atomic: reduce-scatter + all-gather; groups of 8 threads per
  128-byte line; the group's first thread sets its own element to 1 as the
  flag; all 8 atomically add into staging; the line is complete when the flag
  sums to N; about D/N staging; waste about 1.5 % (FP16) and 3 % (FP32).

Readings where the page is silent: LL words are laid out [data0, epoch, data1, epoch] with a
monotone non-zero epoch; the sentinel is the all-ones pattern (a negative NaN
in all three formats) and producers replace a datum equal to it by the
all-ones-minus-one pattern (still a negative NaN); the LL128 flag is 1.0 in
the staging type in slot 0 of the line; element e lives in line e // K, slot
1 + e % K with K = 128 / sizeof(A) - 1; owners hold contiguous balanced line
ranges; the consumer zeroes a line after reading it.
"""
from __future__ import annotations

import itertools
import math
from dataclasses import dataclass, field

import numpy as np

from . import F32, F16, BF16, ELEM_BYTES, BITS_DTYPE, decode, round_to

# ----------------------------------------------------------------------------
# LL: 16-byte line = 8 bytes payload + 8 bytes flag
# ----------------------------------------------------------------------------
LL_LINE_BYTES = 16
LL_PAYLOAD_BYTES = 8


EPOCH_LAST = 0x7FFFFFFF       # last epoch of a range; 0 means 'never written'
DEVICE_EPOCH_BIT = 0x80000000


def next_epoch(e: int, last: int = EPOCH_LAST) -> int:
    """Host-numbered epochs run 1, 2, ..., last, 1, ... (last = 2^31 - 1).
    A smaller `last` gives the same policy on a short cycle for the models
    below."""
    e = e + 1
    return 1 if e > last else e


def next_device_epoch(e: int) -> int:
    """Device-numbered epochs run 2^31 + (1 .. 2^31 - 1): the host range with
    the top bit set, so the two ranges never meet."""
    return DEVICE_EPOCH_BIT | next_epoch(e & EPOCH_LAST)


def epoch_wraps(e: int, last: int = EPOCH_LAST) -> bool:
    """True for the last epoch of a range: the next use reuses a value."""
    return (e & EPOCH_LAST) == last


class LLRegion:
    """A receive buffer of LL lines reused by a sequence of calls, with the
    epoch policy above.  The LL paragraph makes the flag the only arrival
    signal, so a line the consumer accepts must have been written by the
    producer of the same call.  A call of `n_lines` lines with epoch e has
    its producer write lines [0, n_lines) with e; before that, the consumer
    may look at any of them.  `stale_hits` records lines the consumer would
    accept although this call's producer has not written them yet.

    clear_at_wrap=True zeroes the region before the first call after a wrap
    (what the library does); False keeps it (the failure mode)."""

    def __init__(self, n_lines: int, last: int = EPOCH_LAST, clear_at_wrap: bool = True):
        self.flags = np.zeros(n_lines, dtype=np.int64)  # epoch word of each line (0 = zeroed)
        self.last = last
        self.clear_at_wrap = clear_at_wrap
        self.epoch = 1
        self.pending_clear = False
        self.stale_hits = 0

    def call(self, n_lines: int) -> int:
        """One call over the first n_lines lines; returns the stale lines the
        consumer could have accepted before the producer wrote them."""
        if self.pending_clear:
            self.flags[:] = 0
            self.pending_clear = False
        e = self.epoch
        hits = int(np.count_nonzero(self.flags[:n_lines] == e))
        self.stale_hits += hits
        self.flags[:n_lines] = e
        if epoch_wraps(e, self.last) and self.clear_at_wrap:
            self.pending_clear = True
        self.epoch = next_epoch(e, self.last)
        return hits


def ll_pack(payload_words: np.ndarray, epoch: int) -> np.ndarray:
    """(L, 2) uint32 payload words -> (L, 4) uint32 lines [d0, e, d1, e]."""
    p = np.asarray(payload_words, dtype=np.uint32).reshape(-1, 2)
    lines = np.empty((p.shape[0], 4), dtype=np.uint32)
    lines[:, 0] = p[:, 0]
    lines[:, 1] = epoch
    lines[:, 2] = p[:, 1]
    lines[:, 3] = epoch
    return lines


def ll_unpack(lines: np.ndarray, epoch: int):
    """(L, 4) lines -> (valid[L], payload (L, 2)).  A line is valid only when
    both flag words carry the expected epoch (either 8-byte half may land
    first)."""
    ln = np.asarray(lines, dtype=np.uint32).reshape(-1, 4)
    valid = (ln[:, 1] == epoch) & (ln[:, 3] == epoch)
    return valid, ln[:, [0, 2]].copy()


def ll_payload_words(partial_bits: np.ndarray) -> np.ndarray:
    """A partial's bytes, zero-padded to whole 8-byte payloads, as (L, 2) u32."""
    raw = np.ascontiguousarray(partial_bits).view(np.uint8)
    n_lines = -(-raw.size // LL_PAYLOAD_BYTES)
    buf = np.zeros(n_lines * LL_PAYLOAD_BYTES, dtype=np.uint8)
    buf[: raw.size] = raw
    return buf.view(np.uint32).reshape(n_lines, 2)


def ll_staging_bytes(message_bytes: int) -> int:
    """Staging for one message: one 16-byte line per 8 payload bytes."""
    return -(-message_bytes // LL_PAYLOAD_BYTES) * LL_LINE_BYTES


# ----------------------------------------------------------------------------
# Sentinel
# ----------------------------------------------------------------------------
SENTINEL_BITS = {F32: 0xFFFFFFFF, F16: 0xFFFF, BF16: 0xFFFF}


def sentinel_canon(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Replace the sentinel pattern by the pattern one below it (both NaN)."""
    s = SENTINEL_BITS[dtype]
    b = np.asarray(bits, dtype=BITS_DTYPE[dtype])
    return np.where(b == s, BITS_DTYPE[dtype](s - 1), b).astype(BITS_DTYPE[dtype])


def sentinel_ready(bits: np.ndarray, dtype: int) -> np.ndarray:
    return np.asarray(bits) != SENTINEL_BITS[dtype]


def sentinel_reset(n_elems: int, dtype: int) -> np.ndarray:
    return np.full(n_elems, SENTINEL_BITS[dtype], dtype=BITS_DTYPE[dtype])


# ----------------------------------------------------------------------------
# Point-to-point transfer over the LL and Sentinel wires
# ----------------------------------------------------------------------------
def p2p_transfer(send_bits: np.ndarray, dtype: int, wire: str, epoch: int = 1) -> np.ndarray:
    """What the receiver of a one-producer LL or Sentinel transfer writes out.

    The pwwt.cn small-message latency article (section 1.1, the pipeline
    parallel item; section 3.3, an 8 KB hidden state per token) has pipeline
    stages pass activations by send/recv; the LL and Sentinel paragraphs of
    the agihunt.info summary give the two wires.  LL: pack the payload with
    the epoch, unpack it once both flags carry that epoch.  Sentinel: the
    producer canonicalises, the receiver waits until no element holds the
    sentinel and takes the staged value.
    """
    b = np.ascontiguousarray(np.asarray(send_bits, dtype=BITS_DTYPE[dtype]))
    nbytes = b.size * ELEM_BYTES[dtype]
    if wire == "ll":
        valid, payload = ll_unpack(ll_pack(ll_payload_words(b), epoch), epoch)
        assert valid.all()
        raw = np.ascontiguousarray(payload).reshape(-1).view(np.uint8)[:nbytes]
        return raw.view(BITS_DTYPE[dtype]).copy()
    if wire == "sentinel":
        staged = sentinel_canon(b, dtype)
        assert sentinel_ready(staged, dtype).all()
        return staged
    raise ValueError("unknown wire %r" % (wire,))


def all_gather(fragments, dtype: int, wire: str) -> np.ndarray:
    """What every receiving rank of an AllGather holds: all ranks' fragments
    back to back in rank order (the yololab.net article's collective table:
    every rank collects every rank's piece), each as it arrives over the wire
    (``p2p_transfer``); the receiver treats its own fragment the same way so
    that every copy agrees."""
    return np.concatenate([p2p_transfer(f, dtype, wire) for f in fragments])


# ----------------------------------------------------------------------------
# LL128 atomic two-shot
# ----------------------------------------------------------------------------
LL128_LINE_BYTES = 128
LL128_LANES = 8            # threads per line
LL128_LANE_BYTES = 16


@dataclass(frozen=True)
class LL128Geometry:
    n: int                 # elements per rank
    n_ranks: int
    acc_bytes: int         # bytes per staging slot (4 for fp32, 2 for 16-bit)

    @property
    def slots(self) -> int:
        return LL128_LINE_BYTES // self.acc_bytes

    @property
    def k(self) -> int:     # data slots per line
        return self.slots - 1

    @property
    def lines(self) -> int:
        return -(-self.n // self.k)

    def owner_range(self, s: int):
        ln = self.lines
        return (s * ln) // self.n_ranks, ((s + 1) * ln) // self.n_ranks

    def owner_of_line(self, line: int) -> int:
        for s in range(self.n_ranks):
            a, b = self.owner_range(s)
            if a <= line < b:
                return s
        raise IndexError(line)

    def line_slot(self, e: int):
        return e // self.k, 1 + e % self.k

    @property
    def waste(self) -> float:
        """Fraction of every line spent on the flag."""
        return 1.0 / self.slots

    @property
    def staging_bytes(self) -> int:
        return self.lines * LL128_LINE_BYTES

    def max_owner_staging_bytes(self) -> int:
        return max(b - a for a, b in (self.owner_range(s) for s in range(self.n_ranks))) * LL128_LINE_BYTES


def _acc_add(a: np.ndarray, b: np.ndarray, acc: int) -> np.ndarray:
    """One atomic add in the staging type, correctly rounded."""
    if acc == F32:
        return (a.astype(np.float32) + b.astype(np.float32)).astype(np.float32)
    # 16-bit staging: the binary64 sum of two 16-bit values is exact up to a
    # single rounding of the binary64 sum (both fit comfortably), then round
    # to the 16-bit format.
    s = a.astype(np.float64) + b.astype(np.float64)
    return decode(round_to(s, acc), acc)


def ll128_staging_image(partials_bits: np.ndarray, dtype: int, acc: int, order=None) -> np.ndarray:
    """Staging contents (L, slots) as binary64 values after every rank's atomic
    contribution, applied rank by rank in ``order`` with rounding to the
    staging type after each add."""
    parts = np.asarray(partials_bits)
    n_ranks, n = parts.shape
    g = LL128Geometry(n, n_ranks, ELEM_BYTES[acc])
    order = list(range(n_ranks)) if order is None else list(order)
    stage = np.zeros((g.lines, g.slots), dtype=np.float64)
    for r in order:
        contrib = np.zeros((g.lines, g.slots), dtype=np.float64)
        contrib[:, 0] = 1.0
        vals = decode(parts[r], dtype)
        if acc != dtype:
            # conversion to the staging type (exact when widening)
            vals = decode(round_to(vals, acc), acc)
        flat = np.zeros(g.lines * g.k, dtype=np.float64)
        flat[:n] = vals
        contrib[:, 1:] = flat.reshape(g.lines, g.k)
        stage = _acc_add(stage, contrib, acc).astype(np.float64)
    return stage


def ll128_result(stage: np.ndarray, n: int, dtype: int) -> np.ndarray:
    """All-gather half: read each data slot back and round it to the output type."""
    data = stage[:, 1:].reshape(-1)[:n]
    return round_to(data, dtype)


def ll128_error_bound(partials_bits: np.ndarray, dtype: int, acc: int) -> np.ndarray:
    """|staged sum - exact sum| <= (N-1) * u_A * sum_r |p_r| for any add order
    (the first add lands on zero and is exact), plus half an ulp of the output
    type when the staging type differs from it."""
    parts = np.asarray(partials_bits)
    n_ranks = parts.shape[0]
    absum = np.zeros(parts.shape[1], dtype=np.float64)
    for r in range(n_ranks):
        absum += np.abs(decode(parts[r], dtype))
    u = {F32: 2.0 ** -24, F16: 2.0 ** -11, BF16: 2.0 ** -8}[acc]
    bound = (n_ranks - 1) * u * absum * (1 + 1e-12)
    if acc != dtype:
        p = {F32: 24, F16: 11, BF16: 8}[dtype]
        exact = np.abs(sum(decode(parts[r], dtype) for r in range(n_ranks)))
        bound = bound + (exact + bound) * 2.0 ** (-p) + (2.0 ** -149 if dtype == F32 else 2.0 ** -133 if dtype == BF16 else 2.0 ** -24)
    return bound


# ----------------------------------------------------------------------------
# Double buffering with implicit credits: a small model checker
# ----------------------------------------------------------------------------
@dataclass
class PipelineResult:
    states: int
    terminal_ok: int
    violations: list = field(default_factory=list)
    deadlocks: int = 0


def check_pipeline(n_ranks: int, slices: int, chunks: int, parities: int = 2,
                   run_ahead: bool = False, split: bool = False, credit_lag: int = 0,
                   max_states: int = 2_000_000) -> PipelineResult:
    """Explore every interleaving of the chunked two-shot schedule.

    Agents are workgroups (rank r, slice w).  Agent program, for c = 0..C-1:
      produce(c): one atomic contribution into line (parity c % P, owner s,
                  slice w) for every owner s (N separate steps);
      consume(c): wait until line (parity c % P, owner r, slice w) has N
                  contributions of chunk c, read it, zero it.
    With ``run_ahead`` the agent produces chunk c+1 before consuming chunk c
    (a schedule without the credit), which must be caught.

    With ``split`` each workgroup is two agents: a producer that may emit
    chunk c only once its own consumer has finished chunk c-1 (the credit,
    passed inside the workgroup), and a consumer that consumes in order.

    A line's state is (chunk it holds, contribution count).  Checked:
      no overwrite -- a contribution for chunk c only lands on a line that is
                      empty or already holds chunk c;
      no early read -- consume(c) only after N contributions of chunk c;
      progress     -- every state with unfinished agents has a move.
    """
    if split:
        return _check_split(n_ranks, slices, chunks, parities, max_states, credit_lag)
    agents = [(r, w) for r in range(n_ranks) for w in range(slices)]

    def program(c_count):
        steps = []
        if not run_ahead:
            for c in range(c_count):
                steps += [("p", c, s) for s in range(n_ranks)]
                steps.append(("c", c, None))
        else:
            steps += [("p", 0, s) for s in range(n_ranks)]
            for c in range(c_count):
                if c + 1 < c_count:
                    steps += [("p", c + 1, s) for s in range(n_ranks)]
                steps.append(("c", c, None))
        return steps

    prog = program(chunks)
    n_lines = parities * n_ranks * slices

    def line_id(par, owner, w):
        return (par * n_ranks + owner) * slices + w

    # line state: (held_chunk or -1 for empty, count)
    init = (tuple([0] * len(agents)), tuple([(-1, 0)] * n_lines))
    res = PipelineResult(states=0, terminal_ok=0)
    seen = set()
    stack = [init]
    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        res.states += 1
        if res.states > max_states:
            raise RuntimeError("state space too large")
        pcs, lines = st
        if all(pc == len(prog) for pc in pcs):
            res.terminal_ok += 1
            continue
        moved = False
        for ai, (r, w) in enumerate(agents):
            pc = pcs[ai]
            if pc == len(prog):
                continue
            kind, c, s = prog[pc]
            par = c % parities
            if kind == "p":
                lid = line_id(par, s, w)
                held, cnt = lines[lid]
                if held not in (-1, c):
                    res.violations.append(("overwrite", (r, w), c, s, held))
                    continue
                if cnt >= n_ranks:
                    res.violations.append(("overflow", (r, w), c, s))
                    continue
                nl = list(lines)
                nl[lid] = (c, cnt + 1)
                npcs = list(pcs)
                npcs[ai] += 1
                stack.append((tuple(npcs), tuple(nl)))
                moved = True
            else:
                lid = line_id(par, r, w)
                held, cnt = lines[lid]
                if held == c and cnt == n_ranks:
                    nl = list(lines)
                    nl[lid] = (-1, 0)
                    npcs = list(pcs)
                    npcs[ai] += 1
                    stack.append((tuple(npcs), tuple(nl)))
                    moved = True
                # otherwise the consumer spins (no move)
        if not moved:
            res.deadlocks += 1
        if res.violations:
            break
    return res


def _check_split(n_ranks, slices, chunks, parities, max_states, credit_lag=0):
    """Model of the wave-specialised schedule: per (rank r, slice w) a
    producer P and a consumer C.  P emits chunk c (one contribution per
    owner, separate steps) only when C has consumed chunks 0..c-1 (C's count
    of finished chunks is >= c); C consumes chunk c when its line holds all N
    contributions of chunk c.  (A weaker credit, count >= c-1, lets P
    overwrite a peer's unconsumed chunk c-2: the checker finds it.)"""
    pairs = [(r, w) for r in range(n_ranks) for w in range(slices)]
    n_lines = parities * n_ranks * slices

    def line_id(par, owner, w):
        return (par * n_ranks + owner) * slices + w

    # state: producer position (chunk, next owner), consumer chunks done, lines
    init = (tuple([(0, 0)] * len(pairs)), tuple([0] * len(pairs)), tuple([(-1, 0)] * n_lines))
    res = PipelineResult(states=0, terminal_ok=0)
    seen, stack = set(), [init]
    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        res.states += 1
        if res.states > max_states:
            raise RuntimeError("state space too large")
        prod, cons, lines = st
        if all(p[0] == chunks for p in prod) and all(c == chunks for c in cons):
            res.terminal_ok += 1
            continue
        moved = False
        for ai, (r, w) in enumerate(pairs):
            c, s = prod[ai]
            if c < chunks and cons[ai] >= c - credit_lag:
                lid = line_id(c % parities, s, w)
                held, cnt = lines[lid]
                if held not in (-1, c):
                    res.violations.append(("overwrite", (r, w), c, s, held))
                    break
                nl = list(lines)
                nl[lid] = (c, cnt + 1)
                npr = list(prod)
                npr[ai] = (c, s + 1) if s + 1 < n_ranks else (c + 1, 0)
                stack.append((tuple(npr), cons, tuple(nl)))
                moved = True
            cc = cons[ai]
            if cc < chunks:
                lid = line_id(cc % parities, r, w)
                held, cnt = lines[lid]
                if held == cc and cnt == n_ranks:
                    nl = list(lines)
                    nl[lid] = (-1, 0)
                    nco = list(cons)
                    nco[ai] = cc + 1
                    stack.append((prod, tuple(nco), tuple(nl)))
                    moved = True
        if res.violations:
            break
        if not moved:
            res.deadlocks += 1
    return res


def check_owner_credit(n_ranks: int, slices: int, chunks: int, buffers: int, cons_waves: int = 1,
                       wave_order: bool = True, credit: str = "owner", lag: int = 0, prod_groups: int = 1,
                       max_states: int = 2_000_000) -> PipelineResult:
    """Model of the owner-credit schedule over B rotating Sentinel buffers.

    Per (rank r, slice w) a producer P and cons_waves consumer waves (or
    groups of waves that take a chunk together).  Chunk c lives in buffer
    c % B; line (buffer, owner s, slice w) collects one contribution per
    rank (the rank's own shard included).
      P emits chunk c (one contribution per owner, separate steps) once the
        credit allows it: credit "owner" -- every owner s has consumed every
        chunk <= c - B; credit "own" -- only P's own consumer has (a weaker
        credit, which the checker must catch); credit "workgroup" -- P's own
        consumers have consumed every chunk < c - lag (the implicit credit of
        the workgroup pipeline: safe with B >= 2 lag + 2 buffers); with
        prod_groups = PG the pair has PG producers, producer p emitting
        chunks p, p + PG, ... (so chunks may be stored out of order);
      consumer wave q consumes chunks q, q + Q, ... in order; with
        ``wave_order`` chunk c also waits until chunk c - B (another wave's,
        the previous user of the line) is consumed.  Like the Sentinel, a
        wave sees only that the line is full, not which chunk filled it, so
        reading a full line that holds another chunk is a stale read.
    Checked: no overwrite, no stale read, progress.
    """
    Q = cons_waves
    pairs = [(r, w) for r in range(n_ranks) for w in range(slices)]
    idx = {p: i for i, p in enumerate(pairs)}
    n_lines = buffers * n_ranks * slices

    def line_id(b, owner, w):
        return (b * n_ranks + owner) * slices + w

    def consumed(cnts, c):  # chunk c consumed by the pair whose wave counts are cnts
        return cnts[c % Q] > c // Q

    def all_below(cnts, x):  # every chunk < x consumed
        return all(consumed(cnts, c) for c in range(min(x, chunks)))

    PG = prod_groups
    init = (tuple((p, 0) for _ in pairs for p in range(PG)), tuple([tuple([0] * Q)] * len(pairs)),
            tuple([(-1, 0)] * n_lines))
    res = PipelineResult(states=0, terminal_ok=0)
    seen, stack = set(), [init]
    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        res.states += 1
        if res.states > max_states:
            raise RuntimeError("state space too large")
        prod, cons, lines = st
        if all(p[0] >= chunks for p in prod) and all(q + cnt * Q >= chunks for cc in cons
                                                     for q, cnt in enumerate(cc)):
            res.terminal_ok += 1
            continue
        moved = False
        for ai, (r, w) in enumerate(pairs):
            for pg in range(PG):
                pi = ai * PG + pg
                c, s = prod[pi]
                if c >= chunks:
                    continue
                need = c - buffers + 1  # chunks below this must be consumed
                if credit == "owner":
                    ok = all(all_below(cons[idx[(o, w)]], need) for o in range(n_ranks))
                elif credit == "workgroup":
                    ok = all_below(cons[ai], c - lag)
                else:
                    ok = all_below(cons[ai], need)
                if not ok:
                    continue
                lid = line_id(c % buffers, s, w)
                held, cnt = lines[lid]
                if held not in (-1, c):
                    res.violations.append(("overwrite", (r, w), c, s, held))
                    break
                nl = list(lines)
                nl[lid] = (c, cnt + 1)
                npr = list(prod)
                npr[pi] = (c, s + 1) if s + 1 < n_ranks else (c + PG, 0)
                stack.append((tuple(npr), cons, tuple(nl)))
                moved = True
            if res.violations:
                break
            for q in range(Q):
                cc = q + cons[ai][q] * Q
                if cc >= chunks:
                    continue
                if wave_order and cc >= buffers and not consumed(cons[ai], cc - buffers):
                    continue
                lid = line_id(cc % buffers, r, w)
                held, cnt = lines[lid]
                if cnt < n_ranks:
                    continue  # not full yet: the wave keeps polling
                if held != cc:
                    res.violations.append(("stale read", (r, w), cc, held))
                    break
                nl = list(lines)
                nl[lid] = (-1, 0)
                nco = list(cons)
                nq = list(cons[ai])
                nq[q] += 1
                nco[ai] = tuple(nq)
                stack.append((prod, tuple(nco), tuple(nl)))
                moved = True
            if res.violations:
                break
        if res.violations:
            break
        if not moved:
            res.deadlocks += 1
    return res


# ----------------------------------------------------------------------------
# Speed-of-light arithmetic and the alpha + beta * size model
# ----------------------------------------------------------------------------
def sol_floor(t_l2_round_trip: float, t_remote_write: float) -> float:
    """Lower bound of one AllReduce: two L2 round trips plus one remote write."""
    return 2.0 * t_l2_round_trip + t_remote_write


def fit_alpha_beta(sizes, times):
    """Least-squares fit of T(size) = alpha + beta * size."""
    x = np.asarray(sizes, dtype=np.float64)
    y = np.asarray(times, dtype=np.float64)
    a = np.vstack([np.ones_like(x), x]).T
    (alpha, beta), *_ = np.linalg.lstsq(a, y, rcond=None)
    return float(alpha), float(beta)
