"""A host-side model of how the library plans the routed waves of an offloaded chunk and
stages them through the ring, for tests that predict the ring's hit and miss counts exactly.
Test infrastructure only.

Per chunk pass: the offloaded experts the chunk uses, ascending, are cut into waves of at most
(n_lines - pinned) // 2; even passes run the waves in ascending order, odd passes in descending
order (and stage each wave's experts top-down). Before wave i runs, waves i and i + 1 are
staged (the second only if enough lines are free); wave i is released after its GEMMs. Staging
marks hits first; each miss evicts the least recently used unheld line that holds no expert a
later wave of the same pass asks for, else the least recently used unheld line.

Per layer call of several chunks (layer()): the experts to pin are chosen from every chunk's
expert set as the library chooses them (choose_pinned), staged first and held until the last
chunk is done; the chunks stream only the others."""
from __future__ import annotations


PIN_SIXTEENTHS = (0, 4, 8, 12, 14, 15)    # shares of the lines a layer call may pin
COPY_PER_WAVE = 8                         # a copy weighs 8 waves in the estimate


def estimate_cost(used, by_freq, H, cap, sweep0):
    """COPY_PER_WAVE x copies + waves with by_freq[:H] pinned and the rest streaming through
    cap lines in waves of cap // 2, least recently used first, chunk passes alternating
    direction from sweep0, holds ignored."""
    hot = set(by_freq[:H])
    last = {}
    clock, copies, waves = 0, H, 0
    per = max(1, cap // 2)
    for c, u in enumerate(used):
        streamed = sum(1 for e in u if e not in hot)
        waves += max(1, (streamed + per - 1) // per)
        seq = u[::-1] if (sweep0 + c) & 1 else u
        for e in seq:
            if e in hot:
                continue
            if e not in last:
                copies += 1
                if len(last) == cap:
                    del last[min(last, key=last.get)]
            clock += 1
            last[e] = clock
    return COPY_PER_WAVE * copies + waves


def choose_pinned(used, n_lines, sweep0):
    """The experts a layer call of several chunks pins (ascending): H = n * PIN_SIXTEENTHS / 16,
    the experts most chunks use first (ties to the lower id), H with the lowest estimated
    cost (ties to the smaller H)."""
    freq = {}
    for u in used:
        for e in u:
            freq[e] = freq.get(e, 0) + 1
    by_freq = sorted(freq, key=lambda e: (-freq[e], e))
    best_h, best = 0, None
    for q, sx in enumerate(PIN_SIXTEENTHS):
        H = min(n_lines * sx // 16, len(by_freq))
        if q > 0 and H == 0:
            continue
        c = estimate_cost(used, by_freq, H, n_lines - H, sweep0)
        if best is None or c < best:
            best, best_h = c, H
    return sorted(by_freq[:best_h])


class RingModel:
    def __init__(self, n_lines: int):
        self.n = n_lines
        self.expert = [None] * n_lines      # (layer, expert) held by each line
        self.last = [0] * n_lines
        self.held = [False] * n_lines
        self.clock = 0
        self.sweeps = 0
        self.hits = 0
        self.misses = 0
        self.pinned_uses = 0                # chunk uses of experts pinned for a layer call
        self.copied = [0, 0, 0, 0]          # misses by kind: initial, ahead, demand, cross-layer
        self.requested = [0, 0, 0, 0]
        self.log = []                       # ("stage", kind, experts, later) / ("release", experts)

    def _stage(self, layer, experts, later):
        where = {k: i for i, k in enumerate(self.expert) if k is not None}
        hit = [where.get((layer, e)) for e in experts]
        misses = sum(h is None for h in hit)
        free = sum(1 for l in range(self.n) if not self.held[l] and l not in set(h for h in hit if h is not None))
        if misses > free:
            return None
        out = [None] * len(experts)
        for i, h in enumerate(hit):
            if h is None:
                continue
            self.held[h] = True
            self.clock += 1
            self.last[h] = self.clock
            self.hits += 1
            out[i] = h
        for i, e in enumerate(experts):
            if hit[i] is not None:
                continue
            best, best_needed = None, None
            for l in range(self.n):
                if self.held[l]:
                    continue
                k = self.expert[l]
                needed = k is not None and k[0] == layer and k[1] in later
                if needed:
                    if best_needed is None or self.last[l] < self.last[best_needed]:
                        best_needed = l
                elif best is None or self.last[l] < self.last[best]:
                    best = l
            v = best if best is not None else best_needed
            self.expert[v] = (layer, e)
            self.held[v] = True
            self.clock += 1
            self.last[v] = self.clock
            self.misses += 1
            out[i] = v
        return out

    def layer(self, layer: int, used_chunks: list[list[int]]):
        """A layer call over chunks with these (ascending) offloaded experts each."""
        pin = choose_pinned(used_chunks, self.n, self.sweeps) if len(used_chunks) >= 2 else []
        lines = []
        if pin:
            m0 = self.misses
            lines = self._stage(layer, pin, set())
            assert lines is not None, "the model could not pin its experts"
            self.log.append(("stage", 0, list(pin), []))
            self.copied[0] += self.misses - m0
            self.requested[0] += len(pin)
        pinset = set(pin)
        for u in used_chunks:
            self.pinned_uses += sum(1 for e in u if e in pinset)
            self.chunk(layer, [e for e in u if e not in pinset], n_pinned=len(pin))
        for l in lines:
            self.held[l] = False
        if pin:
            self.log.append(("release", list(pin)))
        return pin

    def chunk(self, layer: int, used: list[int], n_pinned: int = 0):
        """One chunk pass over the (ascending) offloaded experts the chunk uses."""
        per = max(1, (self.n - n_pinned) // 2)
        nw = max(1, (len(used) + per - 1) // per)
        waves = [list(used[w * per:(w + 1) * per]) for w in range(nw)]
        down = self.sweeps & 1
        self.sweeps += 1
        if down:
            waves = [w[::-1] for w in waves]
        order = list(range(nw))[::-1] if down else list(range(nw))
        later = set(used)
        lines = {}
        staged = 0
        for i in range(nw):
            while staged < nw and staged <= i + 1:
                w = order[staged]
                later -= set(waves[w])
                kind = 0 if staged == 0 else (1 if staged > i else 2)
                m0 = self.misses
                got = self._stage(layer, waves[w], later)
                self.log.append(("stage", kind, list(waves[w]), sorted(later)))
                if got is None and staged > i:
                    break
                assert got is not None, "the model ran out of lines for the current wave"
                self.copied[kind] += self.misses - m0
                self.requested[kind] += len(waves[w])
                lines[w] = got
                staged += 1
            for l in lines[order[i]]:
                self.held[l] = False
            self.log.append(("release", list(waves[order[i]])))

    def write_log(self, path: str, n_experts: int):
        """The staging and release sequence in the host check's replay format."""
        with open(path, "w") as f:
            f.write(f"ring {self.n} {n_experts}\n")
            for op in self.log:
                if op[0] == "stage":
                    _, kind, ex, later = op
                    f.write(f"stage {kind} {len(ex)} {' '.join(map(str, ex))} "
                            f"later {len(later)} {' '.join(map(str, later))}\n")
                else:
                    f.write(f"release {len(op[1])} {' '.join(map(str, op[1]))}\n")
