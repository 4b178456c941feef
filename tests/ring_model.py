"""A host-side model of how the library plans the routed waves of an offloaded chunk and
stages them through the ring, for tests that predict the ring's hit and miss counts exactly.
Test infrastructure only.

Per chunk pass: the offloaded experts the chunk uses, ascending, are cut into waves of at most
n_lines // 2; even passes run the waves in ascending order, odd passes in descending order
(and stage each wave's experts top-down). Before wave i runs, waves i and i + 1 are staged
(the second only if enough lines are free); wave i is released after its GEMMs. Staging marks
hits first; each miss evicts the least recently used unheld line that holds no expert a later
wave of the same pass asks for, else the least recently used unheld line."""
from __future__ import annotations


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

    def chunk(self, layer: int, used: list[int]):
        """One chunk pass over the (ascending) offloaded experts the chunk uses."""
        per = max(1, self.n // 2)
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
