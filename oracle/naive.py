"""Second, pure-Python statement of the resolver -- TEST INFRASTRUCTURE ONLY.

Written independently of ``hs_oracle.c`` to pin it: instead of sorting the
candidate slots once, every missing token (taken in ascending token order)
scans all slots and takes the least recently used one, (stamp, slot index)
smallest, among those that hold no hit and were not already taken in this
step; then every selected token's slot is stamped with the step.  This is the
HiSparse replacement step ("HiSparse" note, section 2: a miss is swapped in
from host memory and the eviction candidate is chosen by LRU; paper abstract:
hit detection, LRU replacement, host-to-device fetch), with the tie rules
stated in ``hs_oracle.c``.

Small inputs only (O(misses x B) per step in Python).
"""
from __future__ import annotations


_M64 = (1 << 64) - 1


def splitmix64_at(s: int, c: int) -> int:
    """Output number c of SplitMix64 started from state s (Steele, Lea, Flood 2014)."""
    z = (s + (c + 1) * 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def random_perm(seed: int, rl: int, t: int, N: int, x: int) -> int:
    """RANDOM eviction's permutation of range(N): four Feistel rounds over halves of h bits
    (4**h >= N, h >= 1), round i XORs the left half with the low h bits of SplitMix64 output
    i * 2**32 + right from the per-(request-layer, step) key; results outside range(N) are
    encrypted again (cycle walking) until they fall inside."""
    key = splitmix64_at(seed, ((rl << 32) | (t & 0xFFFFFFFF)) & _M64)
    h = 1
    while 4 ** h < N:
        h += 1
    mask = (1 << h) - 1
    while True:
        left, right = x >> h, x & mask
        for i in range(4):
            left, right = right, left ^ (splitmix64_at(key, (i << 32) | right) & mask)
        x = (left << h) | right
        if x < N:
            return x


class NaiveState:
    def __init__(self, B: int, cap: int, policy: str = "lru", seed: int = 0, rl: int = 0):
        assert policy in ("lru", "fifo", "random")
        self.policy, self.seed, self.rl = policy, seed, rl
        self.B, self.cap = B, cap
        self.pt = {}                  # token -> slot (absent = not resident)
        self.owner = [None] * B       # slot -> token
        self.stamp = [-1] * B
        self.t = 0
        self.rows = [None] * B        # what each slot holds (a token's row, by value)

    def resolve(self, S, host_row=None):
        valid = [s for s in S if s != -1]
        if any(not (0 <= s < self.cap) for s in valid):
            raise ValueError("token out of range")
        if len(set(valid)) != len(valid):
            raise ValueError("duplicate token")
        hit_slots = {self.pt[s] for s in valid if s in self.pt}
        misses = sorted(s for s in valid if s not in self.pt)
        taken = set()
        free = [j for j in range(self.B) if j not in hit_slots]     # RANDOM's candidates, slot order
        for i, s in enumerate(misses):
            if self.policy == "random":
                if len(free) < len(misses):
                    raise ValueError("no free slot")
                j = free[random_perm(self.seed, self.rl, self.t, len(free), i)]
            else:
                best = None
                for j in range(self.B):
                    if j in hit_slots or j in taken:
                        continue
                    key = (self.stamp[j], j)
                    if best is None or key < best[0]:
                        best = (key, j)
                if best is None:
                    raise ValueError("no free slot")
                j = best[1]
            taken.add(j)
            old = self.owner[j]
            if old is not None:
                del self.pt[old]
            self.pt[s] = j
            self.owner[j] = s
            if host_row is not None:
                self.rows[j] = host_row(s)
            self.stamp[j] = self.t                                # a fill counts as a use
        if self.policy != "fifo":                                 # FIFO: hits keep their fill step
            for s in valid:
                self.stamp[self.pt[s]] = self.t
        self.t += 1
        slots = [(-1 if s == -1 else self.pt[s]) for s in S]
        return slots, len(misses)

    def append(self, s, row=None):
        """Write-through append of a new token s (the note's introduction: KV is offloaded to
        host memory actively): it becomes resident before the next step -- in its own slot if
        it already has one, else in the slot used longest ago over all slots, (stamp, slot)
        smallest -- and that slot is stamped with the next step's number."""
        if self.policy == "random":
            raise ValueError("append needs a stamp-ordered policy")
        if not (0 <= s < self.cap):
            raise ValueError("token out of range")
        if s in self.pt:
            j = self.pt[s]
            if self.policy == "lru":
                self.stamp[j] = self.t
            if row is not None:
                self.rows[j] = row
            return j
        else:
            j = min(range(self.B), key=lambda i: (self.stamp[i], i))
            old = self.owner[j]
            if old is not None:
                del self.pt[old]
            self.pt[s] = j
            self.owner[j] = s
            self.stamp[j] = self.t
        if row is not None:
            self.rows[j] = row
        return j

    def arrays(self):
        """(PT[cap], RM[B], ST[B]) as plain lists with -1 for absent."""
        PT = [-1] * self.cap
        for s, j in self.pt.items():
            PT[s] = j
        RM = [(-1 if o is None else o) for o in self.owner]
        return PT, RM, list(self.stamp)
