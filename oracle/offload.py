"""Oracle: the device expert-slot cache of a stack larger than HBM.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[P1 §3C] one engine (FreeToken) keeps every expert in a pinned host store
and a slot cache on the device; a layer's missing experts are copied to the
device or computed on the CPU, the number copied set from the two channels'
measured bandwidths; [P1 §5] states the balance as f / (1 - f) = effective
PCIe rate / effective CPU rate; [P2 §六] gives the first-order form
q* ~ m * B_P / B_H.  [P3 §五.2] a device LRU of experts in front of a pinned
host arena.  ([P2] = "Model task radar 2026-11-03: when the accelerator
flips", neodrop.ai.)

Readings where the pages are silent (each also in the design notes):
  * f = B_P / (B_P + B_C): the share at which copies and CPU work end
    together (it solves f / (1 - f) = B_P / B_C; for B_P << B_C it is the
    page's m * B_P / B_H);
  * q is a whole number of experts: of the two next to m * f, the one whose
    slower channel finishes first (copies take time in proportion to
    q * (1 - f), the CPU's experts (m - q) * f), the larger on a tie;
  * the copied misses are those chosen by the most pairs of the step, then
    the lower expert id; the rest go to the CPU;
  * a copy takes a free slot (lowest index), else the least recently used
    slot not used by this step (lowest index on ties); with no such slot the
    miss goes to the CPU;
  * a hit or a copy marks its slot used at the current step.

cpu_expert_ffn: the CPU tier's arithmetic is the expert FFN of oracle.moe
(parity of the library's CPU FFN is checked against moe.expert_ffn).
"""



class SlotCache:
    """Plain LRU over (layer, expert) keys with a step counter."""

    def __init__(self, n_layers, n_experts, n_slots):
        self.L, self.E, self.S = n_layers, n_experts, n_slots
        self.slot_of = {}                  # (layer, expert) -> slot
        self.owner = [None] * n_slots      # slot -> (layer, expert)
        self.last_use = [0] * n_slots      # slot -> step (0 = never)
        self.step = 0

    def _victim(self):
        for s in range(self.S):
            if self.owner[s] is None:
                return s
        best = None
        for s in range(self.S):
            if self.last_use[s] == self.step:
                continue
            if best is None or self.last_use[s] < self.last_use[best]:
                best = s
        return best

    def plan(self, layer, idx, copy_share):
        """idx: list of rows, each a list of expert ids.  Returns
        (slot_of list [E], copies [(expert, slot)], cpu [experts ascending],
        idx_gpu rows with CPU experts as -1)."""
        for row in idx:
            for e in row:
                if not (0 <= e < self.E):
                    raise ValueError("expert id out of range")
        if not (0.0 <= copy_share <= 1.0):
            raise ValueError("share out of range")
        self.step += 1
        count = {}
        for row in idx:
            for e in row:
                count[e] = count.get(e, 0) + 1
        misses = []
        for e in sorted(count):
            key = (layer, e)
            if key in self.slot_of:
                self.last_use[self.slot_of[key]] = self.step
            else:
                misses.append(e)
        m = len(misses)
        f = copy_share
        best = None
        for cand in range(m + 1):                      # brute force over every count
            if abs(cand - m * f) >= 1.0:
                continue                               # only the two next to m * f
            t = max(cand * (1 - f), (m - cand) * f)
            if best is None or t < best[0] or (t == best[0] and cand > best[1]):
                best = (t, cand)
        q = best[1]
        misses.sort(key=lambda e: (-count[e], e))
        copies, cpu = [], []
        for j, e in enumerate(misses):
            s = self._victim() if j < q else None
            if s is None:
                cpu.append(e)
                continue
            if self.owner[s] is not None:
                del self.slot_of[self.owner[s]]
            self.owner[s] = (layer, e)
            self.slot_of[(layer, e)] = s
            self.last_use[s] = self.step
            copies.append((e, s))
        cpu.sort()
        on_cpu = set(cpu)
        idx_gpu = [[-1 if e in on_cpu else e for e in row] for row in idx]
        slot_of = [self.slot_of.get((layer, e), -1) for e in range(self.E)]
        return slot_of, copies, cpu, idx_gpu


def copy_share(pcie_rate, cpu_rate):
    """f with f / (1 - f) = pcie_rate / cpu_rate; 0 when both are 0."""
    if pcie_rate < 0 or cpu_rate < 0:
        return 0.0
    t = pcie_rate + cpu_rate
    return pcie_rate / t if t > 0 else 0.0
