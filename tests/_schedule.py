"""The split kernel's schedule as include/kvq.h documents it, in plain
Python: which 16-token blocks each split workgroup takes.  The GPU tests
merge the partials the kernel leaves by it; the CPU tests check the
properties the schedule is built for."""

SEG_COST = 24  # positions between one unit and the next


def cost_line(block_counts, c=SEG_COST):
    """C: the units' blocks plus c positions between consecutive units."""
    return sum(block_counts) + c * max(len(block_counts) - 1, 0)


def ways(C, nwg):
    """Workgroups that get work."""
    lo = min(max((C + 255) // 256, 4), 128)
    return max(1, min((C + lo - 1) // lo, nwg))


def unit_start(block_counts, u, c=SEG_COST):
    """Cost position of unit u's block 0."""
    return sum(block_counts[:u]) + c * u


def owner(C, n, y):
    """The workgroup that holds cost position y (0 <= y < C)."""
    return ((y + 1) * n - 1) // C


def ranges(block_counts, nwg, c=SEG_COST):
    """For each workgroup, the (unit, first block, block count) segments it
    takes, in order."""
    C = cost_line(block_counts, c)
    n = ways(C, nwg)
    out = [[] for _ in range(nwg)]
    for u, nb in enumerate(block_counts):
        s = unit_start(block_counts, u, c)
        i = 0
        while i < nb:
            w = owner(C, n, s + i)
            j = i
            while j < nb and owner(C, n, s + j) == w:
                j += 1
            out[w].append((u, i, j - i))
            i = j
    return out
