"""Token ranges of every sequence's splits under a plan, restated from the
partition rules fd.h documents for fd_plan.split_mode (host arithmetic only,
no attention)."""


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# List positions a sequence takes before its tiles in the balanced list (the
# library's share cost, FD_SHARE_COST when it is built).
SHARE_COST = 4


def plan_cuts(lens, plan, share_cost: int = SHARE_COST):
    """[(lo, hi), ...] per sequence: split s of sequence b holds tokens [lo, hi)."""
    C = plan.chunk_tokens
    if plan.split_mode == 0:
        return [[(s, min(s + C, L)) for s in range(0, L, C)] for L in lens]
    P = C // 16
    cuts, U = [], 0
    for L in lens:
        n = ceil_div(L, 16)
        T = U + share_cost  # position of the sequence's first tile
        first, last = T // P, (T + n - 1) // P
        cuts.append([(16 * (max(T, w * P) - T), min(L, 16 * (min(T + n, (w + 1) * P) - T)))
                     for w in range(first, last + 1)])
        U = T + n
    return cuts
