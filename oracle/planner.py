"""Row-budget planner.

"Speculative decoding" (gpillon.github.io/ignis), section "The row budget": a
round carries lanes x (drafts + 1) rows, the budget caps the rows of a round
(a budget of 0 means 8), and each lane drafts min(draft tokens,
rows / lanes - 1).  Integer division; a negative result means no drafts (the
page: a busy server falls back to plain rounds).
"""


def plan_drafts(k: int, row_budget: int, lanes: int) -> int:
    if lanes <= 0 or k < 0 or row_budget < 0:
        raise ValueError("lanes must be >= 1, k and row_budget >= 0")
    rows = 8 if row_budget == 0 else row_budget
    return max(0, min(k, rows // lanes - 1))


def plan_drafts_bruteforce(k: int, row_budget: int, lanes: int) -> int:
    """The largest draft count d <= k whose round lanes x (d + 1) fits the budget; 0 if none."""
    rows = 8 if row_budget == 0 else row_budget
    best = 0
    for d in range(k + 1):
        if lanes * (d + 1) <= rows:
            best = d
    return best
