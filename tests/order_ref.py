"""The start order of a mixed-length batch, written out in numpy for the
tests (CPU and GPU): the stable descending sort of the page counts, then the
documented start positions."""
import numpy as np


def host_rank(ctx, max_context_len, round_len=0):
    """The stable descending sort of the page counts, then each sorted rank
    placed at its start position: with P = round_len // 4 and a batch of at
    least 4P sequences, the 3P longest first with the middle quarter of them
    reversed, then the P shortest (shortest first), then the rest longest
    first."""
    n = np.minimum(np.asarray(ctx, np.int64), max_context_len)
    pages = np.where(n > 0, -(-n // 16), 0)
    ranked = np.argsort(-pages, kind="stable").astype(np.int32)
    B, P = ranked.size, round_len // 4
    if P < 1 or B < 4 * P:
        return ranked
    first = ranked[:3 * P].copy()
    first[P:2 * P] = first[P:2 * P][::-1].copy()
    shortest = ranked[B - P:][::-1]
    return np.concatenate([first, shortest, ranked[3 * P:B - P]]).astype(np.int32)
