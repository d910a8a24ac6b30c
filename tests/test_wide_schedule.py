"""The wide-chunk output kernel's per-chunk unit schedule (C = 128, 256), read from
its source and simulated on the host over full and partial last chunks.

The schedule orders the units (query sub-block i, key sub-block jj <= i) of each
chunk and names the k/v tile half each one reads and whether it stages it.  The
producers stage unit u + 1 while the consumers read unit u, so correctness rests
on these invariants: a staging never writes the half unit u reads; a unit that
reuses a half finds its own key sub-block of the same chunk there; q and the gate
(staged at a row's first unit, by the parity of i) never overwrite the row being
read; each row's units are contiguous, cover jj = 0..i once, begin with the row's
first-unit flag (the inter-chunk term) and end with the diagonal (the store)."""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "hybrid_sparse_linear_la_amd", "csrc", "la_prefill.hip")


def schedule(ksub):
    text = open(SRC).read()
    m = re.search(r"struct WideSchedule<%d> \{\s*static constexpr uint32_t (.*?);" % ksub, text, re.S)
    assert m, f"no schedule for kSub = {ksub}"
    f = {k.strip(): int(v, 0) for k, v in (x.split("=") for x in m.group(1).split(","))}
    n = ksub * (ksub + 1) // 2
    return [((f["kI"] >> 2 * e) & 3, (f["kJ"] >> 2 * e) & 3, (f["kHalfBuf"] >> e) & 1, (f["kStage"] >> e) & 1,
             (f["kFirst"] >> e) & 1) for e in range(n)]


@pytest.mark.parametrize("ksub", (2, 4))
@pytest.mark.parametrize("nchunks", (1, 2, 3))
def test_schedule_invariants(ksub, nchunks):
    tab = schedule(ksub)
    for last in range(1, ksub + 1):  # sub-blocks in the segment's last chunk
        seq = []
        for c in range(nchunks):
            nsub = ksub if c < nchunks - 1 else last
            seq += [(c,) + e for e in tab[: nsub * (nsub + 1) // 2]]
        assert all(e[0] < (ksub if c < nchunks - 1 else last) for c, *e in seq)
        content = [None, None]
        rows = {}
        for u, (c, i, jj, half, stage, first) in enumerate(seq):
            if stage:
                assert u == 0 or half != seq[u - 1][3], (u, "staged into the half being read")
                content[half] = (c, jj)
            else:
                assert content[half] == (c, jj), (u, "reused half holds another sub-block")
            if u + 1 < len(seq) and seq[u + 1][5]:
                assert (seq[u + 1][1] & 1) != (i & 1), (u, "q/gate staging overwrites the row being read")
            rows.setdefault((c, i), []).append((u, jj, first))
        for (c, i), units in rows.items():
            us = [u for u, _, _ in units]
            assert us == list(range(us[0], us[0] + len(us))), "a row's units are not contiguous"
            assert sorted(jj for _, jj, _ in units) == list(range(i + 1))
            assert [f for _, _, f in units] == [1] + [0] * i
            assert units[-1][1] == i, "a row must end with its diagonal unit"
        # the first unit of a segment stages (its hi/lo rows come from that staging)
        assert seq[0][4] == 1 and seq[0][5] == 1
