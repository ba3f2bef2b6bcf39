"""Host restatement of how the sparse MLA's XCD-mapped launches (mla_fp8d_kernel,
mla_bf16d_kernel) turn a workgroup index into (query row, chunk), and of the host's choice of
row group.  For every batch shape the grid must cover each (row, chunk) exactly once, and when
a sequence's verify rows form a group they must share one XCD (workgroup index mod 8) and take
each chunk in consecutive workgroups of that XCD.  CPU only."""


def _group(batch, q_per_seq):
    # the host's choice: a sequence's rows form a group when the sequences fill the 8 XCDs evenly
    return q_per_seq if q_per_seq > 1 and batch >= 8 and batch % 8 == 0 else 1


def _grid(rows, group, n_split):
    return ((rows // group + 7) // 8 * 8 * group if rows >= 8 else rows) * n_split


def _row_split(bid, rows, group, n_split):
    if rows >= 8:
        xcd, jx = bid & 7, bid >> 3
        t, ri = jx // group, jx % group
        uu, split = t // n_split, t % n_split
        r = (8 * uu + xcd) * group + ri
        return None if r >= rows else (r, split)
    return bid // n_split, bid % n_split


def test_mla_xcd_map_covers_every_row_and_chunk_once():
    for batch in range(1, 70):
        for q in (1, 2, 3, 4, 5):
            rows, g = batch * q, _group(batch, q)
            for ns in (1, 2, 3, 8, 10):
                got = [_row_split(b, rows, g, ns) for b in range(_grid(rows, g, ns))]
                live = [x for x in got if x is not None]
                assert sorted(live) == [(r, s) for r in range(rows) for s in range(ns)], (batch, q, ns)


def test_mla_xcd_map_keeps_a_sequences_rows_together():
    for batch in (8, 16, 24, 64):
        for q in (2, 3, 4):
            rows, g = batch * q, _group(batch, q)
            assert g == q
            for ns in (1, 2, 5):
                seen = {}
                for b in range(_grid(rows, g, ns)):
                    x = _row_split(b, rows, g, ns)
                    if x is None:
                        continue
                    r, s = x
                    seq = r // q
                    assert b & 7 == seq % 8                      # the sequence's XCD
                    seen.setdefault((seq, s), []).append(b >> 3)
                for (seq, s), js in seen.items():
                    js.sort()
                    assert len(js) == q and js[-1] - js[0] == q - 1   # consecutive on that XCD
