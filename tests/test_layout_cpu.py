"""Host restatements of index arithmetic that the GPU kernels rely on (CPU only).

* The few-rows sparse MLA (mla_bf16n_kernel in sparse_attention_10_amd/csrc/mla.hip): its
  workgroup numbering covers every (query row, chunk, 16-head group) exactly once; each wave's
  18 tile loads cover its 16 rows' 1152 pieces exactly once, each load reading at most two rows;
  the pieces land in the 64-head kernel's swizzled layout with no LDS bank conflict inside a
  16-lane group; and the chunk's slot list stays inside its LDS array.
* The decode indexer's ring depth (launch_indexer in sparse_attention_10_amd/csrc/indexer.hip):
  for one query row of one sequence, the depth it picks leaves no loop iteration on dummy
  blocks at one, two or a multiple of four blocks per wave.
"""
import pytest

ROW_BYTES = 1152          # bf16 latent row
PIECES = ROW_BYTES // 16  # 72 pieces of 16 bytes
TN = 128                  # tokens per tile of the few-rows kernel
CHUNK_N = 512             # selected rows per workgroup at most
LOADS = TN * ROW_BYTES // 1024 // 8   # 18 loads of 1 KiB per wave


def bf16_swz(t):
    return ((t >> 4) & 1) | (((t >> 1) & 1) << 1) | (((t >> 3) & 1) << 2)


def bf16_pos(t, p):
    return t * ROW_BYTES + ((p ^ bf16_swz(t)) << 4)


def narrow_load(wave, c, lane):
    """(row of the wave's 16, piece) that load c of `wave` reads in `lane`, as the kernel forms it
    from the two wave-uniform rows r0, r0 + 1 and the lane boundary kb."""
    r0 = 64 * c // 72
    kb = 72 * (r0 + 1) - 64 * c
    lo = lane < kb
    row = r0 if lo else r0 + 1
    pc = lane + (64 * c - 72 * r0 if lo else 64 * c - 72 * (r0 + 1))
    return row, pc


def test_narrow_tile_loads_cover_each_piece_once_without_bank_conflicts():
    assert LOADS == 18
    seen = set()
    for wave in range(8):
        for c in range(LOADS):
            rows = set()
            for g in range(4):                      # one LDS pass of ds_write_b128: 16 lanes
                banks = set()
                for lane in range(16 * g, 16 * g + 16):
                    row, pc = narrow_load(wave, c, lane)
                    # the plain row-major split of piece 64c + lane
                    assert (row, pc) == divmod(64 * c + lane, PIECES)
                    assert 0 <= row < 16 and 0 <= pc < PIECES
                    rows.add(row)
                    t = 16 * wave + row
                    addr = bf16_pos(t, pc)
                    assert 0 <= addr and addr + 16 <= TN * ROW_BYTES
                    seen.add(addr)
                    banks.update(((addr // 4) + k) % 64 for k in range(4))
                assert len(banks) == 64, (wave, c, g)
            assert len(rows) <= 2                   # two wave-uniform slots per load
            r0 = 64 * c // 72
            assert rows <= {r0, min(r0 + 1, 15)}    # the clamped second row index
    assert len(seen) == TN * PIECES                 # every piece of the tile written once


@pytest.mark.parametrize("rows,H,ns", [(1, 64, 16), (1, 64, 7), (2, 64, 16), (3, 64, 4), (4, 64, 16),
                                       (1, 16, 2), (1, 32, 2), (1, 48, 1), (5, 48, 3), (16, 16, 3)])
def test_narrow_grid_covers_each_row_chunk_and_head_group_once(rows, H, ns):
    ng = H // 16
    assert rows * ng <= 16                          # the launcher's condition for this kernel
    rs_total = rows * ns
    blocks = (rs_total + 7) // 8 * 8 * ng
    seen = []
    for b in range(blocks):
        xq, yq = b & 7, b >> 3
        hg = yq % ng
        rs = 8 * (yq // ng) + xq
        if rs >= rs_total:
            continue                                # grid padding
        r, split = divmod(rs, ns)
        seen.append((r, split, hg))
    assert sorted(seen) == sorted((r, s, g) for r in range(rows) for s in range(ns) for g in range(ng))
    # the head groups of one chunk share an XCD (block ids 8 apart: same id mod 8)
    by_chunk = {}
    for b in range(blocks):
        xq, yq = b & 7, b >> 3
        rs = 8 * (yq // ng) + xq
        if rs < rs_total:
            by_chunk.setdefault(rs, set()).add(b % 8)
    assert all(len(x) == 1 for x in by_chunk.values())


@pytest.mark.parametrize("k,ns", [(2048, 16), (2048, 7), (100, 3), (512, 1), (300, 2), (2048, 64), (8192, 16)])
def test_narrow_slot_list_fits(k, ns):
    chunk = (k + ns - 1) // ns
    chunk = (chunk + 31) // 32 * 32
    if chunk > CHUNK_N:
        pytest.skip("the launcher takes the 64-head kernel for longer chunks")
    for split in range(ns):
        j0 = split * chunk
        j1 = min(k, j0 + chunk)
        ntiles = (j1 - j0 + TN - 1) // TN if j1 > j0 else 0
        # slot reads at min(j0 + tid, k - 1); list entries tid < ntiles * 128 <= 512
        assert ntiles * TN <= CHUNK_N
        for v in range(ntiles):
            for t in range(TN):
                e = v * TN + t
                assert e < ntiles * TN
                # entries past the chunk hold -1 (skipped), the rest map to positions < k
                if j0 + e < j1:
                    assert j0 + e < k


# ---- decode indexer, one row of one sequence
RB = 16


def indexer_one_row_depth(max_seq_len, fp8):
    """launch_indexer's choice for B = 1, Q = 1 (no balanced partition): tiles per workgroup
    and ring depth D."""
    NW = 8
    blocks = (max_seq_len + RB - 1) // RB
    R = 256
    tb = max((blocks + R - 1) // R, 1)
    bpw = (tb + NW - 1) // NW
    if bpw <= 1:
        D = 1
    elif bpw == 2:
        D = 2
    elif fp8:
        D = 4
    elif bpw % 4 == 0:
        D = 4
    else:
        D = 3
    return tb, NW, D


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("L", [600, 5000, 32768, 40000, 65536, 131072])
def test_indexer_one_row_ring_runs_no_dummy_block_iterations(L, fp8):
    tb, NW, D = indexer_one_row_depth(L, fp8)
    bpw = (tb + NW - 1) // NW
    if bpw <= 2 or bpw % 4 == 0:
        assert bpw % D == 0                          # a full wave's blocks fill whole ring rounds
    blocks = (L + RB - 1) // RB
    wasted = 0
    for g in range((blocks + tb - 1) // tb):
        nb = min(tb, blocks - g * tb)               # blocks of this key range
        for wave in range(NW):
            nbw = (nb - wave + NW - 1) // NW if nb > wave else 0
            wasted += (nbw + D - 1) // D * D - nbw
    if L in (32768, 131072):                        # every range full: not one dummy iteration
        assert wasted == 0
