"""Host model of the SpMM's prepared stream and of every data-dependent index
the two SpMM kernels read or write, checked against the sizes of their
arrays (no GPU). The model restates, in numpy, what the prep kernels of
csrc/spmm.hip compute:

  bptr[o][b]  first position of segment o (a row of F forward, a column of F
              backward) whose source column is >= b * 64;
  ptr[b][o]   exclusive scan over segments of the (row, block) counts, padded
              to even lengths forward;
  base[b]     exclusive scan of the block totals;
  stream      entry q of segment o in block b at base[b] + ptr[b][o] + q - bptr[o][b],
              the padding after each odd segment (forward).

and then the reads of the forward kernel (run table, segment bounds, the
staged pairs of a workgroup's run, restaged chunks) and of the backward
kernel (the same, odd runs read one entry past their end, the dc partial
stores), for the layer shapes of the five workloads and edge shapes. The
stream is allocated with 16 zero entries past its end; everything read must
fall inside the allocation and everything written inside the run.
"""

import numpy as np
import pytest

import oracle as O

TT, JB = 256, 64                  # tokens per tile, source columns per block
RW, RR, RRDC = 16, 16, 8          # waves per workgroup, rows per wave (plain / with dc)
ENT_CAP, PAD = 1536, 16           # staged entries per block, zero entries past the stream


def plan(n_src, n_out, nnz, dc, jb=JB):
    rows_wg = RW * (RRDC if dc else RR)
    nblk = -(-n_src // jb)
    n_out_pad = -(-n_out // rows_wg) * rows_wg
    mult = 1 if dc else 2
    segs = n_out * nblk
    cap = nnz + (mult - 1) * min(segs, nnz)
    return dict(rows_wg=rows_wg, nblk=nblk, stride=n_out_pad + 1, mult=mult, cap=cap,
                n_out=n_out, jb=jb)


def prep(seg_ptr, keys, pl):
    """Returns bptr [n_out][nblk+1], ptr [nblk][stride], base [nblk+1] and the
    stream position of every entry (segment order), as the prep kernels."""
    n_out, nblk, stride, mult = pl["n_out"], pl["nblk"], pl["stride"], pl["mult"]
    bptr = np.zeros((n_out, nblk + 1), dtype=np.int64)
    for o in range(n_out):
        lo, hi = int(seg_ptr[o]), int(seg_ptr[o + 1])
        seg = keys[lo:hi]
        assert np.all(np.diff(seg) > 0), "columns ascend within a segment"
        bptr[o] = lo + np.searchsorted(seg, np.arange(nblk + 1) * pl["jb"], side="left")
    cnt = np.diff(bptr, axis=1).T                      # [nblk][n_out]
    cnt = -(-cnt // mult) * mult
    ptr = np.zeros((nblk, stride), dtype=np.int64)
    ptr[:, 1:n_out + 1] = np.cumsum(cnt, axis=1)
    ptr[:, n_out + 1:] = ptr[:, n_out:n_out + 1]       # padding rows are empty
    base = np.zeros(nblk + 1, dtype=np.int64)
    base[1:] = np.cumsum(ptr[:, stride - 1])
    pos = np.empty(len(keys), dtype=np.int64)
    for o in range(n_out):
        lo, hi = int(seg_ptr[o]), int(seg_ptr[o + 1])
        q = np.arange(lo, hi)
        b = keys[lo:hi] // pl["jb"]
        pos[lo:hi] = base[b] + ptr[b, o] + (q - bptr[o, b])
    return bptr, ptr, base, pos


def check_stream(seg_ptr, keys, n_src, dc, prep_fn=prep, jb=JB):
    n_out = len(seg_ptr) - 1
    nnz = len(keys)
    pl = plan(n_src, n_out, nnz, dc, jb)
    bptr, ptr, base, pos = prep_fn(seg_ptr, keys, pl)
    nblk, stride, cap = pl["nblk"], pl["stride"], pl["cap"]
    # the scatter: every entry at its own position inside the stream, the
    # padded stream exactly base[nblk] long and no longer than its capacity
    assert base[nblk] <= cap
    assert np.all((pos >= 0) & (pos < base[nblk]))
    assert len(np.unique(pos)) == nnz
    if not dc:
        assert base[nblk] % 2 == 0          # whole pairs
    alloc = cap + PAD                       # entries allocated for the stream
    ptr_size = nblk * stride
    n_groups = -(-n_out // pl["rows_wg"])
    ROWS = pl["rows_wg"]
    for g in range(n_groups):
        rg0 = g * ROWS
        for b in range(nblk):
            # segment bounds of the workgroup's rows (thread tid <= ROWS)
            assert b * stride + rg0 + ROWS < ptr_size
            p0 = ptr[b, rg0]
            k0 = base[b] + p0
            run = ptr[b, rg0 + ROWS] - p0
            assert 0 <= run and k0 + run <= base[nblk]
            # staged pairs: int4 reads at k0 + 2 tid (entries k0 + 2 tid, + 1)
            # for 2 tid < run, tid < ENT_CAP / 2; restaged chunks likewise
            if run > 0:
                last_pair = (run - 1) // 2
                last = k0 + 2 * last_pair + 1
                assert last < alloc, (g, b, last, alloc)
                if not dc:
                    assert run % 2 == 0 and last < base[nblk]
            if dc and run > 0:
                # the dc partial of stream entry k0 + i goes to partial[tile][k0 + i]
                assert k0 + run <= nnz
    return pl


def csr_keys(E):
    return E[:, 1].astype(np.int64)


def csc_keys(E, perm):
    return E[perm, 0].astype(np.int64)


def both_directions(row_ptr, E, col_ptr, perm, d_out, d_in):
    check_stream(row_ptr.astype(np.int64), csr_keys(E), d_in, dc=False)
    # the backward with dc: fp32 dy in 64-column blocks, bf16 dy in 128
    check_stream(col_ptr.astype(np.int64), csc_keys(E, perm), d_out, dc=True)
    check_stream(col_ptr.astype(np.int64), csc_keys(E, perm), d_out, dc=True, jb=128)


@pytest.mark.parametrize("d_out,d_in,p", [
    (37, 2, 74), (300, 64, 2500), (513, 128, 4000), (64, 1024, 6000), (40, 8192, 2000),
    (3, 16384, 300), (1100, 32, 3300), (64, 128, 1920), (16500, 4, 49500), (1, 64, 64),
    (257, 192, 3000)])
def test_stream_bounds_edge_shapes(d_out, d_in, p):
    rng = np.random.default_rng(d_out + d_in)
    dwq = (0.01 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    r = O.init_select(dwq, p, m=min(3, d_in))
    both_directions(r["row_ptr"], r["E"], r["col_ptr"], r["csc_perm"], d_out, d_in)


def _adaalloc_structure(d_out, d_in, p, seed):
    """E with the budgets AdaAlloc gives a layer of this shape (row norms of a
    heavy-tailed error) and uniformly random distinct columns per row: the
    segment structure the prep sees, without the full fp64 transform."""
    rng = np.random.default_rng(seed)
    w = np.abs(rng.standard_normal(d_out)) * 0.3 + 1.0
    w[rng.choice(d_out, size=max(1, d_out // 100), replace=False)] *= 3.0
    budgets = O.adaalloc(w, p, d_in, m=3)
    rows = np.repeat(np.arange(d_out), budgets)
    cols = np.concatenate([np.sort(rng.choice(d_in, size=int(k), replace=False))
                           for k in budgets])
    E = np.stack([rows, cols], axis=1).astype(np.int32)
    row_ptr = np.zeros(d_out + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(budgets)
    col_ptr, perm = O.csc(E, d_in)
    return row_ptr, E, col_ptr, perm


@pytest.mark.parametrize("d_out,d_in,p", [
    (4096, 4096, 524288),            # c2, c5 q / o
    (14336, 4096, 1179648),          # c3
    (8192, 8192, 1048576),           # c4
    (1024, 4096, 327680),            # c5 k / v
    (4096, 14336, 1179648)])         # the down_proj shape (block-diagonal width)
def test_stream_bounds_workload_shapes(d_out, d_in, p):
    row_ptr, E, col_ptr, perm = _adaalloc_structure(d_out, d_in, p, d_out ^ d_in)
    both_directions(row_ptr, E, col_ptr, perm, d_out, d_in)


def test_stream_bounds_c2_selection():
    """The c2 layer's own selection (oracle init at full size)."""
    import synth
    spec = synth.config_specs("c2")[0]
    layer = synth.make_layer(spec, seed=0)
    r = O.init_select(layer.dwq, spec.p, m=3)
    both_directions(r["row_ptr"], r["E"], r["col_ptr"], r["csc_perm"], spec.d_out, spec.d_in)


def test_model_catches_planted_mistakes():
    """The checks bite: a scatter that forgets the block base puts entries of
    different blocks on one position, and a forward prep that forgets the
    even padding leaves odd runs whose last pair reads past the stream."""
    rng = np.random.default_rng(3)
    dwq = (0.01 * rng.standard_normal((300, 256))).astype(np.float32)
    r = O.init_select(dwq, 2500, m=3)
    row_ptr, keys = r["row_ptr"].astype(np.int64), csr_keys(r["E"])

    def no_base(seg_ptr, keys, pl):
        bptr, ptr, base, pos = prep(seg_ptr, keys, pl)
        b = keys // JB
        return bptr, ptr, base, pos - base[b]

    def no_padding(seg_ptr, keys, pl):
        return prep(seg_ptr, keys, dict(pl, mult=1))

    check_stream(row_ptr, keys, 256, dc=False)
    with pytest.raises(AssertionError):
        check_stream(row_ptr, keys, 256, dc=False, prep_fn=no_base)
    with pytest.raises(AssertionError):
        check_stream(row_ptr, keys, 256, dc=False, prep_fn=no_padding)
