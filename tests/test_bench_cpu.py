"""Host-side checks of bench.py's bookkeeping: the source digest that ties a
committed HBM-traffic figure to the code it was measured on."""

import os

import bench


def test_strip_comments_keeps_code_and_strings():
    src = ('int a = 1;  // note "x"\n/* block\n   comment */ const char* s = "a//b/*c*/";\n'
           "char q = '\"'; char e = '\\''; int b; /* trailing */")
    out = bench.strip_comments(src)
    assert out == ("int a = 1; const char* s = \"a//b/*c*/\"; char q = '\"'; "
                   "char e = '\\''; int b;")


def test_strip_comments_ignores_comment_and_spacing_edits_only():
    a = "x = y + 1; // old note\n"
    b = "x = y + 1;   /* new note */\n\n"
    c = "x = y + 2; // old note\n"
    assert bench.strip_comments(a) == bench.strip_comments(b)
    assert bench.strip_comments(a) != bench.strip_comments(c)


def test_every_kernel_source_exists_and_digests():
    d = os.path.join(bench.ROOT, "quantization_aware_sparse_amd", "csrc")
    for kid, names in bench.KERNEL_SOURCES.items():
        for name in names + bench.SHARED_SOURCES:
            assert os.path.exists(os.path.join(d, name)), (kid, name)
        dg = bench.source_digest(kid)
        assert len(dg) == 16 and int(dg, 16) >= 0
    assert bench.source_digest("FWD_SPMM") == bench.source_digest("BWD_SPMM")
    assert bench.source_digest("FWD_SPMM") != bench.source_digest("FWD_FWHT")
