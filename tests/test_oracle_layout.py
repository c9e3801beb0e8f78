"""Pins of the oracle's page map, write and snapshot: paged == contiguous window,
poisoned bytes untouched, resumed == fresh (issue #1142 'What stays as it is' and
'Proposal' piece 1; #1313 'Proposal' step 1 item 3)."""
import numpy as np

from oracle import Geom, PoolImage, block_layout
from oracle import workload as ow
from oracle.attention import sparse_mla_row
from oracle.layout import snapshot_copy
from synth import bf16_to_f64
from synth.configs import tiny

NAN16 = 0x7FC0


def write_stream(img, wl, pt, stride, b, tokens, c=0):
    bits = wl.latent_bits(c, b, tokens)
    for i, t in enumerate(tokens):
        img.write_row(pt, stride, b, int(t), c, bits[i, :512], bits[i, 512:])
    nk = (int(tokens[-1]) + 4) // 4
    kb = wl.pkey_bits(c, b, np.arange(nk))
    for j in range(nk):
        img.write_pkey(pt, stride, b, j, c, kb[j])


def reader_from_image(img, pt, stride, b, c=0):
    def rows(S):
        lat, rope = [], []
        for t in S:
            lb, rb, _ = img.read_row_bytes(pt, stride, b, int(t), c)
            lat.append(bf16_to_f64(lb.view(np.uint16)))
            rope.append(bf16_to_f64(rb.view(np.uint16)))
        return np.array(lat), np.array(rope)
    return rows


def test_address_formula_by_hand():
    g = Geom(n_caches=3, index_dim=64)
    L = block_layout(g)
    assert (L.off_latent, L.off_rope, L.off_pkey) == (0, 512 * 1024, 512 * 1024 + 512 * 128)
    assert L.block == 512 * 1024 + 512 * 128 + 128 * 128
    img = PoolImage(g, 10)
    pt = np.array([[7, 2, 9]])
    # row 1000 of stream 0 in cache 2: page pt[0][1] = 2, slot 488
    assert img.row_addr(pt, 3, 0, 1000, 2, "latent") == 2 * img.page + 2 * L.block + 488 * 1024
    assert img.row_addr(pt, 3, 0, 1000, 2, "rope") == 2 * img.page + 2 * L.block + L.off_rope + 488 * 128
    # pooled key 300 -> page pt[0][2] = 9, slot 44
    assert img.pkey_addr(pt, 3, 0, 300, 1) == 9 * img.page + L.block + L.off_pkey + 44 * 128
    # a null table: stream 1's page 2 is pool page 1 * 3 + 2
    assert img.row_addr(None, 3, 1, 1024, 0, "latent") == 5 * img.page


def test_paged_equals_contiguous_and_poison_intact():
    wl = tiny(0)
    g = Geom(n_caches=1, index_dim=wl.Dk)
    paged = PoolImage(g, wl.n_pages, fill=NAN16)
    contig = PoolImage(g, 2 * 4, fill=NAN16)
    toks = np.arange(2048)
    for b in range(2):
        write_stream(paged, wl, wl.pt, wl.pt_stride, b, toks)
        write_stream(contig, wl, None, 4, b, toks)
    # the 8 unassigned pages of the paged pool are still all NaN pattern
    used = set(wl.pt[wl.pt >= 0].tolist())
    for p in range(wl.n_pages):
        chunk = paged.buf[p * paged.page:(p + 1) * paged.page].view(np.uint16)
        assert np.all(chunk == NAN16) == (p not in used)
    # every row reads back the same through both maps, and equals the generator
    for b in range(2):
        for t in (0, 1, 511, 512, 1023, 2047):
            a = paged.read_row_bytes(wl.pt, wl.pt_stride, b, t, 0)
            c = contig.read_row_bytes(None, 4, b, t, 0)
            assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
            bits = wl.latent_bits(0, b, [t])[0]
            assert np.array_equal(a[0].view(np.uint16), bits[:512])
    # attention through either map (and from the generator's rows) agrees exactly
    q = bf16_to_f64(wl.q_bits(0, [(1, 2047)]))[0]
    rng = np.random.default_rng(0)
    blocks = np.sort(rng.choice(512, 64, replace=False))
    o1 = sparse_mla_row(q, reader_from_image(paged, wl.pt, wl.pt_stride, 1), blocks, 2047, 24.0)
    o2 = sparse_mla_row(q, reader_from_image(contig, None, 4, 1), blocks, 2047, 24.0)
    o3 = sparse_mla_row(q, ow.rows_reader(wl, 0, 1), blocks, 2047, 24.0)
    assert np.array_equal(o1[0], o2[0]) and np.array_equal(o1[0], o3[0])


def test_snapshot_then_resume_equals_fresh():
    wl = tiny(0)
    g = Geom(n_caches=1, index_dim=wl.Dk)
    src = PoolImage(g, wl.n_pages, fill=NAN16)
    write_stream(src, wl, wl.pt, wl.pt_stride, 0, np.arange(2048))
    at = 1536
    dst = PoolImage(g, 4, fill=NAN16)
    dpt = np.array([[3, 0, 2, 1]], dtype=np.int32)
    snapshot_copy(src, wl.pt, wl.pt_stride, dst, dpt, 4, [0], [0], at)
    # rows below at equal, rows past at untouched (still poison)
    for t in (0, 700, at - 1):
        assert np.array_equal(src.read_row_bytes(wl.pt, 4, 0, t, 0)[0],
                              dst.read_row_bytes(dpt, 4, 0, t, 0)[0])
    for t in (at, at + 1, 2047):
        assert np.all(dst.read_row_bytes(dpt, 4, 0, t, 0)[0].view(np.uint16) == NAN16)
    assert np.all(dst.read_pkey_bytes(dpt, 4, 0, at // 4, 0).view(np.uint16) == NAN16)
    assert np.array_equal(dst.read_pkey_bytes(dpt, 4, 0, at // 4 - 1, 0),
                          src.read_pkey_bytes(wl.pt, 4, 0, at // 4 - 1, 0))
    # resume: write rows [at, 2048) again from the generator, then a chunk of query rows
    write_stream(dst, wl, dpt, 4, 0, np.arange(at, 2048))
    rows = [(0, t) for t in range(2040, 2048)]
    q = bf16_to_f64(wl.q_bits(0, rows))
    rng = np.random.default_rng(1)
    for i, (_, t) in enumerate(rows):
        blocks = np.sort(rng.choice(t // 4 + 1, 64, replace=False))
        fresh = sparse_mla_row(q[i], reader_from_image(src, wl.pt, 4, 0), blocks, t, 24.0)
        res = sparse_mla_row(q[i], reader_from_image(dst, dpt, 4, 0), blocks, t, 24.0)
        assert np.array_equal(fresh[0], res[0]) and np.array_equal(fresh[1], res[1])


def test_snapshot_needs_whole_pools():
    g = Geom()
    a, b = PoolImage(g, 1), PoolImage(g, 1)
    try:
        snapshot_copy(a, None, 1, b, None, 1, [0], [0], 6)
    except ValueError:
        return
    raise AssertionError("at % 4 != 0 must be refused")


def test_chunked_prefill_equals_single_pass():
    """Query rows of one chunk computed in pieces equal the whole chunk (logits,
    selection, attention), and the decode row equals the chunk's last row."""
    wl = tiny(0)
    rows = [(0, t) for t in range(2040, 2048)]
    whole = ow.step(wl, 0, rows, 512, 24.0)
    parts = [ow.step(wl, 0, rows[i:i + 3], 512, 24.0) for i in range(0, 8, 3)]
    for k in range(5):
        cat = np.concatenate([p[k] for p in parts])
        assert np.array_equal(cat, whole[k])
    dec = ow.step(wl, 0, [(0, 2047)], 512, 24.0)
    for k in range(5):
        assert np.array_equal(dec[k][0], whole[k][-1])
