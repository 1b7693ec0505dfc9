"""The one-time weight transform (moe_prepare_weights; the pages' weight conversion before
any forward, chenxutan.com/d/1930 section 3.3), checked byte for byte.

The packed buffer is rebuilt on the host from the layout the library documents for its
kernels (FP4 data in MFMA fragment order, four K steps of UE8M0 scales per 32-bit word,
W1's gate and up rows of one 128-block of I in one 256-column tile, W2 in 256-row column
tiles completed with zero rows), and the GPU's buffer must equal it everywhere: every input
byte lands in its one place and every padding byte is zero. Random bytes stand in for the
weights (the transform only moves bytes), so a byte misplaced anywhere, in any fragment,
lane, K step or tile, changes the comparison."""
import numpy as np
import pytest
import torch

from conftest import gpu_available

import block_scaled_fp8_dispatch_amd as moe  # noqa: E402


def _align(v, a=256):
    return -(-v // a) * a


def packed_index_map(E, H, I):
    """For every byte of the packed buffer: which input byte it holds, as (array id, flat
    index) with array ids 0 w1, 1 w1_sf, 2 w2, 3 w2_sf, or id -1 for a zero byte."""
    lane = np.arange(64)
    F, L = np.meshgrid(np.arange(16), lane, indexing="ij")            # [16, 64]
    ks1, nkb1, nb1 = H // 128, -(-H // 512), I // 128
    ks2, nkb2, nt2 = I // 128, -(-I // 512), -(-H // 256)
    e4 = np.arange(E)[:, None, None, None]     # broadcasts against [16, 64, 16]
    e3 = np.arange(E)[:, None, None]           # broadcasts against [16, 64]

    def l1_row(nt):    # W1 row of lane column L of fragment F in the tile of I-block nt
        ff = F & 7
        return np.where(F < 8, 0, I) + nt * 128 + 64 * (ff >> 2) + 4 * (L & 15) + (ff & 3)

    def l2_row(nt):    # W2 row of lane column L of fragment F in column tile nt
        return nt * 256 + 128 * (F >> 3) + 8 * (L & 15) + (F & 7)

    def data(aid, rows_of, n_tiles, nks, n_rows, row_bytes):
        # [E][tile][K step][fragment][lane][16 bytes]: the lane's 32 K values (low nibble first)
        # of its column are bytes 16*(lane/16) .. +15 of the K step's 64 bytes of the row
        ix = np.full((E, n_tiles, nks, 16, 64, 16), -1, dtype=np.int64)
        for nt in range(n_tiles):
            r = rows_of(nt)[None, ..., None]
            for ks in range(nks):
                col = ks * 64 + 16 * (L >> 4)[None, ..., None] + np.arange(16)
                flat = (e4 * n_rows + r) * row_bytes + col
                ix[:, nt, ks] = np.where(r < n_rows, flat, -1)
        return aid, ix.reshape(-1)

    def scales(aid, rows_of, n_tiles, nks, nkb, n_rows, sf_row_bytes):
        # [E][tile][scale word][fragment][lane][4 bytes]: byte b of the word is the scale of K
        # step 4*word + b for the lane's 32-block (lane/16) of its column; 0 past the last step
        ix = np.full((E, n_tiles, nkb, 16, 64, 4), -1, dtype=np.int64)
        for nt in range(n_tiles):
            r = rows_of(nt)[None]
            for kb in range(nkb):
                for b in range(4):
                    ks = 4 * kb + b
                    if ks < nks:
                        flat = (e3 * n_rows + r) * sf_row_bytes + ks * 4 + (L >> 4)[None]
                        ix[:, nt, kb, :, :, b] = np.where(r < n_rows, flat, -1)
        return aid, ix.reshape(-1)

    parts = [data(0, l1_row, nb1, ks1, 2 * I, H // 2), scales(1, l1_row, nb1, ks1, nkb1, 2 * I, H // 32),
             data(2, l2_row, nt2, ks2, H, I // 2), scales(3, l2_row, nt2, ks2, nkb2, H, I // 32)]
    total = 0
    offs = []
    for _, ix in parts:
        offs.append(total)
        total = _align(total + ix.size)
    aid = np.full(total, -1, dtype=np.int64)
    flat = np.full(total, -1, dtype=np.int64)
    for o, (a, ix) in zip(offs, parts):
        aid[o:o + ix.size] = np.where(ix >= 0, a, -1)
        flat[o:o + ix.size] = ix
    return aid, flat


def expected_packed(arrays, aid, flat):
    out = np.zeros(aid.size, dtype=np.uint8)
    for a, arr in enumerate(arrays):
        sel = aid == a
        out[sel] = arr.reshape(-1)[flat[sel]]
    return out


SHAPES = [
    (4, 256, 512),     # the tiny workload's shape
    (2, 384, 256),     # H an odd multiple of 128: W2's last column tile completed with zero rows
    (3, 640, 384),     # several K steps, scale words with unused bytes in both matrices
    (1, 128, 128),     # one K step in each matrix
    (2, 1152, 640),    # more than one scale word per row in both matrices
]


@pytest.mark.parametrize("E,H,I", SHAPES)
def test_index_map_places_every_input_byte_once(E, H, I):
    """The host model of the layout itself: each input byte appears exactly once, every
    other byte is padding (no GPU; runs in the CPU suite too)."""
    aid, flat = packed_index_map(E, H, I)
    sizes = [E * 2 * I * H // 2, E * 2 * I * H // 32, E * H * I // 2, E * H * I // 32]
    for a, n in enumerate(sizes):
        got = np.sort(flat[aid == a])
        assert np.array_equal(got, np.arange(n)), a


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
@pytest.mark.parametrize("E,H,I", SHAPES)
def test_prepare_weights_layout(E, H, I):
    print(f"[pack] E={E} H={H} I={I}", flush=True)
    g = torch.Generator().manual_seed(E * 1000 + H + I)
    rnd = lambda *shape: torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
    w1, w1_sf = rnd(E, 2 * I, H // 2), rnd(E, 2 * I, H // 32)
    w2, w2_sf = rnd(E, H, I // 2), rnd(E, H, I // 32)
    shape = moe.make_shape(E, H, I, 1, 1)
    nb = moe.moe_packed_weights_bytes(shape)
    aid, flat = packed_index_map(E, H, I)
    want = expected_packed([w1.numpy(), w1_sf.numpy(), w2.numpy(), w2_sf.numpy()], aid, flat)
    assert nb == want.size
    packed = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")    # poison
    moe.moe_prepare_weights(shape, w1.cuda(), w1_sf.cuda(), w2.cuda(), w2_sf.cuda(), packed)
    torch.cuda.synchronize()
    got = packed.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    print(f"[pack] {nb} bytes, {len(bad)} differ", flush=True)
    assert len(bad) == 0, f"first differing byte offsets {bad[:8]}"
