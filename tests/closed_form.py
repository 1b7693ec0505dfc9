"""Builder for the inputs of tests/golden/closed_form_ffn.json (the hand-derived example)."""
import numpy as np


def _pack(codes: np.ndarray) -> np.ndarray:
    """nibble codes [..., K] -> bytes [..., K/2], element 2i in the low nibble."""
    codes = codes.astype(np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def build_closed_form_inputs():
    T, E, k, H, I = 2, 2, 2, 128, 128
    x = np.full((T, H), 0x38, dtype=np.uint8)
    x[1, 1::2] = 0x30
    x_sf = np.zeros((T, 4), dtype=np.uint8)
    x_sf[:, 0] = 127
    topk_idx = np.array([[0, 1], [1, -1]], dtype=np.int32)
    topk_w = np.array([[0.75, 0.25], [0.5, 0.5]], dtype=np.float32)

    w1c = np.zeros((E, 2 * I, H), dtype=np.uint8)
    # expert 0: gate row 0 -> c<68 = 1.0 (code 2); gate rows 1.. -> c<64 = 1.0; up rows all 1.0
    w1c[0, 0, :68] = 2
    w1c[0, 1:I, :64] = 2
    w1c[0, I:, :] = 2
    # expert 1: gate rows -> odd elements 2.0 (code 4); up rows all -0.5 (code 9)
    w1c[1, :I, 1::2] = 4
    w1c[1, I:, :] = 9
    w2c = np.zeros((E, H, I), dtype=np.uint8)
    w2c[0, 0::2, :] = 1   # 0.5
    w2c[0, 1::2, :] = 2   # 1.0
    w2c[1, :, :] = 2
    w2c[1, 0, :] = 4      # 2.0
    w1 = _pack(w1c)
    w2 = _pack(w2c)
    w1_sf = np.full((E, 2 * I, H // 32), 127, dtype=np.uint8)
    w2_sf = np.full((E, H, I // 32), 127, dtype=np.uint8)
    return dict(x_fp8=x, x_sf=x_sf, topk_idx=topk_idx, topk_weights=topk_w,
                w1=w1, w1_sf=w1_sf, w2=w2, w2_sf=w2_sf)


def expected_y_bits():
    H = 128
    y = np.zeros((2, H), dtype=np.uint16)
    y[0, 0] = 0xC800
    y[0, 1::2] = 0x4900
    y[0, 2::2] = 0x4800
    y[1, 0] = 0xC8C0
    y[1, 1:] = 0xC840
    return y
