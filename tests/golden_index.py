"""Output positions of the token rows a row-only golden stores (pure index arithmetic, no model)."""
import numpy as np


def rows_positions(cfg, tokens):
    """Flat output positions of every value the given tokens produce, in the order of a row-only golden's
    z [B, T, 4 C_out]: unpatchify writes out[b, c, f, 2h+i, 2w+j] = z[b, n, (2i+j) C_out + c] for token
    n = (f H' + h) W' + w (the printed reshape / permute of the head's output)."""
    B, C, F, H, W = cfg.out_shape
    n = np.asarray(tokens, dtype=np.int64)
    f, h, w = n // (cfg.post_h * cfg.post_w), (n // cfg.post_w) % cfg.post_h, n % cfg.post_w
    b = np.arange(B)[:, None, None]
    k = np.arange(4 * C)[None, None, :]
    ij, c = k // C, k % C
    i, j = ij // 2, ij % 2
    yy = 2 * h[None, :, None] + i
    xx = 2 * w[None, :, None] + j
    return (((b * C + c) * F + f[None, :, None]) * H + yy) * W + xx
