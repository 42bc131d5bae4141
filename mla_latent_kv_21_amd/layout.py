"""Shapes of the device buffers the library reads and writes (pure Python, no GPU).

* latent cache: [num_blocks, block_size, d_c + d_r]; row = [c || k_r], k_r stored rotated.
* expanded GQA cache: [num_blocks, block_size, 2*G*d_h + d_r];
  row = [K_0 .. K_{G-1} || V_0 .. V_{G-1} || k_r].
* block table: int32 [B, max_blocks]; position p of sequence b lives in slot
  table[b][p / block_size] * block_size + p % block_size.
"""


def latent_cache_shape(d_c: int, d_r: int, num_blocks: int, block_size: int):
    return (num_blocks, block_size, d_c + d_r)


def gqa_cache_shape(n_groups: int, d_h: int, d_r: int, num_blocks: int, block_size: int,
                    d_v: int | None = None):
    d_v = d_h if d_v is None else d_v
    return (num_blocks, block_size, n_groups * d_h + n_groups * d_v + d_r)
