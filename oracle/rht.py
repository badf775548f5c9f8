"""32-point randomized Hadamard transform (oracle; test infrastructure only).

The pages name a random Hadamard transform applied before quantizing, to bound
the variance that block outliers cause, with a Hadamard size of 32 for MXFP4
("MXFP4", AI Wiki, §Training with MXFP4 table: Tseng et al.; NVIDIA NVFP4
pretraining row; "Training an MoE LLM in MXFP4", summary).  They do not write
the transform out.  The reading taken:

    y = c * H32 * (d . x)

per 32-element block along the blocking axis, where H32 is the Sylvester
Hadamard matrix H[i][j] = (-1)^popcount(i & j) (natural order, no bit
reversal), d_i = -1 when bit i of a 32-bit sign mask is set (else +1), and
c = float32(1/sqrt(32)) = 0x3E3504F3, so c*H32 is (up to the rounding of c)
orthonormal.  The float32 evaluation order is fixed so that two independent
implementations agree bit for bit: the sign flip (exact), then the in-place
fast Walsh-Hadamard transform with stages h = 1, 2, 4, 8, 16, each mapping
(x_i, x_{i+h}) -> (x_i + x_{i+h}, x_i - x_{i+h}) for every i with i & h == 0,
each sum rounded to float32; then one float32 multiply by c.

The inverse (used by dequantize) is d . (c * H32 * y) in the same order: the
same five stages, the multiply by c, then the sign flip.
"""

import numpy as np

RHT_C_BITS = 0x3E3504F3
RHT_C = np.array([RHT_C_BITS], dtype=np.uint32).view(np.float32)[0]


def _signs(mask):
    bits = (int(mask) >> np.arange(32)) & 1
    return np.where(bits == 1, np.float32(-1.0), np.float32(1.0)).astype(np.float32)


def _fwht_f32(blocks):
    """blocks: float32 [..., 32]; returns the un-normalised transform in float32."""
    x = np.array(blocks, dtype=np.float32, copy=True)
    lead = x.shape[:-1]
    for h in (1, 2, 4, 8, 16):
        v = x.reshape(lead + (32 // (2 * h), 2, h))
        a = v[..., 0, :]
        b = v[..., 1, :]
        s = (a + b).astype(np.float32)
        d = (a - b).astype(np.float32)
        x = np.stack([s, d], axis=-2).reshape(lead + (32,))
    return x


def rht_forward_f32(blocks, mask):
    """Apply y = c * H32 * (d . x) to float32 blocks [..., 32]."""
    x = np.asarray(blocks, dtype=np.float32) * _signs(mask)   # exact sign flips
    y = _fwht_f32(x)
    return (y * RHT_C).astype(np.float32)


def rht_inverse_f32(blocks, mask):
    """Apply x = d . (c * H32 * y) to float32 blocks [..., 32]."""
    y = _fwht_f32(np.asarray(blocks, dtype=np.float32))
    y = (y * RHT_C).astype(np.float32)
    return (y * _signs(mask)).astype(np.float32)


def hadamard32_f64():
    """Sylvester H32 as float64, built by the Kronecker recursion H_{2n} = [[H, H], [H, -H]]."""
    h = np.ones((1, 1))
    while h.shape[0] < 32:
        h = np.block([[h, h], [h, -h]])
    return h
