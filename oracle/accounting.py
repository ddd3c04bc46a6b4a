"""Storage and traffic accounting.

TEST INFRASTRUCTURE (see the package docstring).

Bits per state element ("Preserving Updates in Low-Bit Recurrent State
Quantization", Table 2 "Bits", Tables 6, 8 and 9 "Avg./Peak bits"):
codes b bits, plus one 16-bit step size per group of g, plus the bypass:
n column pairs of fp16 (d_k + d_v values each) spread over d_k*d_v elements.
Over one merge cycle the stored fill at the start of each step runs through
k, k+1, ..., k+m-1 (average k + (m-1)/2), and it peaks at k+m just before a
merge.
"""


def bits_per_element(bits, group, scale_bits, d_k, d_v, k=0, m=0):
    """(average, peak) storage bits per state element."""
    base = bits + scale_bits / group
    per_col = 16.0 * (d_k + d_v) / (d_k * d_v)
    avg = base + (k + (m - 1) / 2.0) * per_col if m > 0 else base
    peak = base + (k + m) * per_col if m > 0 else base
    return avg, peak


def tile_payload_bytes(bits, group, scale_bytes, d_k, d_v, cap=0, yoked=False, pw=0):
    """Bytes of one tile's state: codes + scales + bypass (+ fp32 reference)
    (+ a pure-write window of pw E4M3 pairs, one byte per value)."""
    if bits == 32:
        return 4 * d_k * d_v
    codes = d_k * d_v * bits // 8
    scales = d_k * (d_v // group) * scale_bytes
    bypass = 2 * cap * (d_k + d_v)
    ref = 4 * d_k * d_v if yoked else 0
    return codes + scales + bypass + ref + pw * (d_k + d_v)


def step_bytes_per_tile(bits, group, scale_bytes, d_k, d_v, in_bytes, gate_bytes,
                        k=0, m=0):
    """Bytes one decode step must move for one tile.

    codes and scales read and written, q, k (d_k each) and v (d_v) read, the
    gates read, o (fp32, d_v) written, and with a bypass: U read and written,
    W read (both at the average fill k + (m-1)/2) plus the appended column pair.
    """
    state = d_k * d_v * bits // 8 + d_k * (d_v // group) * scale_bytes if bits != 32 else 4 * d_k * d_v
    b = 2 * state + (2 * d_k + d_v) * in_bytes + gate_bytes + 4 * d_v
    if m > 0:
        nbar = k + (m - 1) / 2.0
        b += nbar * (4 * d_k + 2 * d_v) + 2 * (d_k + d_v)
    return b
