"""Algorithmic bytes of one decode step (the traffic the method must move).

Per tile and step: the codes and step sizes are read and written, q, k (d_k
each) and v (d_v) are read, the gates are read, o (fp32, d_v) is written, and
with a low-rank bypass the decayed U is read and written and W read at the
average fill k + (m-1)/2, plus the appended column pair. With a full
pure-write window of W E4M3 pairs: the W-1 staying keys are read and written,
their values read, the leaving pair read and the new pair written, which is
2 W d_k + (W + 1) d_v bytes. This is the figure
the roofline fraction is computed from; hardware counters report the traffic
actually moved.

A bypass merge (every m steps) reads and writes the codes and step sizes,
reads the k + m held column pairs and writes the k kept ones.
"""


def step_bytes_per_tile(bits, group, scale_bytes, d_k, d_v, in_bytes, gate_bytes, k=0, m=0, pw=0):
    if bits == 32:
        state = 4 * d_k * d_v
    else:
        state = d_k * d_v * bits // 8 + d_k * (d_v // group) * scale_bytes
    b = 2 * state + (2 * d_k + d_v) * in_bytes + gate_bytes + 4 * d_v
    if m > 0:
        nbar = k + (m - 1) / 2.0
        b += nbar * (4 * d_k + 2 * d_v) + 2 * (d_k + d_v)
    if pw > 0:
        b += 2 * pw * d_k + (pw + 1) * d_v
    return b


def merge_bytes_per_tile(bits, group, scale_bytes, d_k, d_v, k, m):
    """Algorithmic bytes of one bypass merge of one tile."""
    state = d_k * d_v * bits // 8 + d_k * (d_v // group) * scale_bytes
    return 2 * state + (k + m) * 2 * (d_k + d_v) + k * 2 * (d_k + d_v)


def workload_merge_bytes(batch, head_bits, group, scale_dtype, d_k, d_v, k, m):
    """Total algorithmic bytes of one merge over batch x heads tiles."""
    sb = 2 if scale_dtype == "f16" else 4
    return batch * sum(merge_bytes_per_tile(int(b), group, sb, d_k, d_v, k, m) for b in head_bits)


def gate_bytes(model, d_k):
    return {"retnet": 0, "mamba2": 4, "gdn": 8, "gla": 4 * d_k}[model]


def workload_step_bytes(model, batch, head_bits, group, scale_dtype, d_k, d_v, in_dtype,
                        lrb_k=0, lrb_m=0, pw=0):
    """Total algorithmic bytes of one step over batch x heads tiles."""
    sb = 2 if scale_dtype == "f16" else 4
    ib = 2 if in_dtype == "bf16" else 4
    gb = gate_bytes(model, d_k)
    per_batch_row = sum(step_bytes_per_tile(int(b), group, sb, d_k, d_v, ib, gb, lrb_k, lrb_m, pw)
                        for b in head_bits)
    return batch * per_batch_row
