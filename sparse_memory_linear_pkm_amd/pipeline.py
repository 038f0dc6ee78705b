"""Host-side chunk schedule of a pipelined single-sequence prefill.

The prefill of one sequence can be split into chunks of consecutive tokens
(every [B, T, H, ...] array of a single sequence is then cut into contiguous
slices): the PKM addressing of chunk c + 1 runs on a second stream, at most
one workgroup per CU (``sdm_pkm_address_overlapped``), while the scan of
chunk c runs on the main stream; the scan over consecutive chunks gives the
same bits as one call over all tokens.  Only the first chunk's addressing is
exposed, and every chunk boundary costs one launch tail of the scan, so the
chunks start small and grow: the overlapped addressing of a token takes
about two thirds of the scan's time per token on the MI355X, so a chunk may
be up to 1.5 times the previous one and its addressing still finishes under
the previous chunk's scan.
"""


def prefill_chunks(T: int, first: int = 16384, growth: float = 1.5, cap: int = 131072, align: int = 512):
    """Token counts of the chunks, in order; they sum to T.  Chunks grow from
    `first` by `growth` up to `cap` tokens, each a multiple of `align` except
    the last (which takes what is left)."""
    if T < 0 or first < align or cap < first or growth < 1.0 or align < 1:
        raise ValueError("prefill_chunks: need T >= 0, align <= first <= cap, growth >= 1")
    out, t, g = [], 0, float(first)
    while t < T:
        c = min(int(g) // align * align, cap, T - t)
        out.append(c)
        t += c
        g = min(g * growth, float(cap))
    return out
