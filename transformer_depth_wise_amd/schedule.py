"""Site schedule of one microbatch, driven through the C ABI.

Full routing ("Multi-Head Attention Residuals", Figure 3 and Appendix E):
before site s the rows it reads are committed (append), then the site routes;
the backward visits the sites in strictly reverse order.  Block routing
("Low-Rank Attention Residuals", Appendix H, Figure 11) is the same loop with
a transient source (the partial block sum) handed to the site's route.
"""

from __future__ import annotations

from .attnres import Bank


def run_microbatch(bank: Bank, nsrc, has_extra, queries, outs, dqs, extras=None, d_extras=None,
                   backward=True, stream=None, gains=None, dgains=None, append_stream=None):
    """Run every site forward, then (optionally) backward.

    The bank rows must already be in ``bank.rows`` (each append commits the
    next row in place) and each site's upstream gradient in
    ``bank.dout_rows[s]``.  ``outs[s]`` receives the site output,
    ``dqs[s]`` its query gradient, ``d_extras[s]`` the transient-source
    gradient; bank-row gradients land in ``bank.drows``.  With ``gains``
    ([S, r] float32 routing RMSNorm gains) their gradients land in ``dgains``.

    Everything runs on ``stream`` (torch's current stream when None), unless
    ``append_stream`` is given: the appends then run one site ahead on that
    stream, and each forward waits only for the appends of the rows it reads.
    An append writes only the cached statistics of later sites, so it may run
    beside the forward of the current site.
    """
    S = len(nsrc)
    extras = extras if extras is not None else [None] * S
    d_extras = d_extras if d_extras is not None else [None] * S
    bank.reset()
    bank.set_queries(nsrc, has_extra, queries)
    if gains is not None:
        bank.set_gains(gains, dgains, stream)
    committed = 0
    if append_stream is None:
        for s in range(S):
            while committed < nsrc[s]:
                bank.append(None, stream)
                committed += 1
            bank.route_fwd(s, extras[s], outs[s], stream)
    else:
        import torch
        main = stream if stream is not None else torch.cuda.current_stream()
        ready = torch.cuda.Event()
        ready.record(main)
        append_stream.wait_event(ready)  # rows written and gains folded before the appends
        done = []  # done[n]: recorded on the append stream after the append of row n
        for s in range(S):
            target = nsrc[s + 1] if s + 1 < S else nsrc[s]  # one site ahead
            while committed < max(target, nsrc[s]):
                bank.append(None, append_stream)
                ev = torch.cuda.Event()
                ev.record(append_stream)
                done.append(ev)
                committed += 1
            main.wait_event(done[nsrc[s] - 1])
            bank.route_fwd(s, extras[s], outs[s], main)
        end = torch.cuda.Event()
        end.record(append_stream)
        main.wait_event(end)
    if backward:
        for s in reversed(range(S)):
            bank.route_bwd(s, extras[s], None, dqs[s], d_extras[s], stream)


def run_block_microbatch(bank: Bank, nsrc, has_partial, queries, x, ys, outs, partials, douts=None,
                         dqs=None, dys=None, stream=None):
    """Block routing over sublayer outputs ("Low-Rank Attention Residuals",
    Appendix H, Figure 11), the partial sums kept by the bank.

    ``x`` [T, d] is the embedding (row 0), ``ys[t]`` the output of sublayer
    t + 1; the read after it sees rows [0, nsrc[t]) and, when
    ``has_partial[t]``, the block's running partial sum, accumulated into
    ``partials[t]`` (caller memory that must outlive the backward); a read
    without a partial follows a block end, whose sum the bank commits as the
    next row.  ``outs[t]`` receives the read's output.  With ``douts``, the
    backward runs too: ``dqs[t]`` gets the query gradient and ``dys[t]``
    (float32 [T, d]) the gradient of ys[t]; the embedding's gradient is left
    in ``bank.drows[0]``.
    """
    M = len(nsrc)
    bank.reset()
    bank.set_queries(nsrc, [2 if p else 0 for p in has_partial], queries)
    bank.append(x, stream)
    for t in range(M):
        if has_partial[t]:
            bank.accumulate(ys[t], partials[t], False, stream)
        else:
            bank.accumulate(ys[t], None, True, stream)
        bank.route_fwd(t, partials[t] if has_partial[t] else None, outs[t], stream)
    if douts is None:
        return
    for t in reversed(range(M)):
        # the row the block of sublayer t + 1 commits into: the last row read
        # after a block end, the next row while the block is open
        row = nsrc[t] if has_partial[t] else nsrc[t] - 1
        d_extra = bank.drows[row] if has_partial[t] else None
        bank.route_bwd(t, partials[t] if has_partial[t] else None, douts[t], dqs[t], d_extra,
                       stream)
        if dys is not None:
            dys[t].copy_(bank.drows[row])  # the gradient of ys[t], in stream order
