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
                   backward=True, stream=None, gains=None, dgains=None):
    """Run every site forward, then (optionally) backward, on one stream.

    The bank rows must already be in ``bank.rows`` (each append commits the
    next row in place) and each site's upstream gradient in
    ``bank.dout_rows[s]``.  ``outs[s]`` receives the site output,
    ``dqs[s]`` its query gradient, ``d_extras[s]`` the transient-source
    gradient; bank-row gradients land in ``bank.drows``.  With ``gains``
    ([S, r] float32 routing RMSNorm gains) their gradients land in ``dgains``.
    """
    S = len(nsrc)
    extras = extras if extras is not None else [None] * S
    d_extras = d_extras if d_extras is not None else [None] * S
    bank.reset()
    bank.set_queries(nsrc, has_extra, queries)
    if gains is not None:
        bank.set_gains(gains, dgains, stream)
    committed = 0
    for s in range(S):
        while committed < nsrc[s]:
            bank.append(None, stream)
            committed += 1
        bank.route_fwd(s, extras[s], outs[s], stream)
    if backward:
        for s in reversed(range(S)):
            bank.route_bwd(s, extras[s], None, dqs[s], d_extras[s], stream)
