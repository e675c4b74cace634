"""Memory accounting from the pages (exact integer arithmetic).

Test infrastructure only (see the package docstring).
"""


def value_budget(n_tokens, head_dim=128, ratio=4, hidden=128, index_numbers=2):
    """The explainer's memory worked example for one head.

    The dense value cache holds n_tokens * head_dim numbers; a target ratio
    leaves that divided by the ratio. The predictor costs its three weight
    matrices (head_dim x hidden, hidden x head_dim and the head_dim x head_dim
    linear map) plus the hidden and output biases. Each residual costs its
    head_dim numbers plus an index counted as two numbers. Returns a dict of
    the intermediate quantities; ``residuals`` is the real quotient (the page
    rounds it).
    """
    dense = n_tokens * head_dim
    budget = dense // ratio
    predictor = 2 * head_dim * hidden + head_dim * head_dim + hidden + head_dim
    remaining = budget - predictor
    per_residual = head_dim + index_numbers
    residuals = remaining / per_residual
    return {"dense": dense, "budget": budget, "predictor": predictor,
            "remaining": remaining, "per_residual": per_residual,
            "residuals": residuals, "token_fraction": residuals / n_tokens,
            "predictor_share": predictor / budget}


def dense_kv_bytes_per_token(n_layers=32, n_kv_heads=8, head_dim=128, elem_bytes=2):
    """Uncompressed K and V bytes per cached token over all layers."""
    return n_layers * 2 * n_kv_heads * head_dim * elem_bytes
