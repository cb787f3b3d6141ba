"""Benchmark of the sparse MoE feed-forward layer (placeholder, filled in below)."""


def decode_tokens_per_s_bound(bandwidth_Bps: float, bytes_per_token: float) -> float:
    """Bandwidth-bound decode rate: every token streams its active weights once."""
    return bandwidth_Bps / bytes_per_token
