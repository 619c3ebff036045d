"""Named workloads: shapes, generator settings and budgets.

Budgets E and S are shares of all N keys per sparse call: the exact set holds
about E*N keys and the shared sample m = round(S*N) draws.  Cq = 100 and
Ck = 500 are SVG2's clustering sizes, which the InstaGen pages report for
their SVG2-parameterised runs (InstaGen, thelatestinai.com page, Figure 2);
the 4+4 % .. 32+32 % sweep is the budget range of the same figure.
"""

WORKLOADS = {
    "tiny_f32": dict(
        B=1, H=1, N=2048, d=64, dtype="f32", n_centers=16, grid=None, q_scale=1.0,
        Cq=8, Ck=32, iters=5, sweep=[(0.25, 0.25)]),
    "wan1.3b_480p": dict(
        B=1, H=12, N=32760, d=128, dtype="bf16", n_centers=64, grid=(21, 30, 52),
        q_scale=1.0, Cq=100, Ck=500, iters=5, sweep=[(0.08, 0.08)]),
    "wan1.3b_720p": dict(
        B=1, H=12, N=75600, d=128, dtype="bf16", n_centers=64, grid=(21, 45, 80),
        q_scale=1.0, Cq=100, Ck=500, iters=5,
        sweep=[(0.04, 0.04), (0.16, 0.16), (0.32, 0.32)]),
    "wan14b_720p": dict(
        B=1, H=40, N=75600, d=128, dtype="bf16", n_centers=64, grid=(21, 45, 80),
        q_scale=1.0, Cq=100, Ck=500, iters=5,
        sweep=[(0.04, 0.04), (0.08, 0.08), (0.16, 0.16), (0.32, 0.32)]),
    # 84 latent frames (4x the 720p clip): the sequence-length scaling check
    "wan14b_720p_84f": dict(
        B=1, H=2, N=302400, d=128, dtype="bf16", n_centers=64, grid=(84, 45, 80),
        q_scale=1.0, Cq=100, Ck=500, iters=5, sweep=[(0.08, 0.08)]),
    # the headline shape with a log-normal spread of token norms (|q| |k| over a
    # wide range): the Cauchy-Schwarz bound of the logits is far above many rows'
    # logits (robustness of the attention's fixed per-row reference)
    "wan14b_720p_wide_norms": dict(
        B=1, H=40, N=75600, d=128, dtype="bf16", n_centers=64, grid=(21, 45, 80),
        q_scale=1.0, norm_spread=0.35, Cq=100, Ck=500, iters=5, sweep=[(0.08, 0.08)]),
    # a wider spread still: many rows' logits leave the fp32 range around the
    # anchored reference, so a share of the tiles goes through the rescaling pass
    "wan14b_720p_wider_norms": dict(
        B=1, H=40, N=75600, d=128, dtype="bf16", n_centers=64, grid=(21, 45, 80),
        q_scale=1.0, norm_spread=0.6, Cq=100, Ck=500, iters=5, sweep=[(0.08, 0.08)]),
    "wan14b_720p_stress_pq": dict(
        B=1, H=40, N=75600, d=128, dtype="bf16", n_centers=64, grid=(21, 45, 80),
        q_scale=0.2, zipf=1.2, Cq=100, Ck=500, iters=5, pq=(8, 256),
        sweep=[(0.08, 0.08)]),
}


def budget_keys(share: float, N: int) -> int:
    """Round a share of N keys to a key count: floor(share*N + 1/2)."""
    return int(share * N + 0.5)
