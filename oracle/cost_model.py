"""Oracle of the offload cost model (DAK paper §4.2.1 "The Suboptimality of Uniform
Offloading", Fig. 6; walkthrough sections on the offload-ratio model, the
memory-bound peak and the compute-bound lossless interval).

For one operation that touches C bytes (weights or KV), a fraction x of which
sits in host memory:
  T_g   = (1 - x) C / B_g        time to read the HBM part
  T_h   = x C / B_h              time to read the host part (concurrently)
  T     = max(T_comp, T_g, T_h)  the op is bound by the slowest of the three
  EB    = C / T                  effective bandwidth
Memory-bound ops (C / B_g > T_comp) peak at x* = B_h / (B_h + B_g) with
EB = B_g + B_h.  Compute-bound ops keep EB = B_i = C / T_comp up to
x* = B_h / B_i, after which the host read is exposed.
"""
from __future__ import annotations


def t_gpu(C: float, x: float, b_g: float) -> float:
    return (1.0 - x) * C / b_g


def t_host(C: float, x: float, b_h: float) -> float:
    return x * C / b_h


def op_time(C: float, x: float, t_comp: float, b_g: float, b_h: float) -> float:
    return max(t_comp, t_gpu(C, x, b_g), t_host(C, x, b_h))


def effective_bandwidth(C: float, x: float, t_comp: float, b_g: float, b_h: float) -> float:
    return C / op_time(C, x, t_comp, b_g, b_h)


def memory_bound_peak_ratio(b_g: float, b_h: float) -> float:
    """Where T_g = T_h: x* = B_h / (B_h + B_g)."""
    return b_h / (b_h + b_g)


def compute_bound_threshold(C: float, t_comp: float, b_h: float) -> float:
    """Where the host read time reaches T_comp: x* = B_h / B_i with B_i = C / T_comp."""
    b_i = C / t_comp
    return b_h / b_i


def is_memory_bound(C: float, t_comp: float, b_g: float) -> bool:
    """At x = 0 the op is limited by reading HBM rather than by computing."""
    return C / b_g > t_comp


def decreasing_end(C: float, t_comp: float, b_g: float, b_h: float) -> float:
    """End of the region where raising x lowers T (0 for compute-bound ops).

    T_g falls until it meets either T_h (at B_h/(B_h+B_g)) or T_comp
    (at 1 - T_comp B_g / C), whichever comes first.
    """
    if not is_memory_bound(C, t_comp, b_g):
        return 0.0
    return max(0.0, min(memory_bound_peak_ratio(b_g, b_h), 1.0 - t_comp * b_g / C))


def turning_point(C: float, t_comp: float, b_g: float, b_h: float) -> float:
    """Largest x at which T is still minimal (the op's turning point), capped at 1.

    Reduces to B_h/(B_h+B_g) when T_comp <= C/(B_g+B_h) and to B_h/B_i otherwise.
    """
    return min(1.0, b_h * max(t_comp, C / (b_g + b_h)) / C)


def unit_time(n: int, u: int, h: int, t_comp: float, b_g: float, b_h: float) -> float:
    """T for an op of n units of u bytes with h units on the host.

    Byte counts are integers, converted to double once, then divided by the
    bandwidth: the exact evaluation order the planner uses.
    """
    return max(t_comp, float((n - h) * u) / b_g, float(h * u) / b_h)


def two_tier_roofline_time(C: float, x_eff: float, b_hbm: float, b_host: float) -> float:
    """Memory-bound floor of a split op: max((1 - x) C / B_hbm, x C / B_host)."""
    return max((1.0 - x_eff) * C / b_hbm, x_eff * C / b_host)
