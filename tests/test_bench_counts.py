"""The benchmark's algorithmic work counts (the numerators of every reported
roofline fraction), checked against the same quantities counted a second way:
from the tensor sizes of the workloads, element by element, on the CPU."""
import math

import bench

B, T, H, D, N, C = 8, 2048, 48, 64, 64, 64  # the Mamba-style layer


def test_chunk_scan_flops_counts_the_causal_triangle():
    # per chunk: score tiles over the l >= s triangle (N-long complex dot products),
    # the same triangle times X (D columns), and the C x N x D carried-state readout
    nC = T // C
    pairs = sum(l + 1 for l in range(C))  # (l, s) with s <= l
    cmacs = pairs * N + pairs * D + C * N * D
    assert bench.chunk_scan_flops(B, T, H, D, N, C) == 8 * B * H * nC * cmacs
    assert bench.chunk_scan_flops(B, T, H, D, N, C) == 51_942_260_736


def test_chunk_state_flops():
    assert bench.chunk_state_flops(B, T, H, D, N, C) == 8 * B * H * (T // C) * C * N * D
    assert round(bench.chunk_state_flops(B, T, H, D, N, C) / 1e9, 1) == 25.8


def test_forward_bytes_from_tensor_sizes():
    plane = 4  # bytes of one fp32 plane element
    x = y = B * T * H * D * 2 * plane
    b = c = B * T * H * N * 2 * plane
    dt = B * T * H * 4
    hT = B * H * N * D * 2 * plane
    assert bench.forward_hbm_bytes(B, T, H, D, N) == x + b + c + dt + y + hT
    assert round(bench.forward_hbm_bytes(B, T, H, D, N) / 1e9, 3) == 1.626


def test_state_scan_bytes_from_tensor_sizes():
    rows = B * T * H
    reads = rows * (N + D) * 2 * 4
    writes = B * H * (T // C) * N * D * 2 * 4 + B * H * N * D * 2 * 4  # H_c, then hT
    assert bench.state_scan_hbm_bytes(B, T, H, D, N, C) == reads + writes


def test_decode_bytes_from_tensor_sizes():
    Bd, Hd, Nd, Dd = 256, 48, 128, 64
    state = Bd * Hd * Nd * Dd * 2 * 4
    io = Bd * Hd * (Dd + Dd + Nd + Nd) * 2 * 4  # x, y (D each), B, C (N each), complex
    dt = Bd * Hd * 4
    assert bench.decode_hbm_bytes(Bd, Hd, Dd, Nd) == 2 * state + io + dt
    assert round(bench.decode_hbm_bytes(Bd, Hd, Dd, Nd) / 1e9, 3) == 1.648


def test_born_flops_per_pair():
    Bb, Tb, Hb, Db = 2, 5, 3, 16
    pairs = sum(i + 1 for i in range(Tb))
    per_pair = 8 * Db + 3 + 4 * Db + 1  # overlap, modulus, weighted sum, normaliser
    assert bench.born_flops(Bb, Tb, Hb, Db) == Bb * Hb * pairs * per_pair


def test_phase_scan_bytes():
    Bp, Tp, Hp, Np = 3, 7, 2, 16
    per_step = (4 + 4 + 8) + 8  # phi, u, b read; psi written
    assert bench.phase_scan_hbm_bytes(Bp, Tp, Hp, Np) == Bp * Tp * Hp * Np * per_step + Bp * Hp * Np * 16
    assert math.isclose(bench.cumsum_hbm_bytes(1, 64, 1, 64), 64 * 4 + 64 * 32 + 8)
