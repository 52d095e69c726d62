"""Measurement programs behind the design notes: matrix-unit and
transcendental throughput, LDS read bandwidth, and the per-phase cycle split
of the forward. Not part of the library."""
