"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

Holds only input generation (value streams, shapes, schedules) and its device
fill / feed kernels; none of the decode method's arithmetic lives here.
"""
