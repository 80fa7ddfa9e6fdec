"""MI355X-native Muon bank step: HIP kernels for gfx950 behind a C ABI.

The compute lives in ``libmuonbank.so`` (built from ``csrc/``); this package
only marshals arguments to it.  ``workloads`` draws the seeded synthetic
inputs used by the tests and the benchmark.
"""
