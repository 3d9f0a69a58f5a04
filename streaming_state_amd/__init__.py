"""MI355X-native Mamba-2 streaming-state library (HIP kernels behind a C ABI).

``streaming_state_amd.ssm`` is the Python binding of ``libssm_stream.so``; it
raises ImportError when the library has not been built.  ``inputs`` holds the
seeded synthetic workload generators.
"""
