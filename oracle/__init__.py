"""CPU oracle for CD-RGE on an LSTM language model: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. The HIP product path (``zero_order_recurrent_amd``) never imports it, and the two
share no code: the oracle is plain single-threaded C++ compiled with g++.
"""
from .oracle import Oracle, OracleConfig, build_oracle, oracle_library_path  # noqa: F401
