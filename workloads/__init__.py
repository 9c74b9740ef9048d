"""Seeded synthetic inputs for absorbed-MLA decoding, shared by the tests,
the benchmark and the smoke check.  Holds none of the method's arithmetic:
only random numbers, paged block tables, top-k index lists and the cache
encoders that turn random values into 656-, 528- and 288-byte records."""

from .gen import (Workload, make_config, make_dense, make_sparse, make_fp8_dense,  # noqa: F401
                  make_fp8_sparse, make_sparse_prefill, PrefillWorkload, make_v41_sparse, encode_v41_records,
                  make_fp4_sparse, encode_fp4_records, CONFIG_NAMES)
from .accounting import flops_and_bytes  # noqa: F401
