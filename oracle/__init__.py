"""Float64 CPU oracle for absorbed-MLA split-KV decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code,
header, table or helper with the HIP library under ``mla_split_kv_02_amd/`` and
never imports it.
"""

from .mla_oracle import *  # noqa: F401,F403
