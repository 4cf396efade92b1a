"""CPU oracle for tree-summarised (ZHA) decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``hierarchical_kv_cache_amd``) never imports it and shares no
code with it; the two meet only on inputs drawn by ``synth``.

Everything here is plain numpy in float64, written from the definitions on the
pages, one (sequence, KV head) at a time, with no blocking or fusion beyond what
those definitions state.  See ``oracle.zha`` for the citations of each step.
"""
from .zha import *  # noqa: F401,F403
from .zha import __all__  # noqa: F401
