"""CPU oracle for the RWKV-7 WKV7 recurrence and time-mix block.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, f64 restatement of
what the method computes, written from the pages (each function cites the
page and section it follows).  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import or execute it.  It shares
no code with the HIP library and never imports it; the HIP path never imports
this package.

Modules:
  wkv7      -- ctypes front end of ``wkv7_oracle.c`` (the recurrence, f64 C).
  timemix   -- the time-mix block forward and hand-derived backward (numpy f64).
  stack     -- LayerNorm, channel-mix, embedding/head and the decode stack.
  build     -- compiles ``wkv7_oracle.c`` with gcc.
"""
