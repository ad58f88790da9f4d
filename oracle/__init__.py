"""CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct float64 references written from the pages'
definitions.  Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import, call or link anything in this package; the
HIP product path never does, and the two share no code.

Pins (what fixes these references other than themselves) live in
``tests/test_oracle.py``: the worked row printed on the pages, library routines
(scipy's softmax/logsumexp, PyTorch's float64 CPU attention), closed forms,
invariants, and exact-sum brute force on tiny inputs.  No function here is
"parity unpinned".
"""
