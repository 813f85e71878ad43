"""CPU oracle for centroid-indexed KV-cache retrieval (LouisKV's hot path).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, constants or
helpers with the HIP library; both sides receive the same seeded inputs from
``workloads`` and are compared afterwards.

Everything here is plain numpy in float64 (plus pure-Python loops for the
brute-force cases), written to be checked against the pages by eye:

* ``kmeans``    -- Lloyd K-means per KV head, centroid = member mean
                   (LouisKV note, key design 2).
* ``boundary``  -- semantic-boundary test r_t < tau on adjacent queries
                   (LouisKV note, key design 1, the r_t equation).
* ``select``    -- group-consistent centroid scoring and budgeted selection of
                   variable-size units (LouisKV note, key design 3 items 2-3;
                   overall-framework flowchart "Top-B").
* ``attend``    -- exact softmax attention over the retrieved rows
                   (flowchart "Attention + FFN", attention part only).
* ``segments``  -- decode-time temporal segments and the fixed-size local
                   buffer (LouisKV note, key design 2, decode half).
* ``decode``    -- one decode loop composing the above in the flowchart's
                   order.

Readings of points the pages leave open are listed in each module's header.
"""
from . import attend, boundary, decode, kmeans, precision, segments, select  # noqa: F401
