"""CPU oracle for exact tiled attention: TEST INFRASTRUCTURE ONLY.

Plain, slow FP64 definitions written from the source pages. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. The HIP library never imports, links or calls it, and it
never imports the HIP library.
"""
