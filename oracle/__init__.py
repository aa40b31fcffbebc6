"""fp64 CPU oracle of jagged GDPA / JFA — TEST INFRASTRUCTURE ONLY.

Importable only by the tests, the smoke check and the benchmark's CPU-baseline
leg.  It shares no code with the GPU path; see ``ref.c`` for what it computes.
"""
