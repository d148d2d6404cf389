"""pytest plugin of the oracle mutation check (tests/test_oracle_mutations.py).

Loaded with ``-p tests.mutant_plugin`` in a child pytest process.  Before any
test runs it swaps in a mutated copy of the oracle, planted on the CPU:

- ORACLE_MUTANT_LIB=<path>: a shared library built from a mutated copy of
  oracle/ct_oracle.c replaces the oracle's C library;
- ORACLE_MUTANT_PY=<module>=<path>: the mutated source of an oracle Python
  module is executed in that module's namespace, replacing its functions.
"""
import ctypes
import importlib
import os


def pytest_configure(config):
    import oracle
    lib = os.environ.get("ORACLE_MUTANT_LIB")
    if lib:
        oracle._lib = oracle.bind(ctypes.CDLL(lib))
    py = os.environ.get("ORACLE_MUTANT_PY")
    if py:
        name, path = py.split("=", 1)
        mod = importlib.import_module(name)
        with open(path) as f:
            src = f.read()
        exec(compile(src, mod.__file__, "exec"), mod.__dict__)
