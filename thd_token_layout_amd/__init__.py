"""MI355X-native THD context-parallel token layout and owner gradient return.

The compute path is the HIP library ``libcpthd.so`` (C ABI declared in
``include/cpthd.h``).  ``thd_token_layout_amd.cpthd`` is its Python binding:
importing it loads the library and raises if the library has not been built.
``thd_token_layout_amd.workloads`` holds the seeded synthetic input generators.
"""
