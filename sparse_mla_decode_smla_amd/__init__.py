"""Head-batched sparse MLA decode for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libsmla.so`` built from ``csrc/``;
``sparse_mla_decode_smla_amd.binding`` marshals torch tensors into its calls
and ``sparse_mla_decode_smla_amd.inputs`` makes seeded synthetic workloads.
Import the submodule you need; nothing is loaded at package import, so the
input generator also works where the library is not built.
"""
