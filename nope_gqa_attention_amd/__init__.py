"""MI355X-native attention core of the hybrid sliding-window / NoPE GQA layer.

The compute path is the C-ABI library libbeamattn.so (hand-written HIP for gfx950);
`nope_gqa_attention_amd.beamattn` is its thin Python binding. Importing this package
loads nothing: the library is loaded on first use and fails loudly if it is missing.
"""
