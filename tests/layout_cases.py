"""Problems with launch hints that force each register-resident W_hh layout
of the scan (shared by the CPU planner test and the GPU parity test).

Each entry: name, mode, dtype, T, B, F, H, P, tile_batch, tile_hidden,
bidirectional, layout, varlen, expected (wreg, tiles per wave, K split,
chunks per tile)."""

REG_CASES = [
    ("reg_nt1_ks2", "lstm", "f32", 8, 16, 24, 128, 0, 16, 8, False, "padded", None, (1, 1, 2, 4)),
    ("reg_nt1_ks4_gru", "gru", "f32", 8, 16, 24, 256, 0, 16, 4, False, "padded", None, (1, 1, 4, 4)),
    ("reg_nt2_bf16_gru", "gru", "bf16", 8, 16, 32, 128, 0, 16, 32, False, "padded", None, (1, 2, 1, 4)),
    ("reg_nt1_bf16", "lstm", "bf16", 8, 16, 32, 128, 0, 16, 16, False, "padded", None, (1, 1, 1, 4)),
    ("reg_valu_bf16", "lstm", "bf16", 8, 3, 16, 512, 0, 3, 16, False, "padded", None, (1, 0, 4, 16)),
    ("reg_valu_unsplit", "lstm", "f32", 8, 2, 16, 32, 0, 2, 8, False, "padded", None, (1, 0, 1, 8)),
    ("reg_valu_rows_gru", "gru", "f32", 8, 7, 16, 64, 0, 7, 64, False, "padded", None, (1, 0, 1, 16)),
    ("reg_two_rowtiles", "lstm", "f32", 8, 40, 16, 64, 0, 32, 16, False, "padded", None, (1, 1, 1, 4)),
    ("reg_nt4_lstmp_bf16", "lstmp", "bf16", 8, 16, 32, 128, 128, 16, 64, False, "padded", None, (1, 4, 1, 4)),
    ("reg_bi_packed", "lstm", "f32", 12, 20, 16, 128, 0, 16, 8, True, "packed", (1, 12), (1, 1, 2, 4)),
    ("lds_odd_k", "gru", "f32", 8, 16, 24, 33, 0, 16, 11, False, "padded", None, (0, 0, 0, 0)),
]
