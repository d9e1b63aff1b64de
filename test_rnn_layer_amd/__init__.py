"""MI355X-native TTT-MLP layer scan: a C-ABI HIP library plus a thin Python binding."""
