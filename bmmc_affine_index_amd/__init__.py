"""MI355X-native BMMC index permutations (placeholder; the binding follows)."""
