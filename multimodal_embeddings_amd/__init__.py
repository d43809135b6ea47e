"""MI355X-native forward pass of the uniform byte encoder (placeholder; binding follows)."""
