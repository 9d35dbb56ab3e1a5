"""MI355X-native BLASST block-skipping attention (placeholder, filled below)."""
