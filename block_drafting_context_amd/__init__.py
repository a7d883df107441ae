"""MI355X-native DFlash2 block-drafting hot path (package under construction)."""
