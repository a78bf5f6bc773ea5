"""MI355X-native multi-head scaled dot-product attention (forward)."""
