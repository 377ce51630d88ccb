"""MI355X-native varlen FlashAttention backward (TND layout)."""
