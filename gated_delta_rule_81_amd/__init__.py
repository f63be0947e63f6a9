"""MI355X-native Kimi Delta Attention (KDA) operator."""
