"""MI355X-native Exact Flow Linear Attention (EFLA) hot path."""
