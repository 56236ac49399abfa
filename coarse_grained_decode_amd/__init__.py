"""SPICY-KV coarse-grained decode for MI355X (placeholder; binding added with the library)."""
