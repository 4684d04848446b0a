"""The streaming-read yardstick bench.py measures the decode step against (measurement equipment, not part of the library)."""
