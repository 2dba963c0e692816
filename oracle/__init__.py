"""CPU oracle package: TEST INFRASTRUCTURE ONLY (see snapkv_oracle.py)."""
