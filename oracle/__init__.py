"""CPU oracle of RocketKV's hot path (test infrastructure only; never imported by the product)."""
