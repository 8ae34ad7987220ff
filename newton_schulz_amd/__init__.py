"""libmuon: Muon optimizer hot path (momentum, Newton-Schulz, apply) for AMD MI355X."""
