"""Test-only GPU probes of hardware behaviour the kernels' error bounds rest on."""
