"""Units (batch row x KV head) and steps the full-size parity tests compare one by one."""
H2O_UNITS = (0, 77, 255)      # of 64 x 4 units of the 16K H2O workload
OMNI_UNITS = (3, 130)         # of 64 x 4 units of the 16K OmniKV workload
OMNI_STEPS = (0, 3)           # decode steps of the OmniKV sweep compared (steps 0..3 run)
SNAP_UNITS = (0, 13, 31)      # of 8 x 4 units of the 128K SnapKV workload
