"""MI355X (gfx950) parallel Newton / quasi-Newton solver for nonlinear recurrences.

``evaluation_nonlinear_rnns_amd.deer`` binds the HIP library (include/deer.h);
``evaluation_nonlinear_rnns_amd.inputs`` draws the seeded synthetic workloads.
The library is loaded on first use, never at import.
"""
