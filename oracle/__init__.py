"""CPU oracle of the compressed attention core (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  ``csa_oracle`` is the per-query float64 definition; ``brute`` is an
independent dense-mask formulation used to pin it on tiny shapes.
"""
