"""CPU oracle for the DSA path. Test infrastructure: see dsa_oracle's header."""
