"""CPU oracle package (test infrastructure only; see ``lao.c``)."""
