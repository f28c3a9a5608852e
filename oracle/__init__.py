"""CPU oracle for the Lynx codec and anchor-only decode attention (test infrastructure only)."""
