"""CPU oracle for one GPT-2 training step.  Test infrastructure only."""
