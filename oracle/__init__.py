"""CPU reference of the Llama-3 decoder forward pass: test infrastructure only."""
