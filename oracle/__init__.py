"""CPU oracle for speculative KV coding.  Test infrastructure only: the product
package never imports it (see skvref.c for what it computes and why)."""
