"""MI355X-native FlashHead two-stage retrieval head (HIP kernels, C ABI)."""
