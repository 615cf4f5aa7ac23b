// Device scan and radix sort used by the device mask compiler and the device-built plans
// (the library's own kernels; deterministic, stable, one stream, no host synchronisation).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace bsfa {

// Exclusive prefix sum of n int32 values (out may equal in).  temp: device memory of at
// least dev_scan_temp_bytes(n) bytes, 16-byte aligned.
size_t dev_scan_temp_bytes(int64_t n);
hipError_t dev_exclusive_scan(const int32_t *in, int32_t *out, int64_t n, void *temp, size_t temp_bytes,
                              hipStream_t stream);

// Stable ascending sort of n 64-bit keys on bits [0, end_bit) (keys_in is not written).
size_t dev_sort_keys_temp_bytes(int64_t n, int32_t end_bit);
hipError_t dev_sort_keys_u64(const uint64_t *keys_in, uint64_t *keys_out, int64_t n, int32_t end_bit, void *temp,
                             size_t temp_bytes, hipStream_t stream);

// Stable ascending sort of n (32-bit key, int32 value) pairs on key bits [0, end_bit)
// (the inputs are not written).
size_t dev_sort_pairs_temp_bytes(int64_t n, int32_t end_bit);
hipError_t dev_sort_pairs_u32(const uint32_t *keys_in, uint32_t *keys_out, const int32_t *vals_in, int32_t *vals_out,
                              int64_t n, int32_t end_bit, void *temp, size_t temp_bytes, hipStream_t stream);

}  // namespace bsfa
