// sfag_sort.hip -- radix sort of 64-bit (key row << 32 | pair) sort keys for the deterministic
// dK / dV reduction: after sorting, the pairs of every key row are contiguous and in ascending
// pair order, which fixes the order of the summation.
#include <hipcub/hipcub.hpp>

#include "sfag_launch.h"

namespace sfag {

size_t sort_temp_bytes(int64_t n, int end_bit) {
  size_t bytes = 0;
  hipcub::DeviceRadixSort::SortKeys(nullptr, bytes, static_cast<const uint64_t*>(nullptr),
                                    static_cast<uint64_t*>(nullptr), (int)n, 0, end_bit);
  return bytes;
}

hipError_t sort_pair_keys(void* temp, size_t temp_bytes, const uint64_t* in, uint64_t* out, int64_t n,
                          int end_bit, hipStream_t st) {
  return hipcub::DeviceRadixSort::SortKeys(temp, temp_bytes, in, out, (int)n, 0, end_bit, st);
}

}  // namespace sfag
