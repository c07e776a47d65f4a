// Byte layout of the planar uintx shards (page uintx_quant.py, pack_uintx): one shard
// per power of two present in nbits, widest first, the k-bit shard holding bits
// [off, off + k) of every code; each shard is ceil(numel / (8/k)) bytes, and byte i of
// a shard holds the codes i, i + L, i + 2L, ... (L = that shard's byte count).
#pragma once

#include <stdint.h>

namespace gwb {

struct Shards {                  // byte offsets of the present shards in the packed buffer
  int64_t base4, base2, base1;
};
inline Shards shards_of(int nbits, int64_t numel) {
  Shards s{};
  const int64_t L4 = (numel + 1) / 2, L2 = (numel + 3) / 4;
  s.base4 = 0;
  s.base2 = (nbits & 4) ? L4 : 0;
  s.base1 = s.base2 + ((nbits & 2) ? L2 : 0);
  return s;
}
// bit offsets of the 2-bit and 1-bit shards' fields within a code (pack order 4, 2, 1)
template <int NB> struct ShardBits {
  static constexpr bool has4 = NB & 4, has2 = NB & 2, has1 = NB & 1;
  static constexpr int off2 = has4 ? 4 : 0;
  static constexpr int off1 = (has4 ? 4 : 0) + (has2 ? 2 : 0);
};

// The same layout with nbits known only at run time (any numel).
struct RaggedShards {
  int64_t base4, base2, base1;
  int off2, off1;
  bool has4, has2, has1;
};
inline RaggedShards ragged_shards(int nbits, int64_t numel) {
  const Shards b = shards_of(nbits, numel);
  return RaggedShards{b.base4, b.base2, b.base1, (nbits & 4) ? 4 : 0,
                      ((nbits & 4) ? 4 : 0) + ((nbits & 2) ? 2 : 0),
                      (nbits & 4) != 0, (nbits & 2) != 0, (nbits & 1) != 0};
}

}  // namespace gwb
