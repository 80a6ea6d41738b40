// SHA-256 (FIPS 180-4) for the host prefix cache's block keys.
#pragma once

#include <array>
#include <cstddef>
#include <cstdint>

namespace pa {

using Digest = std::array<uint8_t, 32>;

// Digest of the concatenation of the given byte ranges.
Digest sha256(const uint8_t* const* parts, const size_t* sizes, int num_parts);

}  // namespace pa
