// Stand-ins for the kernel launchers behind the C ABI, for a host-only build
// of api.hip's argument validation under AddressSanitizer and
// UndefinedBehaviorSanitizer. Each stand-in only counts the call; nothing is
// launched and no pointer is dereferenced.
#include "internal.hpp"

extern "C" int sep_stub_launches;
int sep_stub_launches = 0;

namespace sep {

namespace {
hipError_t hit() {
  ++sep_stub_launches;
  return hipSuccess;
}
}  // namespace

hipError_t launch_is_sep(const int32_t*, int64_t, const int32_t*, int, uint8_t*, hipStream_t) { return hit(); }
hipError_t launch_tile_class(const uint8_t*, int, int, int, int, int, int, uint8_t*, hipStream_t) { return hit(); }
hipError_t launch_dense_mask(const uint8_t*, int, int, int, int, uint8_t*, hipStream_t) { return hit(); }
hipError_t launch_index_compact(const uint8_t*, int, int, int32_t*, int32_t*, int32_t*, hipStream_t) { return hit(); }
hipError_t launch_mask_compact(const int32_t*, int, int, const int32_t*, int, uint8_t*, int32_t*, int32_t*, int32_t*,
                               hipStream_t) {
  return hit();
}
hipError_t launch_prefill(const void*, const void*, const void*, int, int, int, int, int, int, const uint8_t*,
                          const int32_t*, const int32_t*, int, int, float, void*, float*, hipStream_t) {
  return hit();
}
hipError_t launch_prefill_backward(const void*, const void*, const void*, const void*, const void*, const float*, int,
                                   int, int, int, int, int, const uint8_t*, const int32_t*, const int32_t*, int, int,
                                   float, float*, float*, float*, float*, hipStream_t) {
  return hit();
}
hipError_t launch_cache_reset(const sep_cache&, hipStream_t) { return hit(); }
hipError_t launch_cache_update(const sep_cache&, const void*, const void*, const int32_t*, int, const int32_t*, int,
                               hipStream_t) {
  return hit();
}
hipError_t launch_decode_update(const void*, const void*, const void*, const int32_t*, const int32_t*, int,
                                const sep_cache&, int, float, const float*, void*, float*, hipStream_t) {
  return hit();
}
hipError_t launch_decode(const void*, const void*, const void*, const sep_cache&, int, float, const float*, void*,
                         float*, hipStream_t) {
  return hit();
}
// the workspace rule of the real library is not needed here: a fixed size
size_t chunk_workspace_bytes(const sep_cache&, int C) { return 4096 + 256 * static_cast<size_t>(C); }
hipError_t launch_prefill_chunk(const void*, const void*, const void*, const int32_t*, int, const int32_t*, int,
                                const sep_cache&, int, int, float, void*, void*, float*, hipStream_t) {
  return hit();
}
hipError_t launch_rope_table(double, int, int, float*, hipStream_t) { return hit(); }

}  // namespace sep
