// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Records a failure message for pkv_last_error() and returns `s`.
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Descriptor checks shared by the device entry points.
pkv_status validate_desc(const pkv_cache_desc* d);
bool is_16bit_kv(int32_t kv);

// Device launchers (defined in the .hip files).
pkv_status launch_reshape_and_cache(const pkv_cache_desc& d, const void* k, const void* v,
                                    int32_t N, const int64_t* slots, void* k_pool, void* v_pool,
                                    void* k_meta, void* v_meta, pkv_stream_t stream);

}  // namespace pkv
